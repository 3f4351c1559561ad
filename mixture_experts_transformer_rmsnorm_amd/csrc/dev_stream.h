// Device code of the weight-streaming grouped expert matmuls (decode-sized
// batches), shared by the stand-alone kernels (k_stream.hip, one block per compute
// unit of rs_threads<GU>() lanes) and the fused decode kernel (k_decode.hip, two
// blocks of 256 lanes per compute unit).  The design is described in
// k_stream.hip; NTH is the lane count of the blocks that run it.
#pragma once

#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kRsChunk = 16;  // weight rows of the smallest K range

// Lanes of a block: whole rows of the GLM-5 shapes (gate_up: 4 KiB of gate and
// 4 KiB of up columns, I = 2048; down: 12 KiB, d = 6144).
template <bool GU>
__host__ __device__ constexpr int rs_threads() { return GU ? 512 : 768; }

// Consecutive weight rows a lane reads per step: 8 (gate_up) or 16 (down) 16-byte
// vectors in flight per lane.
template <bool GU>
__host__ __device__ constexpr int rs_rows_per_step() { return GU ? 8 : 16; }

// Output columns of one item (a strip): one 16-byte vector per lane for down;
// for gate_up half the lanes read gate and half up columns.
template <typename T, bool GU, int NTH>
__host__ __device__ constexpr int rs_strip_cols() {
  return (GU ? NTH / 2 : NTH) * (16 / (int)sizeof(T));
}

// Split of `total` chunks (items of C chunks each) over `blocks` blocks: blocks
// [0, hblocks) take one whole item each; blocks [hblocks, blocks) split the
// remaining chunks into equal contiguous ranges, lo(b) = head + floor((b -
// hblocks) * (total - head) / (blocks - hblocks)).
struct RsRange {
  int64_t total, C;
  int blocks, hblocks;
  // (total - head) = q * (blocks - hblocks) + r: lo(b) = head + b' q + floor(b' r /
  // (blocks - hblocks)) with b' = b - hblocks, so lo() needs one 32-bit division
  // (the fixup evaluates it for every part it adds; a 64-bit division each was most
  // of its time)
  int64_t q;
  int r;
  __device__ __forceinline__ void split_rest() {
    const int64_t rest = total - (int64_t)hblocks * C;
    const int tb = blocks - hblocks;
    q = tb > 0 ? rest / tb : 0;
    r = tb > 0 ? (int)(rest - q * tb) : 0;
  }
  __device__ __forceinline__ int64_t lo(int b) const {
    if (b <= hblocks) return (int64_t)b * C;
    const int bb = b - hblocks;
    return (int64_t)hblocks * C + (int64_t)bb * q +
           (int64_t)((uint32_t)(bb * r) / (uint32_t)(blocks - hblocks));
  }
  // The block whose range holds chunk x: the largest b with lo(b) <= x.
  __device__ __forceinline__ int block_of(int64_t x) const {
    const int64_t head = (int64_t)hblocks * C;
    if (x < head) return (int)(x / C);
    const int tb = blocks - hblocks;
    int b = hblocks + (int)min<int64_t>(tb - 1, (x - head) * tb / (total - head));
    while (b + 1 < blocks && lo(b + 1) <= x) ++b;
    while (lo(b) > x) --b;
    return b;
  }
};

// Geometry of one launch, the same in the main and the fixup kernel.  With P
// resident blocks and n items: P/2 <= n <= P, block b < n takes item b whole
// (enough blocks to keep HBM busy, no item split); otherwise (few items, or more
// than P) equal chunk ranges over the P blocks.
template <typename T, bool GU, int NTH>
struct RsGeom {
  int K, n_out, strips, C;
  int64_t ldw;
  RsRange R;
  __device__ __forceinline__ RsGeom(const GroupArgs& g, int n_passes, int blocks) {
    K = GU ? g.d : g.I;
    n_out = GU ? g.I : g.d;
    ldw = GU ? 2 * (int64_t)g.I : (int64_t)g.d;
    strips = (n_out + rs_strip_cols<T, GU, NTH>() - 1) / rs_strip_cols<T, GU, NTH>();
    C = K / kRsChunk;
    const int64_t items = (int64_t)n_passes * strips;
    R.total = items * C;
    R.C = C;
    if (items > blocks || 2 * items < (int64_t)blocks) {
      R.hblocks = 0;
      R.blocks = blocks;
    } else {
      R.hblocks = R.blocks = (int)items;
    }
    R.split_rest();
  }
};

// Tokens and weights of an item.
struct RsItem {
  int e, seg, m0, mt, strip;
};

// Item `item` given the pass prefix s_pass[0..n_active] and the active expert
// index `ai` of an earlier item (or 0): the active expert of pass pidx is the
// last i with s_pass[i] <= pidx.
template <bool SEARCH>
__device__ __forceinline__ RsItem rs_item(const GroupArgs& g, const int* s_pass, int n_active,
                                          int strips, int64_t item, int* ai) {
  const int pidx = (int)(item / strips);
  if (SEARCH) {
    int l = 0, r = n_active - 1;
    while (l < r) {
      const int mid = (l + r + 1) / 2;
      if (s_pass[mid] <= pidx) l = mid; else r = mid - 1;
    }
    *ai = l;
  } else {
    while (s_pass[*ai + 1] <= pidx) ++*ai;
  }
  RsItem it;
  it.e = g.active[*ai];
  it.seg = g.offsets[it.e];
  it.m0 = (pidx - s_pass[*ai]) * kStreamMaxMT;
  it.mt = min(kStreamMaxMT, g.counts[it.e] - it.m0);
  it.strip = (int)(item % strips);
  return it;
}

// Columns of this lane: output columns [ocol, ocol + V) of the strip, read from
// weight column wcol (the up half for gate_up lanes in the second half of a
// wave).  In a partial-sum slot row (gate sums, then up sums for gate_up) the
// lane's V sums sit as V / 4 groups of four, group j at spos + j * sgap, so that
// each group's store by a wave covers one contiguous kilobyte.
template <typename T, bool GU, int NTH>
struct RsLane {
  int grp, ocol, spos, sgap;
  int64_t wcol;
  bool is_up, ok;
  // tid: the lane's index in a block of NTH lanes (its thread index, or in the
  // fixup kernel, whose blocks are one wave each, wave w of the item's NTH lanes)
  __device__ __forceinline__ RsLane(const GroupArgs& g, int n_out, int strip, int tid) {
    constexpr int V = Elem<T>::kVec, SW = rs_strip_cols<T, GU, NTH>();
    const int lane = tid % kWave, wave = tid / kWave;
    is_up = GU && lane >= kWave / 2;
    grp = GU ? wave * (kWave / 2) + lane % (kWave / 2) : tid;
    ocol = strip * SW + grp * V;
    ok = ocol < n_out;  // n_out is a multiple of V
    wcol = (is_up ? (int64_t)g.I : 0) + ocol;
    const int wq = min(SW, n_out);  // slot floats of the gate (or the only) half
    spos = (is_up ? wq : 0) + grp * 4;
    sgap = wq / V * 4;
  }
};

// fp32 words of a slot row: the strip's columns (gate, then up for gate_up).
template <typename T, bool GU, int NTH>
__device__ __forceinline__ int64_t rs_slot_ld(int n_out) {
  return (GU ? 2 : 1) * (int64_t)min(rs_strip_cols<T, GU, NTH>(), n_out);
}

// RPI consecutive elements of one fp32 activation row.
template <typename T, int RPI>
__device__ __forceinline__ void load_act(const T* p, float* f) {
#pragma unroll
  for (int r = 0; r < RPI; r += 4) Elem<float>::unpack(ldg16(p + r), f + r);
}

// c + x.lo * y.lo + x.hi * y.hi for two packed bf16 pairs (v_dot2c_f32_bf16).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2_bf16(uint32_t x, uint32_t y, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, x),
                                         __builtin_bit_cast(bf16x2_t, y), c, false);
}

// acc[m][c] = sum over the weight rows k0 + i * kstep + r (r < RPI, below k1) of
// A[row m][k] * W[k][wcol + c]: the lane's runs of RPI consecutive rows, kstep
// apart (kstep = RPI: every row of [k0, k1)), RPI weight vectors in flight per
// lane.  LN: the lane's ok and wcol.
//   gate_up: A = h [T, d] (rows gathered by perm_token), W = gate_up[e] [d, 2I]
//   down:    A = act [rows, I],                          W = down[e] [I, d]
// A's row r is read at A + (r - row0) * lda (row0: the first row of an A that
// holds only the item's rows).
template <typename T, bool GU, int MT, typename LN, int RPI = rs_rows_per_step<GU>()>
__device__ __forceinline__ void rs_accumulate(const GroupArgs& g, const T* __restrict__ A,
                                              int64_t lda, const T* __restrict__ W, int64_t ldw,
                                              const RsItem& it, const LN& ln, int k0, int k1,
                                              int kstep, float (&acc)[MT][Elem<T>::kVec],
                                              int64_t row0 = 0) {
  constexpr int V = Elem<T>::kVec;
  static_assert(RPI % 8 == 0, "whole 16-byte activation vectors per step");
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int c = 0; c < V; ++c) acc[m][c] = 0.f;
  if (!ln.ok) return;
  const T* arow[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int mm = m < it.mt ? m : it.mt - 1;  // rows past mt repeat the last one, never stored
    const int64_t prow = it.seg + it.m0 + mm;
    const int64_t r = GU ? (int64_t)g.perm_token[prow] : prow;
    arow[m] = A + (r - row0) * lda;
  }
  const T* wp = W + (int64_t)k0 * ldw + ln.wcol;
  for (int k = k0; k < k1; k += kstep, wp += (int64_t)kstep * ldw) {
    uint4 wv[RPI];
#pragma unroll
    for (int r = 0; r < RPI; ++r) wv[r] = ldg16_stream(wp + (int64_t)r * ldw);
    if constexpr (sizeof(T) == 2) {
      // bf16: products of row pairs (k + 2p, k + 2p + 1) with v_dot2c_f32_bf16,
      // acc += a[2p] * w[2p][c] + a[2p + 1] * w[2p + 1][c].  An activation row's
      // 16-byte pieces hold the pairs in order; the weight pairs are gathered
      // from two rows' words (cols c, c + 1 each) with byte permutes.
      uint32_t a[MT][RPI / 2];
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int h = 0; h < RPI / 8; ++h) {
          const uint4 q = ldg16(arow[m] + k + 8 * h);
          a[m][4 * h] = q.x; a[m][4 * h + 1] = q.y; a[m][4 * h + 2] = q.z; a[m][4 * h + 3] = q.w;
        }
#pragma unroll
      for (int p = 0; p < RPI / 2; ++p) {
        const uint32_t lo[4] = {wv[2 * p].x, wv[2 * p].y, wv[2 * p].z, wv[2 * p].w};
        const uint32_t hi[4] = {wv[2 * p + 1].x, wv[2 * p + 1].y, wv[2 * p + 1].z,
                                wv[2 * p + 1].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t w0 = __builtin_amdgcn_perm(hi[q], lo[q], 0x05040100u);  // column 2q
          const uint32_t w1 = __builtin_amdgcn_perm(hi[q], lo[q], 0x07060302u);  // column 2q + 1
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            acc[m][2 * q] = dot2_bf16(a[m][p], w0, acc[m][2 * q]);
            acc[m][2 * q + 1] = dot2_bf16(a[m][p], w1, acc[m][2 * q + 1]);
          }
        }
      }
    } else {
      float a[MT][RPI];
#pragma unroll
      for (int m = 0; m < MT; ++m) load_act<T, RPI>(arow[m] + k, a[m]);
#pragma unroll
      for (int r = 0; r < RPI; ++r) {
        float f[V];
        Elem<T>::unpack(wv[r], f);
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int c = 0; c < V; ++c) acc[m][c] += a[m][r] * f[c];
      }
    }
  }
}

// Stores an item's outputs: act = silu(gate) * up for gate_up (the up sums sit
// in the lane kWave / 2 further on; every lane takes part in the shuffle), the
// sums themselves for down.
template <typename T, bool GU, int MT, int NTH>
__device__ __forceinline__ void rs_store(const float (&acc)[MT][Elem<T>::kVec], const RsItem& it,
                                         const RsLane<T, GU, NTH>& ln, int n_out,
                                         T* __restrict__ out) {
  constexpr int V = Elem<T>::kVec;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    if (m >= it.mt) break;
    float v[V];
    if constexpr (GU) {
#pragma unroll
      for (int c = 0; c < V; ++c) {
        const float u = __shfl_xor(acc[m][c], kWave / 2, kWave);
        v[c] = silu(acc[m][c]) * u;
      }
    } else {
#pragma unroll
      for (int c = 0; c < V; ++c) v[c] = acc[m][c];
    }
    if (ln.ok && !ln.is_up)
      stg16(out + (int64_t)(it.seg + it.m0 + m) * n_out + ln.ocol, Elem<T>::pack(v));
  }
}

// Row 0 of the slot of block b's part of an item starting at chunk item0: slot
// 2b when the part starts the block's range, else 2b + 1 (the part then ends the
// range).  A slot holds kStreamMaxMT rows of ld floats, one after the other.
__device__ __forceinline__ float* rs_slot(const StreamFix& fx, const RsRange& R, int b,
                                          int64_t item0, int64_t ld) {
  const int sl = item0 > R.lo(b) ? 1 : 0;
  return fx.parts + ((int64_t)b * 2 + sl) * kStreamMaxMT * ld;
}

template <typename T, bool GU, int MT, int NTH>
__device__ __forceinline__ void rs_part(const GroupArgs& g, const StreamFix& fx,
                                        const RsGeom<T, GU, NTH>& G, const T* __restrict__ A,
                                        const T* __restrict__ Wall, const RsItem& it, int c0,
                                        int c1, int b, int64_t item0, T* __restrict__ out) {
  constexpr int V = Elem<T>::kVec;
  const RsLane<T, GU, NTH> ln(g, G.n_out, it.strip, threadIdx.x);
  const T* W = Wall + (int64_t)it.e * G.K * G.ldw;
  float acc[MT][V];
  rs_accumulate<T, GU, MT>(g, A, G.K, W, G.ldw, it, ln, c0 * kRsChunk, c1 * kRsChunk,
                           rs_rows_per_step<GU>(), acc);
  if (c0 == 0 && c1 == G.C) {
    rs_store<T, GU, MT, NTH>(acc, it, ln, G.n_out, out);
    return;
  }
  if (!ln.ok) return;
  const int64_t ld = rs_slot_ld<T, GU, NTH>(G.n_out);
  float* mine = rs_slot(fx, G.R, b, item0, ld);
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    if (m >= it.mt) break;
#pragma unroll
    for (int c = 0; c < V; c += 4)
      *reinterpret_cast<float4*>(mine + m * ld + ln.spos + (c / 4) * ln.sgap) =
          make_float4(acc[m][c], acc[m][c + 1], acc[m][c + 2], acc[m][c + 3]);
  }
}

// Finishes the item that runs past the end of block b's range, when the item
// starts in that range (so each cut item is finished once): adds its parts'
// slots in block order and stores the outputs.
template <typename T, bool GU, int MT, int NTH>
__device__ __forceinline__ void rs_finish(const GroupArgs& g, const StreamFix& fx,
                                          const RsGeom<T, GU, NTH>& G, const RsItem& it, int b,
                                          int64_t item0, T* __restrict__ out, int tid) {
  constexpr int V = Elem<T>::kVec;
  const RsLane<T, GU, NTH> ln(g, G.n_out, it.strip, tid);
  const int64_t ld = rs_slot_ld<T, GU, NTH>(G.n_out);
  const int bl = G.R.block_of(item0 + G.C - 1);
  float acc[MT][V];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int c = 0; c < V; ++c) acc[m][c] = 0.f;
  if (ln.ok) {
    // The parts of U blocks at a time are loaded together (at one token an item
    // spans about 32 blocks, and one part after another took a load latency
    // each), then added in block order; blocks with an empty range hold no part.
    constexpr int U = 16 / MT;  // 32 float4 of parts in flight per lane
    for (int bb0 = b; bb0 <= bl; bb0 += U) {
      float4 v[U][MT][V / 4];
      bool use[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int bb = bb0 + u;
        use[u] = bb <= bl && G.R.lo(bb) != G.R.lo(bb + 1);
        if (use[u]) {
          const float* src = rs_slot(fx, G.R, bb, item0, ld);
#pragma unroll
          for (int m = 0; m < MT; ++m)
            if (m < it.mt)
#pragma unroll
              for (int c = 0; c < V; c += 4)
                v[u][m][c / 4] = *reinterpret_cast<const float4*>(src + m * ld + ln.spos +
                                                                  (c / 4) * ln.sgap);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (!use[u]) continue;
#pragma unroll
        for (int m = 0; m < MT; ++m)
          if (m < it.mt)
#pragma unroll
            for (int c = 0; c < V; c += 4) {
              acc[m][c] += v[u][m][c / 4].x;
              acc[m][c + 1] += v[u][m][c / 4].y;
              acc[m][c + 2] += v[u][m][c / 4].z;
              acc[m][c + 3] += v[u][m][c / 4].w;
            }
      }
    }
  }
  rs_store<T, GU, MT, NTH>(acc, it, ln, G.n_out, out);
}


// Block b's work in a launch of `blocks` blocks of NTH lanes: its range of the
// chunk list, item by item.  s_pass: the routing's pass prefix in LDS
// (s_pass[i] = first pass of the i-th active expert, s_pass[n_active] = passes).
// No block barrier inside.
template <typename T, bool GU, int NTH>
__device__ __forceinline__ void rs_block(const GroupArgs& g, const StreamFix& fx,
                                         const int* s_pass, int n_active, const T* __restrict__ A,
                                         const T* __restrict__ Wall, T* __restrict__ out, int b,
                                         int blocks) {
  const RsGeom<T, GU, NTH> G(g, s_pass[n_active], blocks);
  if (b >= G.R.blocks) return;
  const int64_t lo = G.R.lo(b), hi = G.R.lo(b + 1);
  int ai = 0;
  for (int64_t pos = lo; pos < hi;) {
    const int64_t item = pos / G.C;
    const int c0 = (int)(pos - item * G.C);
    const int c1 = (int)min<int64_t>(G.C, c0 + (hi - pos));
    const RsItem it = pos == lo ? rs_item<true>(g, s_pass, n_active, G.strips, item, &ai)
                                : rs_item<false>(g, s_pass, n_active, G.strips, item, &ai);
#define MOE_PART(MT) rs_part<T, GU, MT, NTH>(g, fx, G, A, Wall, it, c0, c1, b, item * G.C, out)
    if (it.mt == 1) MOE_PART(1);
    else if (it.mt == 2) MOE_PART(2);
    else if (it.mt <= 4) MOE_PART(4);
    else MOE_PART(8);
#undef MOE_PART
    pos += c1 - c0;
  }
}

// Block b's fixup: finishes the item cut at the end of its range when the item
// starts in that range (so each cut item is finished once); tid as for RsLane.  No
// block barrier inside.
template <typename T, bool GU, int NTH>
__device__ __forceinline__ void rs_fixup_block(const GroupArgs& g, const StreamFix& fx,
                                               const int* s_pass, int n_active,
                                               T* __restrict__ out, int b, int blocks, int tid) {
  const RsGeom<T, GU, NTH> G(g, s_pass[n_active], blocks);
  if (b + 1 >= G.R.blocks) return;  // every block took whole items, or no successor
  const int64_t lo = G.R.lo(b), x = G.R.lo(b + 1);
  if (lo == x || x >= G.R.total || x % G.C == 0) return;  // empty range, or no item cut at its end
  const int64_t item = x / G.C, item0 = item * G.C;
  if (item0 < lo) return;  // the item started in an earlier block, which finishes it
  int ai = 0;
  const RsItem it = rs_item<true>(g, s_pass, n_active, G.strips, item, &ai);
#define MOE_FIN(MT) rs_finish<T, GU, MT, NTH>(g, fx, G, it, b, item0, out, tid)
  if (it.mt == 1) MOE_FIN(1);
  else if (it.mt == 2) MOE_FIN(2);
  else if (it.mt <= 4) MOE_FIN(4);
  else MOE_FIN(8);
#undef MOE_FIN
}

}  // namespace moe
