// Weight-streaming grouped kernels for the routed experts (gfx950).
//
// For decode-sized batches each active expert holds a handful of tokens, so the
// expert matmuls are bound by reading the expert weights from HBM once.  The
// weights stay in their grouped layout (page
// "nemo_automodel.components.models.glm4_moe.state_dict_adapter", class
// Glm4MoeStateDictAdapter: gate_and_up_projs [E, d, 2I] and down_projs [E, I, d],
// both with the output dimension contiguous).
//
// Row streaming.  A block reads whole weight rows, one 16-byte vector per lane:
// for down, 768 lanes cover a 12 KiB row of d = 6144 columns; for gate_up, 512
// lanes cover the 4 KiB of gate and the 4 KiB of up columns of a row (I = 2048):
// the first half of each wave reads gate columns and the second half the
// matching up columns, and the halves meet through a lane shuffle to form
// silu(gate) * up ("GLM-5 · Input features", excerpt mlp: the SwiGLU form).
// Wider outputs take several strips of that many columns.  The few token
// activations are the same for every lane (scalar loads) and the products are
// v_dot2c_f32_bf16 on row pairs (fp32 FMAs for fp32 weights) kept in registers:
// no LDS and no reduction across lanes.
//
// Balance.  The launch's work is the list of items (active expert i, pass p,
// strip s) in that order, a pass being up to kStreamMaxMT of the expert's tokens,
// each item cut into K / kRsChunk chunks of kRsChunk weight rows.  Calls whose
// items fill at most half of the resident blocks (known on the host from T * k)
// take the column split below instead.  When the items fill at least half of the
// resident blocks, blocks take whole items (RsGeom).  Otherwise (more items than
// resident blocks) the P resident blocks split the chunk list into equal contiguous
// ranges, lo(b) = floor(b * total / P), so every block reads the same number of
// weight bytes and the launch ends without a tail of lone blocks (the Stream-K
// decomposition of Osama et al., 2023, applied to a memory-bound product).  An item whose chunks
// fall in several blocks leaves one fp32 partial sum per part in a slot, and a
// small fixup kernel launched right after adds the parts in block order and
// applies the epilogue; the kernel boundary orders the two, so no block ever
// waits for or signals another.
#include <algorithm>
#include <atomic>

#include "common.h"
#include "dev_stream.h"
#include "kernels.h"

namespace moe {

template <typename T, bool GU>
__global__ __launch_bounds__(rs_threads<GU>()) void stream_kernel(GroupArgs g, StreamFix fx,
                                                                  const T* __restrict__ A,
                                                                  const T* __restrict__ Wall,
                                                                  T* __restrict__ out) {
  __shared__ int s_pass[kMaxStreamExperts + 1];
  const int n_active = g.hdr->n_active;
  for (int i = threadIdx.x; i <= n_active; i += rs_threads<GU>()) s_pass[i] = g.pass_base[i];
  __syncthreads();
  rs_block<T, GU, rs_threads<GU>()>(g, fx, s_pass, n_active, A, Wall, out, blockIdx.x, fx.blocks);
}

// The fixup runs one wave per block: block x finishes the columns of wave x % W
// (W = waves of the main kernel's blocks) of the item cut at the end of main block
// x / W's range.  A cut item's parts are then added by W compute units at once,
// not one (at one token an item spans about 32 parts, and one compute unit
// adding a down item's 768 KiB of them took 27 us).
template <typename T, bool GU>
__global__ __launch_bounds__(kWave) void stream_fixup_kernel(GroupArgs g, StreamFix fx,
                                                             T* __restrict__ out) {
  constexpr int W = rs_threads<GU>() / kWave;
  __shared__ int s_pass[kMaxStreamExperts + 1];
  const int b = blockIdx.x / W, tid = (blockIdx.x % W) * kWave + threadIdx.x;
  {
    // nothing to finish when every block took whole items (or this block has no successor)
    const RsGeom<T, GU, rs_threads<GU>()> G0(g, g.hdr->n_passes, fx.blocks);
    if (b + 1 >= G0.R.blocks) return;
  }
  const int n_active = g.hdr->n_active;
  for (int i = threadIdx.x; i <= n_active; i += kWave) s_pass[i] = g.pass_base[i];
  __syncthreads();
  rs_fixup_block<T, GU, rs_threads<GU>()>(g, fx, s_pass, n_active, out, b, fx.blocks, tid);
}

// Column split, for calls whose streaming passes (times the strips of a row) fill
// at most half the resident blocks: no item is cut along K, so no partial sums and
// no fixup.  Each pass's columns are split into J parts (J the largest power of
// two, at most 32, with passes * strips * P(J) <= blocks, P(J) the parts that hold
// columns: J at the GLM-5 widths), and a block takes one (pass, part)
// unit: all K weight rows of its columns.  Its lanes form J row groups of NTH / J
// lanes; a lane reads runs of RPI consecutive rows, J * RPI rows apart, over the
// part's columns (gate_up: the first half of a group's lanes read gate and the
// second half the matching up columns), and the J groups' sums meet in LDS, one
// token row at a time, for the epilogue.  A down unit at one token (8 passes,
// J = 32) reads 384 bytes per weight row.  The gate_up would read 128 bytes of gate
// and 128 of up columns per row at J = 32, so where J would exceed 8 it splits K
// instead (gu_ksplit below): J = 8 parts times S row ranges per pass, 512-byte runs
// per row at the GLM-5 width; each unit leaves fp32 gate and up sums of its range,
// and each down unit first forms its pass's act rows from those sums (silu of the
// gate sum times the up sum, rounded to D, as the gate_up epilogue otherwise does)
// in LDS.  At one token the gate_up launch takes 62-63 us instead of 70, the down
// launch 2-3 us longer.
struct ColLane {
  bool ok, is_up;
  int64_t wcol;
};

// K split of the gate_up for the fewest passes (ColKSplit).  When `pairs` (pass,
// strip) pairs of the gate_up over `blocks` blocks would cut each strip into more
// than 8 column parts, it cuts it into 8 parts times S row ranges, S the largest
// power of two up to 8 with pairs * parts * S <= blocks: each unit then reads
// 512-byte runs of gate and of up columns per weight row at the GLM-5 width (128
// bytes at 32 parts), which stream faster.  Returns S, or 0 for no split.  The
// down launch evaluates the same function on the gate_up's geometry.
template <typename T>
__device__ __forceinline__ int gu_ksplit(int64_t pairs, int blocks, int I) {
  constexpr int SW = rs_strip_cols<T, true, rs_threads<true>()>();
  auto parts = [&](int J) {
    const int swj = SW / J;
    return (min(I, SW) + swj - 1) / swj;
  };
  if (pairs * parts(16) > blocks) return 0;
  int S = 1;
  while (S < 8 && pairs * parts(8) * S * 2 <= blocks) S *= 2;
  return S >= 2 ? S : 0;
}

// A unit's share of the K split: S ranges (0: none), this gate_up unit's range s.
struct ColKs {
  float* part;  // [S][rows][2I]
  int64_t rows;
  int S, s;
};

template <typename T, bool GU, int MT>
__device__ __forceinline__ void cols_unit(const GroupArgs& g, const T* __restrict__ A,
                                          const T* __restrict__ Wall, T* __restrict__ out,
                                          const RsItem& it, int q, int J, float* s_red,
                                          const ColKs& kc, T* act, T* s_act) {
  // 8 rows in flight per lane for both products: the down blocks' 768 lanes leave
  // at most 168 registers per lane, too few for 16 rows and 8 token rows
  constexpr int NTH = rs_threads<GU>(), V = Elem<T>::kVec, RPI = 8;
  const int K = GU ? g.d : g.I, n_out = GU ? g.I : g.d;
  const int64_t ldw = GU ? 2 * (int64_t)g.I : (int64_t)g.d;
  const int LPR = NTH / J;                     // lanes per weight row
  const int SWJ = (GU ? LPR / 2 : LPR) * V;    // output columns of a part
  const int tid = threadIdx.x, rg = tid / LPR, cl = tid % LPR;
  const int64_t row0 = it.seg + it.m0;         // the item's first permuted row
  int kb = 0, ke = K;
  int64_t a_row0 = 0;
  if (GU && kc.S) {
    kb = kc.s * (K / kc.S);
    ke = kb + K / kc.S;
  }
  if (!GU && kc.S) {
    // act of the item's rows from the gate_up's range sums, rounded to D as the
    // gate_up epilogue rounds it, into LDS; the first column part also stores it
    // (4 consecutive columns per lane and pass of the loop, every range's loads
    // issued before the sums)
    const int I = g.I, I4 = I / 4;
    for (int i = tid; i < it.mt * I4; i += NTH) {
      const int m = i / I4, c = (i % I4) * 4;
      float4 gv[8], uv[8];
#pragma unroll
      for (int z = 0; z < 8; ++z) {
        if (z < kc.S) {
          const float* p = kc.part + ((int64_t)z * kc.rows + row0 + m) * 2 * I + c;
          gv[z] = *reinterpret_cast<const float4*>(p);
          uv[z] = *reinterpret_cast<const float4*>(p + I);
        }
      }
      float gs[4] = {0.f, 0.f, 0.f, 0.f}, us[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int z = 0; z < 8; ++z) {
        if (z < kc.S) {
          gs[0] += gv[z].x; gs[1] += gv[z].y; gs[2] += gv[z].z; gs[3] += gv[z].w;
          us[0] += uv[z].x; us[1] += uv[z].y; us[2] += uv[z].z; us[3] += uv[z].w;
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float v = silu(gs[j]) * us[j];
        Elem<T>::store1(s_act + m * I + c + j, v);
        if (q == 0) Elem<T>::store1(act + (row0 + m) * I + c + j, v);
      }
    }
    __syncthreads();
    A = s_act;
    a_row0 = row0;
  }
  ColLane ln;
  ln.is_up = GU && cl >= LPR / 2;
  const int ocol = q * SWJ + (GU ? cl % (LPR / 2) : cl) * V;
  ln.ok = ocol < n_out;  // n_out is a multiple of V
  ln.wcol = (ln.is_up ? (int64_t)g.I : 0) + ocol;
  float acc[MT][V];
  rs_accumulate<T, GU, MT, ColLane, RPI>(g, A, K, Wall + (int64_t)it.e * K * ldw, ldw, it, ln,
                                         kb + rg * RPI, ke, J * RPI, acc, a_row0);
  // s_red[rg][cl * V + c]: a row group's sums, gate columns first (for gate_up)
  const int vals = LPR * V;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    if (m >= it.mt) break;  // the same for the whole block
#pragma unroll
    for (int c = 0; c < V; ++c) s_red[tid * V + c] = acc[m][c];
    __syncthreads();
    T* orow = out + (row0 + m) * n_out;
    float* prow = GU && kc.S ? kc.part + ((int64_t)kc.s * kc.rows + row0 + m) * 2 * g.I : nullptr;
    for (int t = tid; t < SWJ; t += NTH) {
      float a = 0.f, u = 0.f;
      for (int r = 0; r < J; ++r) {
        a += s_red[r * vals + t];
        if (GU) u += s_red[r * vals + SWJ + t];
      }
      const int col = q * SWJ + t;
      if (col < n_out) {
        if (GU && kc.S) {
          prow[col] = a;
          prow[g.I + col] = u;
        } else {
          Elem<T>::store1(orow + col, GU ? silu(a) * u : a);
        }
      }
    }
    __syncthreads();
  }
}

// gu_blocks: the blocks of the gate_up launch (the down launch uses them to see
// whether the gate_up split K).  act: for the down launch, its activation rows
// (A itself), which it stores when it forms them from the K split's sums; A is
// then never read.
template <typename T, bool GU>
__global__ __launch_bounds__(rs_threads<GU>()) void stream_cols_kernel(GroupArgs g, int blocks,
                                                                       ColKSplit ks, int gu_blocks,
                                                                       const T* A, T* act,
                                                                       const T* __restrict__ Wall,
                                                                       T* __restrict__ out) {
  constexpr int NTH = rs_threads<GU>(), V = Elem<T>::kVec;
  __shared__ int s_pass[kMaxStreamExperts + 1];
  __shared__ float s_red[NTH * V];
  extern __shared__ uint4 s_dyn[];  // kRsLdsHold bytes: the down units' act rows
  const int n_active = g.hdr->n_active;
  for (int i = threadIdx.x; i <= n_active; i += NTH) s_pass[i] = g.pass_base[i];
  __syncthreads();
  const int n_out = GU ? g.I : g.d;
  constexpr int SW = rs_strip_cols<T, GU, NTH>();
  const int strips = (n_out + SW - 1) / SW;
  const int64_t passes = (int64_t)s_pass[n_active] * strips;  // (pass, strip) pairs
  // Parts of a strip that hold columns when it is cut in J (all J for the GLM-5
  // widths, fewer for outputs narrower than a strip).
  auto parts = [&](int J) {
    const int swj = SW / J;
    return (min(n_out, SW) + swj - 1) / swj;
  };
  ColKs kc{ks.part, ks.rows, 0, 0};
  if (ks.ok) {
    constexpr int SWG = rs_strip_cols<T, true, rs_threads<true>()>();
    kc.S = gu_ksplit<T>((int64_t)s_pass[n_active] * ((g.I + SWG - 1) / SWG), gu_blocks, g.I);
  }
  int J = 1;
  if (GU && kc.S) {
    J = 8;
  } else {
    while (J < 32 && passes * parts(J * 2) <= blocks) J *= 2;
  }
  const int jv = parts(J);
  const int S = GU && kc.S ? kc.S : 1;
  const int64_t units = passes * jv * S;
  T* s_act = reinterpret_cast<T*>(s_dyn);
  for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
    kc.s = (int)(u % S);
    const int64_t ur = u / S;
    const int64_t ps = ur / jv;
    const int q = (int)(ps % strips) * J + (int)(ur % jv);  // column part within the pass
    int ai = 0;
    const RsItem it = rs_item<true>(g, s_pass, n_active, 1, ps / strips, &ai);
    if (it.mt == 1) cols_unit<T, GU, 1>(g, A, Wall, out, it, q, J, s_red, kc, act, s_act);
    else if (it.mt == 2) cols_unit<T, GU, 2>(g, A, Wall, out, it, q, J, s_red, kc, act, s_act);
    else if (it.mt <= 4) cols_unit<T, GU, 4>(g, A, Wall, out, it, q, J, s_red, kc, act, s_act);
    else cols_unit<T, GU, 8>(g, A, Wall, out, it, q, J, s_red, kc, act, s_act);
  }
}

// The partition assumes one block per compute unit (the dispatcher spreads the
// blocks of a launch over the CUs only when no CU can hold two), so each launch
// asks for more dynamic LDS than half a CU's 160 KiB; the kernels do not use it.
constexpr size_t kRsLdsHold = 96 * 1024;

// Blocks of stream_kernel<T, GU> resident on the current device at once (all
// compute units), capped at kStreamMaxBlocks; queried once per device.
template <typename T, bool GU>
static hipError_t resident_blocks(int* blocks) {
  static std::atomic<int> cached[64];  // zero-initialised (static storage)
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    int cus = 0, per_cu = 0;
    err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess) return err;
    err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, stream_kernel<T, GU>,
                                                       rs_threads<GU>(), kRsLdsHold);
    if (err != hipSuccess) return err;
    n = std::max(1, std::min(kStreamMaxBlocks, std::max(per_cu, 1) * std::max(cus, 1)));
    cached[dev].store(n, std::memory_order_relaxed);
  }
  *blocks = n;
  return hipSuccess;
}

// Whether the GU product of a call with at most max_passes passes runs the column
// split on `blocks` resident blocks: J >= 2 whatever the routing.
template <typename T, bool GU>
static bool col_mode(const GroupArgs& g, int64_t max_passes, int blocks) {
  constexpr int SW = rs_strip_cols<T, GU, rs_threads<GU>()>();
  const int64_t strips = ((GU ? g.I : g.d) + SW - 1) / SW;
  return 2 * max_passes * strips <= blocks;
}

template <typename T, bool GU>
static hipError_t launch_stream(const GroupArgs& g, const StreamFix& fx_in, int64_t max_passes,
                                const ColKSplit& ks_in, const void* A, const void* W, void* out,
                                hipStream_t s) {
  StreamFix fx = fx_in;
  hipError_t err = resident_blocks<T, GU>(&fx.blocks);
  if (err != hipSuccess) return err;
  if (fx.blocks < 1 || fx.blocks > kStreamMaxBlocks || g.E > kMaxStreamExperts)
    return hipErrorInvalidValue;
  if (col_mode<T, GU>(g, max_passes, fx.blocks)) {
    // The K split is allowed only when both products run the column split (the down
    // units form act) and a unit's act rows fit the LDS the launch holds anyway;
    // both launches decide it alike.
    int gu_blocks = 0, dn_blocks = 0;
    err = resident_blocks<T, true>(&gu_blocks);
    if (err == hipSuccess) err = resident_blocks<T, false>(&dn_blocks);
    if (err != hipSuccess) return err;
    ColKSplit ks = ks_in;
    ks.ok = ks.ok && ks.part && col_mode<T, true>(g, max_passes, gu_blocks) &&
            col_mode<T, false>(g, max_passes, dn_blocks) &&
            (size_t)kStreamMaxMT * g.I * sizeof(T) <= kRsLdsHold;
    stream_cols_kernel<T, GU><<<dim3((unsigned)fx.blocks), rs_threads<GU>(), kRsLdsHold, s>>>(
        g, fx.blocks, ks, gu_blocks, (const T*)A, GU ? nullptr : (T*)A, (const T*)W, (T*)out);
    return hipGetLastError();
  }
  stream_kernel<T, GU><<<dim3((unsigned)fx.blocks), rs_threads<GU>(), kRsLdsHold, s>>>(
      g, fx, (const T*)A, (const T*)W, (T*)out);
  err = hipGetLastError();
  if (err != hipSuccess || fx.blocks == 1) return err;
  stream_fixup_kernel<T, GU><<<dim3((unsigned)(fx.blocks - 1) * (rs_threads<GU>() / kWave)), kWave, 0,
                               s>>>(g, fx, (T*)out);
  return hipGetLastError();
}

hipError_t launch_stream_gate_up(int dtype, const GroupArgs& g, const StreamFix& fx,
                                 int64_t max_passes, const ColKSplit& ks, const void* h,
                                 const void* gate_up, void* act, hipStream_t s) {
  if (dtype == kBF16) return launch_stream<bf16, true>(g, fx, max_passes, ks, h, gate_up, act, s);
  return launch_stream<float, true>(g, fx, max_passes, ks, h, gate_up, act, s);
}

hipError_t launch_stream_down(int dtype, const GroupArgs& g, const StreamFix& fx,
                              int64_t max_passes, const ColKSplit& ks, void* act,
                              const void* down, void* y, hipStream_t s) {
  if (dtype == kBF16) return launch_stream<bf16, false>(g, fx, max_passes, ks, act, down, y, s);
  return launch_stream<float, false>(g, fx, max_passes, ks, act, down, y, s);
}

}  // namespace moe
