// bf16 matrix-core (MFMA) kernels for gfx950: the grouped expert matmuls of
// prefill-sized batches and the dense K-contiguous products (router logits,
// shared expert).
//
// Tile: 128 (rows) x 128 (B columns) x 64 (K) per 256-thread block, four
// wavefronts in a 2 x 2 arrangement, each owning 64 rows x 64 B-columns as
// 2 x 2 tiles of v_mfma_f32_32x32x16_bf16 (fp32 accumulation; on MI355X this
// form sustains about 2.0 PFLOP/s against about 1.7 for the 16x16x32 form).  A and B tiles
// are staged in LDS with K contiguous (row stride 72 elements, so the 16-byte
// fragment reads of 16 consecutive rows hit distinct banks) and double
// buffered: the global loads of K-tile t+1 are in flight while tile t is
// multiplied.
//
// B layouts:
//  - K-contiguous ([N, K], nn.Linear weights: router, shared expert) is copied
//    to LDS as is.
//  - N-contiguous ([K, N], the grouped expert layout of
//    Glm4MoeStateDictAdapter: gate_and_up_projs [E, d, 2I], down_projs
//    [E, I, d]) is copied to LDS row by row as loaded (rows padded to 144
//    elements) and the K-contiguous MFMA fragments are formed by gfx950's
//    transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group G,
//    output lane i, element j is element i%4 of the 8-byte chunk addressed by
//    lane 4j + i/4 of the group.  The 32x32x16 B operand wants lane
//    l = 32*hk + 16*nb + i to hold B[8hk .. 8hk+7][16nb + i]; so lane (G, j, q)
//    addresses row 8*(G/2) + 4h + j, column 16*(G%2) + 4q, and two reads
//    (h = 0, 1) give the 8 K-consecutive values.
// The gate_up tile pairs gate columns [c, c+64) with up columns [I+c, I+c+64)
// so that silu(gate) * up is formed in registers ("GLM-5 · Input features",
// excerpt mlp).
#include "common.h"
#include "kernels.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

constexpr int BM = kMfmaBM, BN = kMfmaBN, BK = kMfmaBK;
constexpr int kXcds = 8;  // accelerator complex dies of an MI355X, one L2 each
constexpr int LDK = BK + 8;   // K-contiguous LDS rows: 72 elements (144 bytes)
constexpr int LDN = BN + 16;  // N-contiguous LDS rows: 144 elements (288 bytes)
constexpr int kTileElems = BM * LDK;
static_assert(BK * LDN <= kTileElems, "N-contiguous B tile fits the stage buffer");

enum Epi { kEpiPartialF32 = 0, kEpiSwiGLU = 1, kEpiStore = 2 };

struct MfmaProblem {
  // A rows (K-contiguous): dense rows m, or grouped permuted rows gathered
  // through a_gather (A row = a_gather[permuted row]) or taken directly.
  const uint16_t* A;
  int64_t lda;
  const int32_t* a_gather;
  // B, K-contiguous: row n at B1 + n*ldb (n < n_split) else B2 + (n-n_split)*ldb.
  const uint16_t* B1;
  const uint16_t* B2;
  int64_t ldb;
  int n_split;
  // B, N-contiguous grouped: element (k, n) of expert e at Bg + e*b_stride + k*ldb + n;
  // SwiGLU up columns start at column up_off.
  const uint16_t* Bg;
  int64_t b_stride;
  int up_off;
  int K;
  int N;  // output columns (SwiGLU: number of act columns)
  // grouped problems
  const int2* mtiles;
  const RouteHeader* hdr;
  const int32_t* offsets;
  const int32_t* counts;
  int n_tiles;  // N-tiles of a grouped problem
  // dense problems
  int M;
  int kt_per_split;
  // output
  void* C;
  int64_t ldc;
};

__device__ __forceinline__ int b_local_col(int f, int wn) {
  // B-columns of wave column wn: [wn*32, wn*32+32) (f = 0) and [64+wn*32, 64+wn*32+32)
  // (f = 1); for SwiGLU tiles these are the matching gate and up columns.
  return f * 64 + wn * 32;
}

// 32x16 B fragment (K rows ks*16 .., columns col ..) from an N-contiguous LDS
// tile by two transposing reads.
__device__ __forceinline__ bf16x8_t b_frag_tr(const uint16_t* bs, int ks, int col, int lane) {
  const int G = lane >> 4, j = (lane & 15) >> 2, q = lane & 3;
  const uint16_t* p = bs + (ks * 16 + 8 * (G >> 1) + j) * LDN + col + 16 * (G & 1) + 4 * q;
  const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p);
  const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p + 4 * LDN));
  typedef short s16x8_t __attribute__((ext_vector_type(8)));
  const s16x8_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8_t, v);
}

template <bool NN, int EPI>
__global__ __launch_bounds__(256) void mfma_kernel(MfmaProblem p) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2 * kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2 * kTileElems];
  constexpr bool kGrouped = NN;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  int n_tile = blockIdx.x;

  int rows, seg = 0, m0, e = 0;
  if (kGrouped) {
    // Work-groups are dispatched round-robin over the 8 XCDs.  Give XCD x the
    // contiguous range [x*per, (x+1)*per) of the (M-tile, N-tile) pairs that exist,
    // M-tile major: the N-tiles of one M-tile then share x's L2 for the gathered
    // A rows, and consecutive M-tiles of one expert share it for B.
    const int n_tiles = p.n_tiles;
    const int total = p.hdr->n_mtiles * n_tiles;
    const int per = (total + kXcds - 1) / kXcds;
    const int slot = blockIdx.x / kXcds;
    if (slot >= per) return;
    const int logical = (blockIdx.x % kXcds) * per + slot;
    if (logical >= total) return;
    const int mt = logical / n_tiles;
    n_tile = logical % n_tiles;
    const int2 tt = p.mtiles[mt];
    e = tt.x;
    m0 = tt.y;
    seg = p.offsets[e];
    rows = min(BM, p.counts[e] - m0);
  } else {
    m0 = blockIdx.y * BM;
    rows = min(BM, p.M - m0);
  }
  const int nkt = p.K / BK;
  const int kt0 = kGrouped ? 0 : blockIdx.z * p.kt_per_split;
  const int kt1 = kGrouped ? nkt : min(nkt, kt0 + p.kt_per_split);

  // ---- per-thread global load assignments
  // A: rows tid/8 + 32*i, 16-byte chunk tid%8
  // Rows past the tile's valid rows (and B columns past N) load a valid row
  // (column) instead: they only feed outputs the epilogue never stores, and
  // unconditional loads keep the wait counts of the pipeline exact.
  const uint16_t* a_src[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = min(tid / 8 + 32 * i, rows - 1);
    int64_t arow;
    if (kGrouped) {
      const int64_t prow = seg + m0 + r;
      arow = p.a_gather ? (int64_t)p.a_gather[prow] : prow;
    } else {
      arow = m0 + r;
    }
    a_src[i] = p.A + arow * p.lda + (tid % 8) * 8;
  }
  // B
  const uint16_t* b_src[4];
  int64_t b_kstride = 0;
  if (!NN) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int lc = tid / 8 + 32 * i;
      const int n = n_tile * BN + lc;
      const int nn = n < p.N ? n : 0;
      const uint16_t* row = nn < p.n_split ? p.B1 + (int64_t)nn * p.ldb
                                           : p.B2 + (int64_t)(nn - p.n_split) * p.ldb;
      b_src[i] = row + (tid % 8) * 8;
    }
  } else {
    // k-rows tid/16 + 16*i, 16-byte column chunk tid%16 of the 128 tile columns
    const int lc = (tid % 16) * 8;
    int gcol;
    bool ok;
    if (EPI == kEpiSwiGLU) {
      const int c = n_tile * 64 + (lc & 63);
      ok = c < p.N;
      gcol = (lc < 64 ? 0 : p.up_off) + c;
    } else {
      gcol = n_tile * BN + lc;
      ok = gcol < p.N;
    }
    const uint16_t* base = p.Bg + (int64_t)e * p.b_stride + (int64_t)(tid / 16) * p.ldb + (ok ? gcol : 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) b_src[i] = base + (int64_t)(16 * i) * p.ldb;
    b_kstride = (int64_t)BK * p.ldb;
  }

  uint4 ra[4], rb[4];
  auto gload = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) ra[i] = ldg16(a_src[i] + k0);
    if (!NN) {
#pragma unroll
      for (int i = 0; i < 4; ++i) rb[i] = ldg16(b_src[i] + k0);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) rb[i] = ldg16(b_src[i] + (int64_t)kt * b_kstride);
    }
  };
  auto lstore = [&](int buf) {
    uint16_t* as = As + buf * kTileElems;
    uint16_t* bs = Bs + buf * kTileElems;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint4*>(as + (tid / 8 + 32 * i) * LDK + (tid % 8) * 8) = ra[i];
    if (!NN) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<uint4*>(bs + (tid / 8 + 32 * i) * LDK + (tid % 8) * 8) = rb[i];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<uint4*>(bs + (tid / 16 + 16 * i) * LDN + (tid % 16) * 8) = rb[i];
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};

  if (kt0 < kt1) {
    gload(kt0);
    lstore(0);
    __syncthreads();
    for (int kt = kt0; kt < kt1; ++kt) {
      const int buf = (kt - kt0) & 1;
      if (kt + 1 < kt1) gload(kt + 1);
      const uint16_t* as = As + buf * kTileElems;
      const uint16_t* bs = Bs + buf * kTileElems;
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        // 32x16 A fragment: lane holds row lane%32, K elements 8*(lane/32) ..
        const int kof = ks * 16 + (lane >> 5) * 8;
        bf16x8_t af[2], bf[2];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
          af[mi] = *reinterpret_cast<const bf16x8_t*>(as + (wm * 64 + mi * 32 + (lane & 31)) * LDK + kof);
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          if (NN)
            bf[f] = b_frag_tr(bs, ks, b_local_col(f, wn), lane);
          else
            bf[f] = *reinterpret_cast<const bf16x8_t*>(bs + (b_local_col(f, wn) + (lane & 31)) * LDK + kof);
        }
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int f = 0; f < 2; ++f)
            acc[mi][f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bf[f], acc[mi][f], 0, 0, 0);
      }
      if (kt + 1 < kt1) lstore(buf ^ 1);
      __syncthreads();
    }
  }

  // ---- epilogue: in each 32x32 tile, accumulator element i of a lane is row
  // 8*(i/4) + 4*(lane/32) + i%4, column lane%32
  const int col32 = lane & 31;
  auto row_of = [&](int mi, int i) { return wm * 64 + mi * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); };
  if (EPI == kEpiPartialF32) {
    float* out = (float*)p.C + (int64_t)blockIdx.z * p.M * p.N;
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const int n = n_tile * BN + b_local_col(f, wn) + col32;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = row_of(mi, i);
          if (r < rows && n < p.N) out[(int64_t)(m0 + r) * p.N + n] = acc[mi][f][i];
        }
      }
  } else if (EPI == kEpiSwiGLU) {
    uint16_t* out = (uint16_t*)p.C;
    const int c = n_tile * 64 + wn * 32 + col32;  // acc[.][0] gate, acc[.][1] up
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = row_of(mi, i);
        if (r < rows && c < p.N) {
          const float v = silu(acc[mi][0][i]) * acc[mi][1][i];
          out[(int64_t)(seg + m0 + r) * p.ldc + c] = (uint16_t)f32_to_bf16_bits(v);
        }
      }
  } else {
    uint16_t* out = (uint16_t*)p.C;
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const int c = n_tile * BN + b_local_col(f, wn) + col32;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = row_of(mi, i);
          if (r < rows && c < p.N)
            out[(int64_t)(seg + m0 + r) * p.ldc + c] = (uint16_t)f32_to_bf16_bits(acc[mi][f][i]);
        }
      }
  }
}

// ---------------------------------------------------------------------------
// Grouped expert kernel (prefill-sized batches).
//
// Work unit: one M-tile (up to 256 permuted rows of one expert) x one N-tile
// (256 B-columns; gate_up: 128 gate columns and the matching 128 up columns).
// An M-tile holds every row of an expert that has at most 256 rows, so such an
// expert's weights are read from HBM once.
//
// 8 wavefronts per block in a 2 (M) x 4 (N) arrangement.  Wave (wm, wn) owns the
// 32-row sub-tiles wm, wm+2, wm+4, wm+6 (interleaved, so that a tile with few
// rows still keeps both row halves of the block busy) and two 32-column groups;
// sub-tiles past the tile's row count skip their MFMAs.
//
// Operands move from global memory straight into LDS (global_load_lds_dwordx4,
// 16 bytes per lane; the 64 lanes of one instruction fill 1 KiB of LDS in lane
// order) through a ring of 5 stages of K = 32: while stage t is multiplied,
// stages t+1..t+4 are in flight.  The ring occupies all 160 KiB of LDS (5 x 32
// KiB, no padding); bank conflicts are avoided by XOR swizzles applied on the
// load side (each lane chooses which 16-byte chunk it fetches into its fixed
// LDS slot):
//   A stage [256 rows][32 k]: row r, k-chunk c (8 elements) sits at chunk
//     position c ^ ((r >> 2) & 3) of the 64-byte row;
//   B stage [32 k][256 n]:   k-row k, n-chunk c sits at position c ^ (4 * (k & 3))
//     of the 512-byte row.
// One barrier per stage.  Each stage is its own __shared__ object and the loop
// is unrolled over the ring, so that the compiler sees that the reads of stage
// t do not depend on the loads just issued into another stage.
constexpr int GB_M = kGroupBM, GB_N = 256, GB_K = 32, GB_STAGES = 5, GB_THREADS = 512;
constexpr int GB_A_ELEMS = GB_M * GB_K, GB_B_ELEMS = GB_K * GB_N;
constexpr int GB_STAGE_ELEMS = GB_A_ELEMS + GB_B_ELEMS;  // 16384 elements = 32 KiB
constexpr int GB_ACT_COLS = GB_N / 2;
constexpr int GB_LOADS_PER_STAGE = 4;  // per thread: 2 A + 2 B instructions
static_assert(GB_STAGES * GB_STAGE_ELEMS * 2 <= 160 * 1024, "ring fits the LDS of a CU");
static_assert(GB_A_ELEMS == GB_THREADS * 8 * 2 && GB_B_ELEMS == GB_THREADS * 8 * 2,
              "each thread moves two 16-byte chunks of A and two of B per stage");

typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt immediate (gfx9 encoding: vmcnt in bits 3:0, expcnt 6:4, lgkmcnt
// 11:8): wait until at most n vector-memory operations of this wave are
// outstanding and all of its LDS operations have completed.
constexpr int waitcnt_vm_lgkm0(int n) { return 0x0070 | n; }

template <int EPI>
__global__ __launch_bounds__(GB_THREADS) void mfma_grouped_kernel(MfmaProblem p) {
  __shared__ __attribute__((aligned(1024))) uint16_t st0[GB_STAGE_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t st1[GB_STAGE_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t st2[GB_STAGE_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t st3[GB_STAGE_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t st4[GB_STAGE_ELEMS];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // (M-tile, N-tile) of this block, XCD-aware as in mfma_kernel
  const int n_tiles = p.n_tiles;
  const int total = p.hdr->n_mtiles * n_tiles;
  const int per = (total + kXcds - 1) / kXcds;
  const int slot = blockIdx.x / kXcds;
  if (slot >= per) return;
  const int logical = (blockIdx.x % kXcds) * per + slot;
  if (logical >= total) return;
  const int2 tt = p.mtiles[logical / n_tiles];
  const int n_tile = logical % n_tiles;
  const int e = tt.x, m0 = tt.y, seg = p.offsets[e];
  const int rows = min(GB_M, p.counts[e] - m0);
  const int nkt = p.K / GB_K;

  // ---- load side.  Instruction i (0, 1) of wave w fills 1 KiB of a stage:
  // A rows 16*(2w+i) + lane/4, chunk position lane%4; B k-rows 2*(2w+i) + lane/32,
  // chunk position lane%32.  Rows past the tile's end repeat its last row and
  // columns past N read column 0, so every load is in bounds; what they bring
  // only reaches outputs that are never stored.
  const uint16_t* a_src[2];
  const uint16_t* b_src[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 16 * (2 * w + i) + (lane >> 2);
    const int c = (lane & 3) ^ ((r >> 2) & 3);
    const int64_t prow = seg + m0 + min(r, rows - 1);
    const int64_t arow = p.a_gather ? (int64_t)p.a_gather[prow] : prow;
    a_src[i] = p.A + arow * p.lda + c * 8;

    const int k = 2 * (2 * w + i) + (lane >> 5);
    const int cb = (lane & 31) ^ (4 * (k & 3));
    int gcol;
    if (EPI == kEpiSwiGLU) {
      const int col = n_tile * GB_ACT_COLS + (cb & 15) * 8;
      gcol = col < p.N ? (cb < 16 ? 0 : p.up_off) + col : 0;
    } else {
      const int col = n_tile * GB_N + cb * 8;
      gcol = col < p.N ? col : 0;
    }
    b_src[i] = p.Bg + (int64_t)e * p.b_stride + (int64_t)k * p.ldb + gcol;
  }
  const int64_t b_kstep = (int64_t)GB_K * p.ldb;
  auto issue = [&](uint16_t* stage, int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      __builtin_amdgcn_global_load_lds(a_src[i] + kt * GB_K,
                                       (lds_void_t*)(stage + (2 * w + i) * 512), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(b_src[i] + kt * b_kstep,
                                       (lds_void_t*)(stage + GB_A_ELEMS + (2 * w + i) * 512), 16,
                                       0, 0);
    }
  };

  // ---- compute side
  const int wm = w >> 2, wn = w & 3;
  auto bcol = [&](int f) { return EPI == kEpiSwiGLU ? f * GB_ACT_COLS + wn * 32 : wn * 64 + f * 32; };
  bool sub_ok[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) sub_ok[j] = 32 * (wm + 2 * j) < rows;
  f32x16_t acc[4][2];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int f = 0; f < 2; ++f) acc[j][f] = f32x16_t{};

  // per-lane LDS element offsets inside a stage (the same for every stage)
  int a_off[4][2];  // [sub-tile][k-substep of 16]
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int r = 32 * (wm + 2 * j) + (lane & 31);
      const int c = 2 * ks + (lane >> 5);
      a_off[j][ks] = r * GB_K + ((c ^ ((r >> 2) & 3)) * 8);
    }
  // B fragment of column group f, k-substep ks: two transposing reads, the second
  // 4 k-rows further on (same swizzle, since (k + 4) & 3 == k & 3).
  int b_off[2][2];
  {
    const int G = lane >> 4, j4 = (lane & 15) >> 2, q = lane & 3;
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int k = ks * 16 + 8 * (G >> 1) + j4;
        const int c = bcol(f) / 8 + 2 * (G & 1) + (q >> 1);
        b_off[f][ks] = GB_A_ELEMS + k * GB_N + ((c ^ (4 * (k & 3))) * 8) + (q & 1) * 4;
      }
  }

  auto compute = [&](const uint16_t* stage) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8_t bf[2];
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const uint16_t* bp = stage + b_off[f][ks];
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)bp);
        const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(bp + 4 * GB_N));
        typedef short s16x8_t __attribute__((ext_vector_type(8)));
        const s16x8_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        bf[f] = __builtin_bit_cast(bf16x8_t, v);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (!sub_ok[j]) continue;
        const bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(stage + a_off[j][ks]);
#pragma unroll
        for (int f = 0; f < 2; ++f)
          acc[j][f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf[f], acc[j][f], 0, 0, 0);
      }
    }
  };

  // Step t: wait for this wave's loads of stage t (the 3 later stages may stay
  // in flight), barrier (every wave's stage-t data has landed and every wave is
  // done with the slot of stage t-1), refill that slot with stage t+4, multiply
  // stage t.  Stages past the end are requested too (as copies of the last one)
  // so that every step has the same number of loads in flight; they land in
  // slots that are never read again.
  auto step = [&](const uint16_t* cur, uint16_t* refill, int t) __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0((GB_STAGES - 2) * GB_LOADS_PER_STAGE));
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    issue(refill, min(t + GB_STAGES - 1, nkt - 1));
    compute(cur);
  };

  issue(st0, 0);
  issue(st1, min(1, nkt - 1));
  issue(st2, min(2, nkt - 1));
  issue(st3, min(3, nkt - 1));
  int t = 0;
  for (; t + GB_STAGES <= nkt; t += GB_STAGES) {
    step(st0, st4, t);
    step(st1, st0, t + 1);
    step(st2, st1, t + 2);
    step(st3, st2, t + 3);
    step(st4, st3, t + 4);
  }
  if (t < nkt) step(st0, st4, t);
  if (t + 1 < nkt) step(st1, st0, t + 1);
  if (t + 2 < nkt) step(st2, st1, t + 2);
  if (t + 3 < nkt) step(st3, st2, t + 3);
  // no load may still be writing LDS when the block ends
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));

  const int col32 = lane & 31;
  uint16_t* out = (uint16_t*)p.C;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (!sub_ok[j]) continue;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 32 * (wm + 2 * j) + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
      if (r >= rows) continue;
      uint16_t* orow = out + (int64_t)(seg + m0 + r) * p.ldc;
      if (EPI == kEpiSwiGLU) {
        const int c = n_tile * GB_ACT_COLS + wn * 32 + col32;
        if (c < p.N) orow[c] = (uint16_t)f32_to_bf16_bits(silu(acc[j][0][i]) * acc[j][1][i]);
      } else {
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          const int c = n_tile * GB_N + bcol(f) + col32;
          if (c < p.N) orow[c] = (uint16_t)f32_to_bf16_bits(acc[j][f][i]);
        }
      }
    }
  }
}

hipError_t launch_mfma_nt(const NtArgs& a, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  MfmaProblem p = {};
  p.A = (const uint16_t*)a.A;
  p.lda = a.lda;
  p.B1 = (const uint16_t*)a.B1;
  p.B2 = (const uint16_t*)a.B2;
  p.ldb = a.ldb;
  p.n_split = a.n_split;
  p.K = a.K;
  p.N = a.N;
  p.M = a.M;
  p.kt_per_split = a.k_tiles_per_split;
  p.C = a.out;
  dim3 grid((a.N + BN - 1) / BN, (a.M + BM - 1) / BM, a.splits);
  mfma_kernel<false, kEpiPartialF32><<<grid, 256, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_mfma_gate_up(const GroupArgs& g, int max_mtiles, const void* h,
                               const void* gate_up, void* act, hipStream_t s) {
  if (max_mtiles == 0) return hipSuccess;
  MfmaProblem p = {};
  p.A = (const uint16_t*)h;
  p.lda = g.d;
  p.a_gather = g.perm_token;
  p.Bg = (const uint16_t*)gate_up;
  p.ldb = 2 * (int64_t)g.I;
  p.b_stride = (int64_t)g.d * 2 * g.I;
  p.up_off = g.I;
  p.K = g.d;
  p.N = g.I;
  p.mtiles = g.mtiles;
  p.hdr = g.hdr;
  p.offsets = g.offsets;
  p.counts = g.counts;
  p.C = act;
  p.ldc = g.I;
  p.n_tiles = (g.I + GB_ACT_COLS - 1) / GB_ACT_COLS;
  const int64_t blocks = ((int64_t)p.n_tiles * max_mtiles + kXcds - 1) / kXcds * kXcds;
  mfma_grouped_kernel<kEpiSwiGLU><<<dim3((unsigned)blocks), GB_THREADS, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_mfma_down(const GroupArgs& g, int max_mtiles, const void* act, const void* down,
                            void* y, hipStream_t s) {
  if (max_mtiles == 0) return hipSuccess;
  MfmaProblem p = {};
  p.A = (const uint16_t*)act;
  p.lda = g.I;
  p.a_gather = nullptr;
  p.Bg = (const uint16_t*)down;
  p.ldb = g.d;
  p.b_stride = (int64_t)g.I * g.d;
  p.K = g.I;
  p.N = g.d;
  p.mtiles = g.mtiles;
  p.hdr = g.hdr;
  p.offsets = g.offsets;
  p.counts = g.counts;
  p.C = y;
  p.ldc = g.d;
  p.n_tiles = (g.d + GB_N - 1) / GB_N;
  const int64_t blocks = ((int64_t)p.n_tiles * max_mtiles + kXcds - 1) / kXcds * kXcds;
  mfma_grouped_kernel<kEpiStore><<<dim3((unsigned)blocks), GB_THREADS, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace moe
