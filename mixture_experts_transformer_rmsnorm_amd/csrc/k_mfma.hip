// bf16 matrix-core (MFMA) kernels for gfx950: the dense K-contiguous products
// (router logits, shared expert) and the grouped expert matmuls of
// prefill-sized batches.  Both use v_mfma_f32_32x32x16_bf16 (fp32
// accumulation; on MI355X this form sustains about 2.0 PFLOP/s against about
// 1.7 for the 16x16x32 form).  In a 32x32 accumulator tile, element i of lane l
// is row 8*(i/4) + 4*(l/32) + i%4, column l%32; the A operand lane l holds row
// l%32, K elements 8*(l/32) .. +7, and the B operand lane l holds column l%32,
// the same K elements.
//
// Dense kernel (mfma_nt_kernel): out_part[z] = A[M, K] . B[N, K]^T over the K
// range of split z, fp32 partials.  Tile 128 x 128 x 64 per 256-thread block,
// four wavefronts in a 2 x 2 arrangement, each owning 64 rows x 64 columns as
// 2 x 2 MFMA tiles.  A and B tiles are staged in LDS with K contiguous (row
// stride 72 elements, so the 16-byte fragment reads of 16 consecutive rows hit
// distinct banks) and double buffered: the global loads of K-tile t+1 are in
// flight while tile t is multiplied.
//
// Grouped kernel (mfma_grouped_kernel): see its own description below.  Its
// weights are N-contiguous ([K, N], the grouped expert layout of
// Glm4MoeStateDictAdapter: gate_and_up_projs [E, d, 2I], down_projs [E, I, d]);
// the K-contiguous B fragments are formed by gfx950's transposing LDS read
// (ds_read_b64_tr_b16): within each 16-lane group G, output lane i, element j
// is element i%4 of the 8-byte chunk addressed by lane 4j + i/4 of the group.
// The 32x32x16 B operand wants lane l = 32*hk + 16*nb + i to hold
// B[8hk .. 8hk+7][16nb + i]; so lane (G, j, q) addresses k-row 8*(G/2) + 4h + j,
// column 16*(G%2) + 4q, and two reads (h = 0, 1) give the 8 K-consecutive values.
// A gate_up tile pairs gate columns [c, c+128) with up columns [I+c, I+c+128)
// so that silu(gate) * up is formed in registers ("GLM-5 · Input features",
// excerpt mlp).
#include <type_traits>

#include "common.h"
#include "dev_nt.h"
#include "dev_rowdot.h"
#include "kernels.h"

namespace moe {

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

constexpr int kXcds = 8;  // accelerator complex dies of an MI355X, one L2 each

enum Epi { kEpiSwiGLU = 1, kEpiStore = 2 };

struct MfmaProblem {
  // A rows (K-contiguous): dense rows m, or grouped permuted rows gathered
  // through a_gather (A row = a_gather[permuted row]) or taken directly.
  const uint16_t* A;
  int64_t lda;
  const int32_t* a_gather;
  // dense B, K-contiguous: row n at B1 + n*ldb (n < n_split) else B2 + (n-n_split)*ldb.
  const uint16_t* B1;
  const uint16_t* B2;
  int64_t ldb;
  int n_split;
  // grouped B, N-contiguous: element (k, n) of expert e at Bg + e*b_stride + k*ldb + n;
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

// ---------------------------------------------------------------------------
// Dense kernel for fewer rows (mfma_nt_kernel): one 128 x 128 tile per block
// (nt_tile_128, in dev_nt.h).
__global__ __launch_bounds__(256) void mfma_nt_kernel(NtArgs a) {
  __shared__ __attribute__((aligned(16))) NtSmem sm;
  nt_tile_128(a, blockIdx.x, blockIdx.y, blockIdx.z, sm);
}

// ---------------------------------------------------------------------------
// Dense kernel for many rows (mfma_nt_big_kernel): the same product as
// mfma_nt_kernel, 256 x 256 per block, 8 wavefronts in a 2 (M) x 4 (N)
// arrangement, each owning the interleaved 32-row sub-tiles wm, wm+2, wm+4,
// wm+6 and two 32-column groups (sub-tiles past the last row skip their MFMAs).
// Both operands are K-contiguous and move global -> LDS directly
// (global_load_lds_dwordx4) in K-steps of 64, whole 128-byte row pieces,
// through rings of 32 KiB slots, 2 for A (rows of the left operand) and 3 for B
// (rows of the right one, the weights): while step t is multiplied, A of step
// t+1 and B of steps t+1 and t+2 are in flight.  Row r's
// k-chunk c (8 elements) sits at chunk position c ^ ((r >> 1) & 7) of its
// 128-byte LDS row (chosen on the load side), so the 16-byte fragment reads of
// 16 consecutive rows hit distinct banks.  A and B fragments are both plain
// 16-byte LDS reads.  Epilogue kEpiStore writes the tile's fp32 partial sums;
// kEpiSwiGLU (one K split) multiplies 128 gate rows and the matching 128 up rows
// of B per tile, each wave's two column groups holding the gate and the up sums
// of the same 32 columns, and writes silu(gate) * up in bf16.
constexpr int NB_M = kNtBigTile, NB_N = kNtBigTile, NB_K = kMfmaBK, NB_THREADS = 512;
constexpr int NB_TILE_ELEMS = NB_M * NB_K;  // 32 KiB per operand and slot
static_assert(5 * NB_TILE_ELEMS * 2 <= 160 * 1024, "rings fit the LDS of a CU");
static_assert(NB_TILE_ELEMS == NB_THREADS * 8 * 4, "4 loads per thread and operand");

typedef __attribute__((address_space(3))) void lds_void_nt_t;

template <int EPI>
__global__ __launch_bounds__(NB_THREADS) void mfma_nt_big_kernel(MfmaProblem p) {
  __shared__ __attribute__((aligned(1024))) uint16_t sa0[NB_TILE_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t sa1[NB_TILE_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t sb0[NB_TILE_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t sb1[NB_TILE_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t sb2[NB_TILE_ELEMS];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Tiles are numbered in groups of 8 M-tiles: inside a group M-tile fastest, then
  // N-tile; then the next group; then the split.  The numbers are dealt to the 8
  // XCDs in contiguous ranges, so the 32 blocks an XCD runs at a time cover about
  // 8 M-tiles x 4 N-tiles and share their A and B rows through its L2.
  // Output columns of a tile: 256 (fp32 partial sums), or 128 act columns whose
  // 128 gate and 128 up B-rows the tile multiplies (SwiGLU epilogue).
  constexpr int NCOLS = EPI == kEpiSwiGLU ? NB_N / 2 : NB_N;
  const int m_tiles = (p.M + NB_M - 1) / NB_M, n_tiles = (p.N + NCOLS - 1) / NCOLS;
  const int nkt = p.K / NB_K;
  const int splits = (nkt + p.kt_per_split - 1) / p.kt_per_split;
  const int total = m_tiles * n_tiles * splits;
  const int per = (total + kXcds - 1) / kXcds;
  const int slot = blockIdx.x / kXcds;
  if (slot >= per) return;
  const int logical = (blockIdx.x % kXcds) * per + slot;
  if (logical >= total) return;
  constexpr int kGroupM = 8;
  const int z = logical / (m_tiles * n_tiles);
  const int l = logical % (m_tiles * n_tiles);
  const int gm0 = (l / (kGroupM * n_tiles)) * kGroupM;  // first M-tile of l's group
  const int gsz = min(kGroupM, m_tiles - gm0);          // M-tiles in that group
  const int lg = l - gm0 * n_tiles;                     // index inside the group
  const int m_tile = gm0 + lg % gsz;
  const int n_tile = lg / gsz;
  const int m0 = m_tile * NB_M, n0 = n_tile * NCOLS;
  const int rows = min(NB_M, p.M - m0);
  const int kt0 = z * p.kt_per_split;
  const int kt1 = min(nkt, kt0 + p.kt_per_split);

  // Load side.  Instruction i (0..3) of wave w fills rows 8*(4w+i) .. +7 of a
  // slot (lane/8 picks the row, lane%8 the chunk position).  A row groups that
  // lie entirely past the last row are not loaded (rows past it inside a partly
  // valid group repeat the last row); B rows past N read row 0.  Every load is
  // in bounds, and what the clamped ones bring only reaches outputs that are
  // never stored.
  const uint16_t* a_src[4];
  const uint16_t* b_src[4];
  int a_groups = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 8 * (4 * w + i) + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    a_src[i] = p.A + (int64_t)(m0 + min(r, rows - 1)) * p.lda + c * 8;
    a_groups += 8 * (4 * w + i) < rows ? 1 : 0;
    const uint16_t* brow;
    if (EPI == kEpiSwiGLU) {  // B-rows [0, 128): gate rows n0 + r; [128, 256): up rows n0 + r - 128
      const int g = n0 + (r & (NCOLS - 1));
      brow = (r < NCOLS ? p.B1 : p.B2) + (int64_t)(g < p.N ? g : 0) * p.ldb;
    } else {
      const int n = n0 + r < p.N ? n0 + r : 0;
      brow = n < p.n_split ? p.B1 + (int64_t)n * p.ldb : p.B2 + (int64_t)(n - p.n_split) * p.ldb;
    }
    b_src[i] = brow + c * 8;
  }
  a_groups = __builtin_amdgcn_readfirstlane(a_groups);
  auto issue_a = [&](uint16_t* da, int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i < a_groups)
        __builtin_amdgcn_global_load_lds(a_src[i] + kt * NB_K,
                                         (lds_void_nt_t*)(da + (4 * w + i) * 512), 16, 0, 0);
  };
  auto issue_b = [&](uint16_t* db, int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_global_load_lds(b_src[i] + kt * NB_K,
                                       (lds_void_nt_t*)(db + (4 * w + i) * 512), 16, 0, 0);
  };

  // Compute side.
  const int wm = w >> 2, wn = w & 3;
  bool sub_ok[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) sub_ok[j] = 32 * (wm + 2 * j) < rows;
  f32x16_t acc[4][2];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int f = 0; f < 2; ++f) acc[j][f] = f32x16_t{};
  const int ar = wm * 32 + (lane & 31);       // A row of sub-tile 0 (sub-tile j: + 64 j)
  // B rows of column groups 0 and 1: 32 adjacent groups of the tile, or (SwiGLU)
  // the gate rows and the up rows of the wave's 32 act columns.
  const int br0 = (EPI == kEpiSwiGLU ? wn * 32 : wn * 64) + (lane & 31);
  const int br1 = br0 + (EPI == kEpiSwiGLU ? NCOLS : 32);
  const int a_sw = (ar >> 1) & 7, b_sw0 = (br0 >> 1) & 7, b_sw1 = (br1 >> 1) & 7;

  // All four sub-tiles are multiplied whatever the row count (rows past the last
  // one hold stale or repeated data and are never stored), so the MFMA stream has
  // no branches; the fragments of k-substep ks+1 are read while the MFMAs of ks run.
  auto compute = [&](const uint16_t* as, const uint16_t* bs) __attribute__((always_inline)) {
    bf16x8_t af[2][4], bf[2][2];
    auto load = [&](int ks, int buf) __attribute__((always_inline)) {
      const int c = 2 * ks + (lane >> 5);
      bf[buf][0] = *reinterpret_cast<const bf16x8_t*>(bs + br0 * NB_K + ((c ^ b_sw0) * 8));
      bf[buf][1] = *reinterpret_cast<const bf16x8_t*>(bs + br1 * NB_K + ((c ^ b_sw1) * 8));
      const int a_chunk = (c ^ a_sw) * 8;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        af[buf][j] = *reinterpret_cast<const bf16x8_t*>(as + (ar + 64 * j) * NB_K + a_chunk);
    };
    load(0, 0);
#pragma unroll
    for (int ks = 0; ks < NB_K / 16; ++ks) {
      if (ks + 1 < NB_K / 16) load(ks + 1, (ks + 1) & 1);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[j][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks & 1][j], bf[ks & 1][0], acc[j][0], 0, 0, 0);
        acc[j][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks & 1][j], bf[ks & 1][1], acc[j][1], 0, 0, 0);
      }
    }
  };

  // Step t: wait until only this wave's B loads of step t+2 are outstanding (A of
  // step t+1, issued just before them, and B of step t+1, issued a step earlier,
  // have landed; so has all of step t), barrier (every wave's data of step t has
  // landed and every wave is done with the slots of step t-1), refill those slots
  // with A of step t+1 and B of step t+2, multiply step t.  Steps past the end
  // are copies of the last one, so that every step has the same count of loads in
  // flight; they land in slots that are never read again.
  auto step = [&](const uint16_t* a_cur, uint16_t* a_next, const uint16_t* b_cur, uint16_t* b_next,
                  int t) __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0x0070 | 4);  // vmcnt(4) lgkmcnt(0)
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    issue_a(a_next, min(t + 1, kt1 - 1));
    issue_b(b_next, min(t + 2, kt1 - 1));
    compute(a_cur, b_cur);
    // Order of the step's instructions: the 8 loads, the fragments of k-substep 0,
    // then each substep's 8 MFMAs with the next substep's 6 fragment reads between
    // them, so that LDS latency hides under the MFMAs.
    __builtin_amdgcn_sched_group_barrier(0x020, 8, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
    for (int ks = 0; ks < NB_K / 16 - 1; ++ks) {
#pragma unroll
      for (int q = 0; q < 6; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
  };

  if (kt0 < kt1) {
    issue_b(sb0, kt0);
    issue_a(sa0, kt0);
    issue_b(sb1, min(kt0 + 1, kt1 - 1));
    int t = kt0;
    for (; t + 6 <= kt1; t += 6) {
      step(sa0, sa1, sb0, sb2, t);
      step(sa1, sa0, sb1, sb0, t + 1);
      step(sa0, sa1, sb2, sb1, t + 2);
      step(sa1, sa0, sb0, sb2, t + 3);
      step(sa0, sa1, sb1, sb0, t + 4);
      step(sa1, sa0, sb2, sb1, t + 5);
    }
    if (t < kt1) step(sa0, sa1, sb0, sb2, t);
    if (t + 1 < kt1) step(sa1, sa0, sb1, sb0, t + 1);
    if (t + 2 < kt1) step(sa0, sa1, sb2, sb1, t + 2);
    if (t + 3 < kt1) step(sa1, sa0, sb0, sb2, t + 3);
    if (t + 4 < kt1) step(sa0, sa1, sb1, sb0, t + 4);
    // no load may still be writing LDS when the block ends
    __builtin_amdgcn_s_waitcnt(0x0070);
  }

  const int col32 = lane & 31;
  if constexpr (EPI == kEpiSwiGLU) {
    // act[m][n] = silu(gate) * up, bf16, row stride ldc
    uint16_t* act = (uint16_t*)p.C;
    const int n = n0 + wn * 32 + col32;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (!sub_ok[j] || n >= p.N) continue;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 32 * (wm + 2 * j) + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
        if (r < rows)
          act[(int64_t)(m0 + r) * p.ldc + n] =
              (uint16_t)f32_to_bf16_bits(silu(acc[j][0][i]) * acc[j][1][i]);
      }
    }
  } else {
    float* out = (float*)p.C + (int64_t)z * p.M * p.N;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (!sub_ok[j]) continue;
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const int n = n0 + wn * 64 + f * 32 + col32;
        if (n >= p.N) continue;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = 32 * (wm + 2 * j) + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
          if (r < rows) out[(int64_t)(m0 + r) * p.N + n] = acc[j][f][i];
        }
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
// order), in K-steps of 64, through two rings that together fill the 160 KiB
// of LDS: A (activations, mostly L2 hits) has 2 slots of 256 x 64, B (weights,
// streamed from HBM) has 3 slots of 64 x 256.  While step t is multiplied, A of
// step t+1 and B of steps t+1 and t+2 are in flight.  A rows are fetched as
// whole 128-byte lines, and the A loads of 8-row groups that lie entirely past
// the tile's rows are skipped.  Bank conflicts are avoided by XOR swizzles
// applied on the load side (each lane chooses which 16-byte chunk it fetches
// into its fixed LDS slot):
//   A slot [256 rows][64 k]: row r, k-chunk c (8 elements) sits at chunk
//     position c ^ ((r >> 1) & 7) of the 128-byte row;
//   B slot [64 k][256 n]:    k-row k, n-chunk c sits at position c ^ (4 * (k & 3))
//     of the 512-byte row.
// One barrier per K-step.  Each slot is its own __shared__ object and the loop
// is unrolled over both rings (6 steps), so that the compiler sees that the
// reads of step t do not depend on the loads just issued into other slots.
constexpr int GB_M = kGroupBM, GB_N = 256, GB_K = 64, GB_THREADS = 512;
constexpr int kGroupMT = 4;  // M-tiles of one expert per group of the tile order
constexpr int GB_A_ELEMS = GB_M * GB_K, GB_B_ELEMS = GB_K * GB_N;  // 32 KiB each
constexpr int GB_ACT_COLS = GB_N / 2;
constexpr int GB_A_LOADS = GB_A_ELEMS / (GB_THREADS * 8);  // per thread and step: 4
constexpr int GB_B_LOADS = GB_B_ELEMS / (GB_THREADS * 8);  // 4
static_assert((2 * GB_A_ELEMS + 3 * GB_B_ELEMS) * 2 <= 160 * 1024, "rings fit the LDS of a CU");
static_assert(GB_A_LOADS == 4 && GB_B_LOADS == 4, "load assignment below");

typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt immediate (gfx9 encoding: vmcnt in bits 3:0, expcnt 6:4, lgkmcnt
// 11:8): wait until at most n vector-memory operations of this wave are
// outstanding and all of its LDS operations have completed.
constexpr int waitcnt_vm_lgkm0(int n) { return 0x0070 | n; }

template <int EPI, int BAUX>
__global__ __launch_bounds__(GB_THREADS) void mfma_grouped_kernel(MfmaProblem p) {
  __shared__ __attribute__((aligned(1024))) uint16_t sa0[GB_A_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t sa1[GB_A_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t sb0[GB_B_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t sb1[GB_B_ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t sb2[GB_B_ELEMS];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // (M-tile, N-tile) of this block.  Work-groups are dispatched round-robin over
  // the 8 XCDs; XCD x gets the contiguous range [x*per, (x+1)*per) of the
  // (M-tile, N-tile) pairs that exist, M-tile major, so that the N-tiles of one
  // M-tile share x's L2 for the gathered A rows.
  const int n_tiles = p.n_tiles;
  const int total = p.hdr->n_mtiles * n_tiles;
  const int per = (total + kXcds - 1) / kXcds;
  const int slot = blockIdx.x / kXcds;
  if (slot >= per) return;
  const int logical = (blockIdx.x % kXcds) * per + slot;
  if (logical >= total) return;
  // The tiles of one expert hold the logical range [b * n_tiles, (b + me) * n_tiles)
  // (its M-tiles are entries b .. b + me - 1 of the M-tile list).  Inside that range
  // they go in groups of kGroupMT M-tiles, N-tile outer and M-tile inner, so that
  // the blocks that read the same weight columns are adjacent (they start together
  // on one XCD and share its L2), and the 32 blocks an XCD runs at a time cover about
  // 4 M-tiles x 8 N-tiles of a busy expert instead of 2 x 16.
  const int q = logical / n_tiles;
  const int e = p.mtiles[q].x;
  const int b = q - p.mtiles[q].y / GB_M;
  const int me = (p.counts[e] + GB_M - 1) / GB_M;
  const int j = logical - b * n_tiles;
  const int g0 = j / (kGroupMT * n_tiles) * kGroupMT;
  const int gsz = min(kGroupMT, me - g0);
  const int jj = j - g0 * n_tiles;
  const int n_tile = jj / gsz;
  const int m0 = (g0 + jj % gsz) * GB_M, seg = p.offsets[e];
  const int rows = min(GB_M, p.counts[e] - m0);
  const int nkt = p.K / GB_K;

  // ---- load side.  A instruction i (0..3) of wave w fills the 8-row group
  // g = w + 8i, rows 8g .. 8g+7 (lane/8 picks the row, lane%8 the chunk
  // position), so a tile with few rows spreads its A loads over all waves; it is
  // issued only if its first row lies inside the tile (rows past the end inside
  // a partly valid group repeat the tile's last row).  B instruction i fills
  // k-rows 2*(4w+i) + lane/32, chunk position lane%32; columns past N read
  // column 0.  Every load is in bounds, and what the clamped ones bring only
  // reaches outputs that are never stored.
  const uint16_t* a_src[GB_A_LOADS];
  const uint16_t* b_src[GB_B_LOADS];
  int a_groups = 0;  // A instructions of this wave that are issued (a prefix of i)
#pragma unroll
  for (int i = 0; i < GB_A_LOADS; ++i) {
    const int r = 8 * (w + 8 * i) + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    const int64_t prow = seg + m0 + min(r, rows - 1);
    const int64_t arow = p.a_gather ? (int64_t)p.a_gather[prow] : prow;
    a_src[i] = p.A + arow * p.lda + c * 8;
    a_groups += 8 * (w + 8 * i) < rows ? 1 : 0;
  }
  a_groups = __builtin_amdgcn_readfirstlane(a_groups);
#pragma unroll
  for (int i = 0; i < GB_B_LOADS; ++i) {
    const int k = 2 * (4 * w + i) + (lane >> 5);
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
  // Weight loads with cache-policy bits BAUX: nontemporal (2) for gate_up when the
  // experts average fewer rows than one M-tile, so that no other block reads the
  // same weights and keeping them out of L2 keeps the gathered activation rows
  // there (4096-token GLM-5 prefill: gate_up 6 % faster); plain (0) when experts
  // span several M-tiles, whose blocks read each weight column at about the same
  // time on the same XCD through L2 (mid-size and Zipf prefill: 2-5 % faster), and
  // for down, whose activation tile is small.
  auto issue_a = [&](uint16_t* dst, int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < GB_A_LOADS; ++i)
      if (i < a_groups)
        __builtin_amdgcn_global_load_lds(a_src[i] + kt * GB_K,
                                         (lds_void_t*)(dst + (w + 8 * i) * 512), 16, 0, 0);
  };
  auto issue_b = [&](uint16_t* dst, int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < GB_B_LOADS; ++i)
      __builtin_amdgcn_global_load_lds(b_src[i] + kt * b_kstep,
                                       (lds_void_t*)(dst + (4 * w + i) * 512), 16, 0, BAUX);
  };

  // ---- compute side
  const int wm = w >> 2, wn = w & 3;
  auto bcol = [&](int f) { return EPI == kEpiSwiGLU ? f * GB_ACT_COLS + wn * 32 : wn * 64 + f * 32; };
  // Sub-tiles j of this wave (rows 32 (wm + 2j) ..) that hold rows of the tile:
  // a prefix j < nj, the same for the whole block, so each wave runs the K loop
  // specialised for its nj with no branches among its MFMAs.
  int nj = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) nj += 32 * (wm + 2 * j) < rows ? 1 : 0;
  nj = __builtin_amdgcn_readfirstlane(nj);

  // per-lane LDS element offsets inside a slot (the same for every step)
  const int arow_l = wm * 32 + (lane & 31);  // row inside sub-tile 0 of this wave
  const int a_sw = (arow_l >> 1) & 7;        // (r >> 1) & 7 is the same for r + 64 j
  const int a_base = arow_l * GB_K;
  // B fragment of column group f, k-substep ks: two transposing reads, the second
  // 4 k-rows further on (same swizzle, since (k + 4) & 3 == k & 3).
  int b_off[2][4];
  {
    const int G = lane >> 4, j4 = (lane & 15) >> 2, q = lane & 3;
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int k = ks * 16 + 8 * (G >> 1) + j4;
        const int c = bcol(f) / 8 + 2 * (G & 1) + (q >> 1);
        b_off[f][ks] = k * GB_N + ((c ^ (4 * (k & 3))) * 8) + (q & 1) * 4;
      }
  }

  f32x16_t acc[4][2];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int f = 0; f < 2; ++f) acc[j][f] = f32x16_t{};

  // The K loop for a wave with NJ sub-tiles.  The fragments of k-substep ks+1
  // are read while the MFMAs of ks run.  Step t: wait until only this wave's B
  // loads of step t+1 are outstanding (A of step t, issued before them, and B of
  // step t, issued earlier, have landed), barrier (every wave's data of step t
  // has landed and every wave is done with the slots of step t-1), refill those
  // slots with A of step t+1 and B of step t+2, multiply step t.  Steps past the
  // end are requested too (as copies of the last one) so that the count of
  // loads in flight is the same at every step; they land in slots that are
  // never read again.  Every wave passes the same barriers whatever its NJ.
  auto k_loop = [&](auto nj_c) __attribute__((always_inline)) {
    constexpr int NJ = decltype(nj_c)::value;
    auto compute = [&](const uint16_t* as, const uint16_t* bs) __attribute__((always_inline)) {
      bf16x8_t af[2][NJ > 0 ? NJ : 1], bf[2][2];
      auto load = [&](int ks, int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          const uint16_t* bp = bs + b_off[f][ks];
          const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)bp);
          const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(bp + 4 * GB_N));
          typedef short s16x8_t __attribute__((ext_vector_type(8)));
          const s16x8_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          bf[buf][f] = __builtin_bit_cast(bf16x8_t, v);
        }
        const int a_chunk = ((2 * ks + (lane >> 5)) ^ a_sw) * 8;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          af[buf][j] = *reinterpret_cast<const bf16x8_t*>(as + a_base + j * 64 * GB_K + a_chunk);
      };
      load(0, 0);
#pragma unroll
      for (int ks = 0; ks < GB_K / 16; ++ks) {
        if (ks + 1 < GB_K / 16) load(ks + 1, (ks + 1) & 1);
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int f = 0; f < 2; ++f)
            acc[j][f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks & 1][j], bf[ks & 1][f],
                                                                acc[j][f], 0, 0, 0);
      }
    };
    auto step = [&](const uint16_t* a_cur, uint16_t* a_next, const uint16_t* b_cur,
                    uint16_t* b_next, int t) __attribute__((always_inline)) {
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(GB_B_LOADS));
      __asm__ volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      __asm__ volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      issue_a(a_next, min(t + 1, nkt - 1));
      issue_b(b_next, min(t + 2, nkt - 1));
      if constexpr (NJ > 0) {
        compute(a_cur, b_cur);
        // Order: the fragments of substep 0, then each substep's MFMAs with the
        // next substep's fragment reads (4 transposing B reads, NJ A reads)
        // between them, so that LDS latency hides under the MFMAs.
        constexpr int R = 4 + NJ, M = 2 * NJ;
        __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
#pragma unroll
        for (int ks = 0; ks < GB_K / 16 - 1; ++ks) {
#pragma unroll
          for (int q = 0; q < (M < R ? M : R); ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          if constexpr (R > M) __builtin_amdgcn_sched_group_barrier(0x100, R - M, 0);
          if constexpr (M > R) __builtin_amdgcn_sched_group_barrier(0x008, M - R, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, M, 0);
      }
    };
    issue_b(sb0, 0);
    issue_a(sa0, 0);
    issue_b(sb1, min(1, nkt - 1));
    int t = 0;
    for (; t + 6 <= nkt; t += 6) {
      step(sa0, sa1, sb0, sb2, t);
      step(sa1, sa0, sb1, sb0, t + 1);
      step(sa0, sa1, sb2, sb1, t + 2);
      step(sa1, sa0, sb0, sb2, t + 3);
      step(sa0, sa1, sb1, sb0, t + 4);
      step(sa1, sa0, sb2, sb1, t + 5);
    }
    if (t < nkt) step(sa0, sa1, sb0, sb2, t);
    if (t + 1 < nkt) step(sa1, sa0, sb1, sb0, t + 1);
    if (t + 2 < nkt) step(sa0, sa1, sb2, sb1, t + 2);
    if (t + 3 < nkt) step(sa1, sa0, sb0, sb2, t + 3);
    if (t + 4 < nkt) step(sa0, sa1, sb1, sb0, t + 4);
    // no load may still be writing LDS when the block ends
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
  };
  switch (nj) {
    case 0: k_loop(std::integral_constant<int, 0>{}); break;
    case 1: k_loop(std::integral_constant<int, 1>{}); break;
    case 2: k_loop(std::integral_constant<int, 2>{}); break;
    case 3: k_loop(std::integral_constant<int, 3>{}); break;
    default: k_loop(std::integral_constant<int, 4>{}); break;
  }

  // ---- epilogue.  Each wave stages one of its 32-row sub-tiles at a time in a
  // private LDS region (its 32 or 64 columns of the tile, rows padded by 16
  // bytes so that the two row halves of an accumulator write use different
  // banks), then stores whole 16-byte vectors of consecutive columns: a row's
  // piece of the wave is one 128-byte line (down) or half of one (gate_up),
  // written by 8 or 4 lanes of one instruction.  The stores are nontemporal
  // (the outputs are read by the next kernel, not by this one): prefill
  // gate_up and down are 3 % faster than with plain stores, and 16-byte stores
  // are faster than storing each lane's 2-byte elements.
  constexpr int OC = EPI == kEpiSwiGLU ? 32 : 64;  // output columns of a wave
  constexpr int RSE = OC + 8;                       // LDS row stride, elements
  constexpr int CPR = OC / 8;                       // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;                     // rows per store instruction
  static_assert(4 * 32 * RSE <= GB_B_ELEMS, "four waves' regions fit one B slot");
  __syncthreads();  // every wave is done with the rings and its loads have landed
  uint16_t* stage = (w < 4 ? sb0 : sb1) + (w & 3) * 32 * RSE;
  const int col32 = lane & 31;
  const int c0 = EPI == kEpiSwiGLU ? n_tile * GB_ACT_COLS + wn * 32 : n_tile * GB_N + wn * 64;
  uint16_t* out = (uint16_t*)p.C;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (j >= nj) continue;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
      if (EPI == kEpiSwiGLU) {
        stage[r * RSE + col32] = (uint16_t)f32_to_bf16_bits(silu(acc[j][0][i]) * acc[j][1][i]);
      } else {
#pragma unroll
        for (int f = 0; f < 2; ++f)
          stage[r * RSE + f * 32 + col32] = (uint16_t)f32_to_bf16_bits(acc[j][f][i]);
      }
    }
    // LDS operations of a wave complete in order: the reads below see the writes
    // above, and the next sub-tile's writes come after these reads.
#pragma unroll
    for (int q = 0; q < 32 / RPI; ++q) {
      const int rr = q * RPI + lane / CPR, ch = lane % CPR;
      const uint4 v = *reinterpret_cast<const uint4*>(stage + rr * RSE + ch * 8);
      const int r = 32 * (wm + 2 * j) + rr, c = c0 + ch * 8;
      if (r < rows && c < p.N) {
        const u32x4_t t = {v.x, v.y, v.z, v.w};
        __builtin_nontemporal_store(
            t, reinterpret_cast<u32x4_t*>(out + (int64_t)(seg + m0 + r) * p.ldc + c));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Dense kernel for decode-sized batches (mfma_nt_skinny_kernel): the same
// product for M <= 64 rows, one 64 x 128 tile (all rows, 128 B-rows) and the K
// range of split z per block, 4 wavefronts each owning 32 B-rows (the columns of
// the output) for both 32-row halves.  The product streams B (weights, read
// once, nontemporal loads) from HBM: both operands move global -> LDS directly
// through a ring of 6 stages (A 64 x 64 and B 128 x 64 elements each, with the
// XOR swizzle of the 256-row kernel), so 5 K-steps of loads are in flight per
// compute unit while one is multiplied.  Rows past M load row M - 1 and B rows
// past N load row 0 (in bounds; their outputs are not stored), so every stage
// issues the same 6 loads per thread.  No stage is requested past the split's
// last K-tile; the last steps, which have fewer stages after them, wait for
// every load of the wave.
constexpr int NS_M = kNtSkinnyRows, NS_N = kMfmaBN, NS_K = kMfmaBK, NS_THREADS = 256;
constexpr int NS_STAGES = 6;
constexpr int NS_A_ELEMS = NS_M * NS_K, NS_B_ELEMS = NS_N * NS_K;  // 8 and 16 KiB
constexpr int NS_STAGE_ELEMS = NS_A_ELEMS + NS_B_ELEMS;
constexpr int NS_LOADS = (NS_A_ELEMS + NS_B_ELEMS) / (NS_THREADS * 8);  // per thread and stage
static_assert(NS_STAGES * NS_STAGE_ELEMS * 2 <= 160 * 1024, "the ring fits the LDS of a CU");
static_assert(NS_LOADS == 6 && NS_A_ELEMS == 2 * NS_THREADS * 8, "load assignment below");

// s_waitcnt immediate: at most n (< 64) vector-memory operations of this wave
// outstanding (vmcnt bits 3:0 and 15:14) and all of its LDS operations completed.
constexpr int waitcnt_vm_n_lgkm0(int n) { return ((n >> 4) << 14) | 0x0070 | (n & 15); }

// One global -> LDS load of 16 bytes per lane (global_load_lds_dwordx4): lane l's
// bytes land at LDS byte address lds + 16 l; lds must be the same in every lane.
// NT marks the load nontemporal.  Written as an asm statement so that the
// compiler does not track these LDS writes itself: with the ring slot chosen at
// run time it would otherwise wait for every load in flight before each LDS
// read; the kernel's own waits order them.  The instruction has no result
// registers (it writes LDS only); M0 is set in the same statement, one wait
// state ahead of its use, and nothing else in the kernel that calls it uses M0.
template <bool NT>
__device__ __forceinline__ void lds_dma16(const void* src, uint32_t lds) {
  if constexpr (NT)
    __asm__ volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
                     :
                     : "v"(src), "s"(lds)
                     : "memory", "m0");
  else
    __asm__ volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                     :
                     : "v"(src), "s"(lds)
                     : "memory", "m0");
}

// SH: blocks past the product's own compute act_s columns of the shared expert
// (dev_rowdot.h) in the ring's LDS.
template <bool SH>
__global__ __launch_bounds__(NS_THREADS) void mfma_nt_skinny_kernel(NtArgs a, SharedSmall sh) {
  __shared__ __attribute__((aligned(1024))) uint16_t lds[NS_STAGES * NS_STAGE_ELEMS];
  const int n_tiles = (a.N + NS_N - 1) / NS_N;
  if constexpr (SH) {
    static_assert(NS_STAGES * NS_STAGE_ELEMS * 2 >= kRdGroupLds * 4, "row-dot LDS");
    if ((int)blockIdx.x >= n_tiles * a.splits) {
      shared_gate_up_block(sh, (int)blockIdx.x - n_tiles * a.splits, sh.blocks,
                           reinterpret_cast<float*>(lds));
      return;
    }
  }
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_tile = blockIdx.x % n_tiles, z = blockIdx.x / n_tiles;
  const int nkt = a.K / NS_K;
  const int kt0 = z * a.k_tiles_per_split;
  const int kt1 = min(nkt, kt0 + a.k_tiles_per_split);
  if (kt0 >= kt1) return;
  const int n0 = n_tile * NS_N;
  const uint16_t* A = (const uint16_t*)a.A;
  const uint16_t* B1 = (const uint16_t*)a.B1;
  const uint16_t* B2 = (const uint16_t*)a.B2;

  // Load side: instruction i of wave w fills the 8 rows 8 (w + 4i) .. +7 of the
  // A part (i < 2) or of the B part (i < 4), lane / 8 picking the row and
  // lane % 8 the chunk position; row r's k-chunk c sits at position
  // c ^ ((r >> 1) & 7) of its 128-byte LDS row.
  const uint16_t* a_src[2];
  const uint16_t* b_src[4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 8 * (w + 4 * i) + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    a_src[i] = A + (int64_t)min(r, a.M - 1) * a.lda + c * 8;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 8 * (w + 4 * i) + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    const int n = n0 + r < a.N ? n0 + r : 0;
    const uint16_t* brow = n < a.n_split ? B1 + (int64_t)n * a.ldb : B2 + (int64_t)(n - a.n_split) * a.ldb;
    b_src[i] = brow + c * 8;
  }
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint16_t*)lds;
  // Stage of K-tile kt into ring slot q.
  auto issue = [&](int kt, int q) __attribute__((always_inline)) {
    const int k0 = kt * NS_K;
    const uint32_t base = lds_base + (uint32_t)(q * NS_STAGE_ELEMS) * 2;
#pragma unroll
    for (int i = 0; i < 2; ++i) lds_dma16<false>(a_src[i] + k0, base + (w + 4 * i) * 1024);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      lds_dma16<true>(b_src[i] + k0, base + NS_A_ELEMS * 2 + (w + 4 * i) * 1024);
  };

  // Compute side: A fragment of rows 32 j + lane % 32, B fragment of B-rows
  // 32 w + lane % 32, both at k-chunk 2 ks + lane / 32.
  const int ra = lane & 31, rb = 32 * w + (lane & 31);
  f32x16_t acc[2] = {f32x16_t{}, f32x16_t{}};

  // Step kt: wait until only the loads of the stages after kt are outstanding
  // (all of them while fewer than 4 follow), barrier (every wave's stage kt has
  // landed and every wave is done with the slot of step kt - 1), refill that
  // slot with stage kt + 5, multiply stage kt.
  int q = 0;  // slot of step kt
#pragma unroll
  for (int s = 0; s < NS_STAGES - 1; ++s)
    if (kt0 + s < kt1) issue(kt0 + s, s);
  for (int kt = kt0; kt < kt1; ++kt) {
    __builtin_amdgcn_sched_barrier(0);
    if (kt + NS_STAGES - 2 < kt1)
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_n_lgkm0((NS_STAGES - 2) * NS_LOADS));
    else
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_n_lgkm0(0));
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    if (kt + NS_STAGES - 1 < kt1) issue(kt + NS_STAGES - 1, q == 0 ? NS_STAGES - 1 : q - 1);
    const uint16_t* as = lds + q * NS_STAGE_ELEMS;
    const uint16_t* bs = as + NS_A_ELEMS;
#pragma unroll
    for (int ks = 0; ks < NS_K / 16; ++ks) {
      const int ch = 2 * ks + (lane >> 5);
      const bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(bs + rb * NS_K + ((ch ^ ((rb >> 1) & 7)) * 8));
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = 32 * j + ra;
        const bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(as + r * NS_K + ((ch ^ ((r >> 1) & 7)) * 8));
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, b, acc[j], 0, 0, 0);
      }
    }
    q = q == NS_STAGES - 1 ? 0 : q + 1;
  }
  // no load may still be writing LDS when the block ends
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_n_lgkm0(0));

  // fp32 partial sums of split z: element i of lane l in a 32x32 tile is row
  // 8 (i / 4) + 4 (l / 32) + i % 4, column l % 32.
  float* out = a.out + (int64_t)z * a.M * a.N;
  const int n = n0 + 32 * w + (lane & 31);
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 32 * j + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
      if (r < a.M && n < a.N) out[(int64_t)r * a.N + n] = acc[j][i];
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
  int tm, tn, tk;
  mfma_nt_tile(a.M, &tm, &tn, &tk);
  if (tm == NB_M) {
    const int64_t tiles = (int64_t)((a.M + NB_M - 1) / NB_M) * ((a.N + NB_N - 1) / NB_N) * a.splits;
    const int64_t blocks = (tiles + kXcds - 1) / kXcds * kXcds;
    mfma_nt_big_kernel<kEpiStore><<<dim3((unsigned)blocks), NB_THREADS, 0, s>>>(p);
  } else if (tm == NS_M) {
    const int64_t blocks = (int64_t)((a.N + NS_N - 1) / NS_N) * a.splits;
    mfma_nt_skinny_kernel<false><<<dim3((unsigned)blocks), NS_THREADS, 0, s>>>(a, SharedSmall{});
  } else {
    dim3 grid((a.N + kNtBN - 1) / kNtBN, (a.M + kNtBM - 1) / kNtBM, a.splits);
    mfma_nt_kernel<<<grid, 256, 0, s>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_mfma_nt_shared(const NtArgs& a, const SharedSmall& sh, hipStream_t s) {
  int tm, tn, tk;
  mfma_nt_tile(a.M, &tm, &tn, &tk);
  if (a.M == 0 || tm != NS_M || !shared_small_ok(sh) || (sh.T > 0 && sh.T != a.M))
    return hipErrorInvalidValue;
  const int64_t blocks = (int64_t)((a.N + NS_N - 1) / NS_N) * a.splits;
  const unsigned grid = (unsigned)blocks + (sh.T > 0 ? (unsigned)sh.blocks : 0u);
  mfma_nt_skinny_kernel<true><<<dim3(grid), NS_THREADS, 0, s>>>(a, sh);
  return hipGetLastError();
}

hipError_t launch_mfma_nt_swiglu(const NtArgs& a, void* act, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  if (!nt_swiglu_fused(a.M, a.splits) || 2 * a.n_split != a.N) return hipErrorInvalidValue;
  MfmaProblem p = {};
  p.A = (const uint16_t*)a.A;
  p.lda = a.lda;
  p.B1 = (const uint16_t*)a.B1;
  p.B2 = (const uint16_t*)a.B2;
  p.ldb = a.ldb;
  p.n_split = a.n_split;
  p.K = a.K;
  p.N = a.n_split;  // act columns
  p.M = a.M;
  p.kt_per_split = a.K / NB_K;
  p.C = act;
  p.ldc = a.n_split;
  const int64_t tiles = (int64_t)((a.M + NB_M - 1) / NB_M) * ((p.N + NB_N / 2 - 1) / (NB_N / 2));
  const int64_t blocks = (tiles + kXcds - 1) / kXcds * kXcds;
  mfma_nt_big_kernel<kEpiSwiGLU><<<dim3((unsigned)blocks), NB_THREADS, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_mfma_gate_up(const GroupArgs& g, int max_mtiles, int64_t rows, const void* h,
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
  if (rows < (int64_t)GB_M * g.E)  // fewer rows than one M-tile per expert on average
    mfma_grouped_kernel<kEpiSwiGLU, 2><<<dim3((unsigned)blocks), GB_THREADS, 0, s>>>(p);
  else
    mfma_grouped_kernel<kEpiSwiGLU, 0><<<dim3((unsigned)blocks), GB_THREADS, 0, s>>>(p);
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
  mfma_grouped_kernel<kEpiStore, 0><<<dim3((unsigned)blocks), GB_THREADS, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace moe
