// Internal launch interface between the host library (moe_api.hip) and the
// kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

enum DType { kF32 = 0, kBF16 = 1 };

// Tokens handled by one block of the top-k and scatter kernels (one "chunk").
constexpr int kChunkTokens = 16;
// Rows per M-tile of the dense MFMA kernel.
constexpr int kMfmaBM = 128;
// Rows per M-tile of the grouped expert MFMA kernel: an expert's rows are cut
// into tiles of this many rows.
constexpr int kGroupBM = 256;
// B-columns per N-tile of the MFMA kernels (gate+up halves for SwiGLU).
constexpr int kMfmaBN = 128;
constexpr int kMfmaBK = 64;
// Tile of the fp32 FMA GEMM (router / shared expert of fp32 plans).
constexpr int kFmaTile = 32;

// Tile (rows, columns, K-step) of the bf16 dense K-contiguous product for M rows:
// the direct-to-LDS kernel's 256 x 256 x 64 from 256 rows on, the decode-sized
// direct-to-LDS kernel's 64 x 128 x 64 up to 64 rows, else the register-staged
// kernel's 128 x 128 x 64.  Host split-K sizing and the launcher both use this,
// so they agree on the tile.
constexpr int kNtBigTile = 256;
constexpr int kNtSkinnyRows = 64;
inline void mfma_nt_tile(int64_t M, int* tm, int* tn, int* tk) {
  const bool big = M >= kNtBigTile, skinny = M <= kNtSkinnyRows;
  *tm = big ? kNtBigTile : skinny ? kNtSkinnyRows : kMfmaBM;
  *tn = big ? kNtBigTile : kMfmaBN;
  *tk = kMfmaBK;
}

// Device-side routing summary written by the scan kernel.
struct RouteHeader {
  int32_t n_active;  // experts with at least one token
  int32_t n_mtiles;  // M-tiles of kGroupBM rows over all experts
  int32_t n_passes;  // passes of the streaming kernels: sum over experts of ceil(count / kStreamMaxMT)
  int32_t pad[13];
};

// Streaming expert kernels: tokens of one expert handled per pass over its
// weights, most blocks of one launch, most experts.
constexpr int kStreamMaxMT = 8;
constexpr int kStreamMaxBlocks = 256;
constexpr int kMaxStreamExperts = 1024;
// fp32 words of one partial-sum slot of the streaming kernels: kStreamMaxMT rows
// of an item's weight columns, one 16-byte vector per lane at most (gate_up: 256
// lanes of gate and 256 of up columns; down: 768 lanes), enough for both kernels.
inline int64_t stream_slot_floats(int dtype, int I, int d) {
  const int64_t v = dtype == kBF16 ? 8 : 4;
  const int64_t gu = 2 * (256 * v < I ? 256 * v : I), dn = 768 * v < d ? 768 * v : d;
  return (int64_t)kStreamMaxMT * (gu > dn ? gu : dn);
}

// ---------------------------------------------------------------- small kernels
// h[t] = RMSNorm(x[t]) * w for T rows of d features; rows ldx / ldh elements apart.
hipError_t launch_rmsnorm(int dtype, const void* x, int64_t ldx, const void* w, void* h,
                          int64_t ldh, int64_t T, int d, float eps, hipStream_t s);

// out_part[z][m][n] = sum_{k in split z} A[m][k] * B[n][k]; B row n is
// B1 + n*ldb for n < n_split, else B2 + (n - n_split)*ldb.  fp32 results.
struct NtArgs {
  const void* A;
  int64_t lda;
  const void* B1;
  const void* B2;
  int64_t ldb;
  int n_split;
  float* out;  // [splits][M][N]
  int M, N, K;
  int splits;
  int k_tiles_per_split;  // in units of the kernel's K tile
};
hipError_t launch_fma_nt(int dtype, const NtArgs& a, hipStream_t s);
// The decode-sized bf16 product (a.M <= kNtSkinnyRows) plus sh.blocks extra blocks
// that compute act_s columns [sh.col0, sh.col1) of the shared expert (SharedSmall,
// below).
struct SharedSmall;
hipError_t launch_mfma_nt_shared(const NtArgs& a, const SharedSmall& sh, hipStream_t s);
hipError_t launch_mfma_nt(const NtArgs& a, hipStream_t s);
// The gate/up product of a SwiGLU MLP with its epilogue fused (bf16 only, one K
// split, at least kNtBigTile rows): B rows [0, n_split) are the gate rows (B1)
// and [n_split, N) the up rows (B2), N = 2 n_split; writes act [M, n_split] bf16
// = silu(A gate^T) * (A up^T), each element rounded once.
inline bool nt_swiglu_fused(int64_t M, int splits) { return M >= kNtBigTile && splits == 1; }
hipError_t launch_mfma_nt_swiglu(const NtArgs& a, void* act, hipStream_t s);

hipError_t launch_topk(const float* logit_part, int splits, const float* corr_bias, int64_t T,
                       int E, int k, float routed_scale, int32_t* topk_idx, float* topk_w,
                       int32_t* chunk_cnt, hipStream_t s);

// Also writes pass_base[i], the first streaming pass of the i-th active expert
// (i <= n_active; pass_base[n_active] = n_passes).
hipError_t launch_scan(int32_t* chunk_cnt, int nchunks, int E, int32_t* counts, int32_t* offsets,
                       RouteHeader* hdr, int32_t* active, int2* mtiles, int32_t* pass_base,
                       hipStream_t s);

// The shared expert of a bf16 batch of at most kSharedSmallTokens tokens, computed
// by extra blocks of the router product and the two small-batch routing launches
// below: gate/up and the SwiGLU beside the router and the selection (act_s, bf16,
// each launch a range of its columns), down beside the permutation (y_s, fp32, one
// partial-sum set for the combine).  T = 0: no shared work in those launches.
struct bf16;
constexpr int kSharedSmallTokens = 4;
struct SharedSmall {
  const bf16* h;     // [T, d]
  const bf16* gate;  // [Is, d]
  const bf16* up;    // [Is, d]
  const bf16* down;  // [d, Is]
  bf16* act_s;       // [T, Is]
  float* y_s;        // [T, d]
  int T, d, Is;
  int blocks;        // extra blocks of the launch
  int col0, col1;    // act_s columns [col0, col1) of a gate/up launch
};
// Host-side check of a descriptor (T = 0: none).
inline bool shared_small_ok(const SharedSmall& sh) {
  if (sh.T == 0) return true;
  return sh.T > 0 && sh.T <= kSharedSmallTokens && sh.blocks > 0 && sh.blocks <= 65536 &&
         sh.d > 0 && sh.d % 64 == 0 && sh.Is > 0 && sh.Is % 64 == 0 && 0 <= sh.col0 &&
         sh.col0 <= sh.col1 && sh.col1 <= sh.Is && sh.h && sh.gate && sh.up && sh.down &&
         sh.act_s && sh.y_s;
}

// Small batches (T * k <= kRouteSmallMax, E <= 1024): selection with one block
// per token (no chunk histograms), then the whole permutation (counts, what
// launch_scan writes, perm_token and row_of) in one block; each launch also runs
// sh.blocks blocks of shared-expert work when sh.T > 0.
constexpr int kRouteSmallMax = 2048;
hipError_t launch_topk_small(const float* logit_part, int splits, const float* corr_bias,
                             int64_t T, int E, int k, float routed_scale, int32_t* topk_idx,
                             float* topk_w, const SharedSmall& sh, hipStream_t s);
hipError_t launch_route_small(const int32_t* topk_idx, int64_t T, int E, int k, int32_t* counts,
                              int32_t* offsets, RouteHeader* hdr, int32_t* active, int2* mtiles,
                              int32_t* pass_base, int32_t* perm_token, int32_t* row_of,
                              const SharedSmall& sh, hipStream_t s);

hipError_t launch_scatter(const int32_t* topk_idx, const int32_t* chunk_base,
                          const int32_t* offsets, int64_t T, int E, int k, int32_t* perm_token,
                          int32_t* row_of, hipStream_t s);

// act[t][n] = D(silu(sum_z P[z][t][n]) * sum_z P[z][t][Is + n])
hipError_t launch_swiglu_finalize(int dtype, const float* part, int splits, int64_t T, int Is,
                                  void* act, hipStream_t s);

// out[t] = D(x[t] + (sum_z Ps[z][t] + sum_j w[t][j] * y[row_of[t][j]]))
hipError_t launch_combine(int dtype, const void* x, const float* shared_part, int splits,
                          const void* y, const float* topk_w, const int32_t* row_of, int64_t T,
                          int d, int k, void* out, hipStream_t s);

// ---------------------------------------------------------------- layout conversion
// Up to three matrices of equal element count: dst[m][c][r] = src[m][r][c] for an
// rows[m] x cols[m] matrix (both multiples of 64); rows of src / dst are ld_src /
// ld_dst elements apart.
struct TransposeBatch {
  const void* src[3];
  void* dst[3];
  int rows[3], cols[3];
  int64_t ld_src[3], ld_dst[3];
  int count;
};
hipError_t launch_transpose(int dtype, const TransposeBatch& b, hipStream_t s);

// ---------------------------------------------------------------- routed experts
struct GroupArgs {
  const int32_t* counts;
  const int32_t* offsets;
  const RouteHeader* hdr;
  const int32_t* active;     // compacted active expert ids (stream kernels)
  const int2* mtiles;        // (expert, first row) per M-tile (MFMA kernels)
  const int32_t* perm_token; // token of each permuted row (gate_up gathers h rows)
  const int32_t* pass_base;  // first streaming pass of each active expert (stream kernels)
  int E, d, I;
};

// Work balance of the streaming kernels: `blocks` blocks share the launch's rows
// of weights equally, so an (expert, pass, column strip) item can be split
// between blocks; each part leaves its fp32 sums in a slot of `parts` (two per
// block) and a fixup kernel adds them up.
struct StreamFix {
  float* parts;         // 2 * kStreamMaxBlocks slots of slot_floats words
  int64_t slot_floats;  // stream_slot_floats(dtype, I, d)
  int blocks;           // set by the launcher: resident blocks, at most kStreamMaxBlocks
};

// K split of the column-split gate_up for the fewest passes: when allowed (ok) and
// the passes would cut each row into more than 8 column parts, the gate_up launch
// instead cuts each pass into 8 column parts times S row ranges and leaves fp32
// gate and up sums per range in part ([S][rows][2I], rows = the call's permuted
// rows); the down launch then forms act = D(silu(sum gate) * sum up) from them.
struct ColKSplit {
  float* part;
  int64_t rows;
  bool ok;
};
// fp32 words the K split needs for `rows` permuted rows (S <= 8 ranges).
inline int64_t col_ksplit_floats(int64_t rows, int I) { return 8 * rows * 2 * (int64_t)I; }

// act[row][n] = D(silu(h[tok] . G[:, n]) * (h[tok] . G[:, I + n]))  for every permuted row.
// max_passes: an upper bound of the call's streaming passes (T * k); when it fits
// the resident blocks the column split runs (no partial sums, no fixup).
hipError_t launch_stream_gate_up(int dtype, const GroupArgs& g, const StreamFix& fx,
                                 int64_t max_passes, const ColKSplit& ks, const void* h,
                                 const void* gate_up, void* act, hipStream_t s);
// y[row][c] = D(act[row] . down[e][:, c])
hipError_t launch_stream_down(int dtype, const GroupArgs& g, const StreamFix& fx,
                              int64_t max_passes, const ColKSplit& ks, void* act,
                              const void* down, void* y, hipStream_t s);

// rows: T * k, the permuted rows of the call (it picks the weight loads' cache policy)
hipError_t launch_mfma_gate_up(const GroupArgs& g, int max_mtiles, int64_t rows, const void* h,
                               const void* gate_up, void* act, hipStream_t s);
hipError_t launch_mfma_down(const GroupArgs& g, int max_mtiles, const void* act, const void* down,
                            void* y, hipStream_t s);

// ---------------------------------------------------------------- measurement
// Reads bytes (a multiple of 16) of src on `blocks` blocks; sink [1] is written only
// in a case that never arises for real data (it keeps the loads).
hipError_t launch_calib_read(const void* src, size_t bytes, int blocks, uint32_t* sink,
                             hipStream_t s);
// `iters` rounds of MFMAs on `blocks` blocks; *flops receives the FLOPs enqueued.
hipError_t launch_calib_mfma(int iters, int blocks, float* sink, double* flops, hipStream_t s);

// ---------------------------------------------------------------- fused decode
// Words of the fused kernel's synchronisation state: grid-barrier arrivals,
// barrier generation, error flag (set when a barrier wait ran out of time).
constexpr int kFusedSyncWords = 4;

struct bf16;
struct FusedArgs {
  const bf16* x;
  const bf16* norm_w;
  const bf16* router_w;
  const float* corr_bias;
  const bf16* gate_up;
  const bf16* down;
  const bf16* sg;
  const bf16* su;
  const bf16* sd;
  bf16* out;
  int64_t T;
  int d, E, I, Is, k;
  float eps, rs;
  // workspace buffers (the layouts of the multi-kernel path)
  bf16* h;
  float* logits;
  int32_t* topk_idx;
  float* topk_w;
  int32_t* chunk_cnt;
  int32_t* counts;
  int32_t* offsets;
  RouteHeader* hdr;
  int32_t* active;
  int32_t* pass_base;
  int32_t* perm_token;
  int32_t* row_of;
  bf16* act;
  bf16* y;
  float* sh_gu;
  bf16* act_s;
  float* sh_dn;
  float* parts;  // partial sums of the weight streams' split items
  // split-K of the router and shared-expert products
  int r_splits, r_kper, sg_splits, sg_kper, sd_splits, sd_kper;
  uint32_t* sync;  // kFusedSyncWords words
};
// Blocks of the fused kernel: one per compute unit (all resident at once, by the
// cooperative launch), at most kStreamMaxBlocks.
hipError_t fused_decode_blocks(int* blocks);
// Resets the synchronisation state, then runs the kernel on `blocks` blocks (a
// cooperative launch: it fails rather than start with blocks that cannot all be
// resident).
hipError_t launch_fused_decode(const FusedArgs& f, int blocks, hipStream_t s);

}  // namespace moe
