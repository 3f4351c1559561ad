// Bandwidth- and latency-bound kernels of the MoE sublayer for gfx950:
// RMSNorm, the fp32 FMA GEMM (router / shared expert of fp32 plans), router
// top-k, the permutation (chunk scan, expert scan, scatter), the shared-expert
// SwiGLU finalisation and the weighted combine with the residual.
#include <math.h>

#include <type_traits>

#include "common.h"
#include "dev_rowdot.h"
#include "dev_small.h"
#include "kernels.h"

namespace moe {

// ---------------------------------------------------------------------------
// RMSNorm ("GLM-5 · Input features", excerpt rmsnorm: fp32 normalisation by the
// root mean square over the feature dimension, no centring, cast back to the
// input dtype, then the per-feature gain).  The mean of squares is accumulated
// in fp64 and rounded once to fp32; sqrt and the reciprocal are evaluated in
// fp64 and rounded once, which gives exactly the IEEE fp32 sqrt and divide.
// Rows are `ldx` / `ldh` elements apart; each element of a row is read before
// the same thread writes it, so h may alias x.

// Wide rows: one 256-thread block per row (rows of up to 4 * 256 vectors are read once).
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const T* x, int64_t ldx, const T* __restrict__ w,
                                                      T* h, int64_t ldh, int d, float eps) {
  __shared__ double red[4];
  const int64_t row = blockIdx.x;
  rms_block_row<T>(x + row * ldx, w, h + row * ldh, d, eps, red);
}

// Narrower rows (the latent and per-head norms): LPR lanes per row, 256 / LPR
// rows per block, up to NV vectors per lane held in registers; the row's partial
// sums are combined by shuffles inside its lanes.
template <typename T, int LPR, int NV>
__global__ __launch_bounds__(256) void rmsnorm_rows_kernel(const T* x, int64_t ldx,
                                                           const T* __restrict__ w, T* h,
                                                           int64_t ldh, int64_t rows, int d,
                                                           float eps) {
  constexpr int V = Elem<T>::kVec;
  const int64_t row = (int64_t)blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
  if (row >= rows) return;  // whole lane groups leave together; no block barrier follows
  auto reduce = [](double ss) {
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off, kWave);
    return ss;
  };
  rms_row<T, NV>(x + row * ldx, w, h + row * ldh, d / V, threadIdx.x % LPR, LPR, d, eps, reduce);
}

template <typename T>
static hipError_t launch_rmsnorm_t(const void* x, int64_t ldx, const void* w, void* h, int64_t ldh,
                                   int64_t T_, int d, float eps, hipStream_t s) {
  constexpr int V = Elem<T>::kVec;
  const int nvec = d / V;
  const T* xp = (const T*)x;
  const T* wp = (const T*)w;
  T* hp = (T*)h;
  auto rows_launch = [&](auto lpr_tag, auto nv_tag) {
    constexpr int LPR = decltype(lpr_tag)::value, NV = decltype(nv_tag)::value;
    const int64_t blocks = (T_ + 256 / LPR - 1) / (256 / LPR);
    rmsnorm_rows_kernel<T, LPR, NV><<<dim3((unsigned)blocks), 256, 0, s>>>(xp, ldx, wp, hp, ldh, T_,
                                                                         d, eps);
  };
  using I64 = std::integral_constant<int, 64>;
  if (nvec >= 512)
    rmsnorm_kernel<T><<<dim3((unsigned)T_), 256, 0, s>>>(xp, ldx, wp, hp, ldh, d, eps);
  else if (nvec >= 256)
    rows_launch(I64{}, std::integral_constant<int, 8>{});
  else if (nvec >= 128)
    rows_launch(I64{}, std::integral_constant<int, 4>{});
  else if (nvec >= 64)
    rows_launch(I64{}, std::integral_constant<int, 2>{});
  else if (nvec >= 32)
    rows_launch(std::integral_constant<int, 32>{}, std::integral_constant<int, 2>{});
  else if (nvec >= 16)
    rows_launch(std::integral_constant<int, 16>{}, std::integral_constant<int, 2>{});
  else if (nvec >= 8)
    rows_launch(std::integral_constant<int, 8>{}, std::integral_constant<int, 2>{});
  else
    rows_launch(std::integral_constant<int, 4>{}, std::integral_constant<int, 2>{});
  return hipGetLastError();
}

hipError_t launch_rmsnorm(int dtype, const void* x, int64_t ldx, const void* w, void* h,
                          int64_t ldh, int64_t T, int d, float eps, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (dtype == kBF16) return launch_rmsnorm_t<bf16>(x, ldx, w, h, ldh, T, d, eps, s);
  return launch_rmsnorm_t<float>(x, ldx, w, h, ldh, T, d, eps, s);
}

// ---------------------------------------------------------------------------
// out[z][m][n] = sum over split z of A[m][k] * B[n][k] (both K-contiguous), fp32
// accumulation.  32x32 output tile per 256-thread block, 2x2 outputs per thread.
template <typename T>
__global__ __launch_bounds__(256) void fma_nt_kernel(NtArgs a) {
  __shared__ float As[kFmaTile][kFmaTile + 1];
  __shared__ float Bs[kFmaTile][kFmaTile + 1];
  const int tid = threadIdx.x;
  const int m0 = blockIdx.y * kFmaTile, n0 = blockIdx.x * kFmaTile, z = blockIdx.z;
  const int nkt = a.K / kFmaTile;
  const int kt0 = z * a.k_tiles_per_split;
  const int kt1 = min(nkt, kt0 + a.k_tiles_per_split);
  const T* A = (const T*)a.A;
  const int ty = tid / 16, tx = tid % 16;
  float acc[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
  for (int kt = kt0; kt < kt1; ++kt) {
    const int k0 = kt * kFmaTile;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + 256 * i, r = e / kFmaTile, c = e % kFmaTile;
      const int m = m0 + r, n = n0 + r;
      As[c][r] = (m < a.M) ? Elem<T>::load1(A, (int64_t)m * a.lda + k0 + c) : 0.f;
      float bv = 0.f;
      if (n < a.N) {
        const T* Brow = n < a.n_split ? (const T*)a.B1 + (int64_t)n * a.ldb
                                      : (const T*)a.B2 + (int64_t)(n - a.n_split) * a.ldb;
        bv = Elem<T>::load1(Brow, k0 + c);
      }
      Bs[c][r] = bv;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < kFmaTile; ++kk) {
      const float a0 = As[kk][ty * 2], a1 = As[kk][ty * 2 + 1];
      const float b0 = Bs[kk][tx * 2], b1 = Bs[kk][tx * 2 + 1];
      acc[0][0] += a0 * b0;
      acc[0][1] += a0 * b1;
      acc[1][0] += a1 * b0;
      acc[1][1] += a1 * b1;
    }
    __syncthreads();
  }
  float* out = a.out + (int64_t)z * a.M * a.N;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int m = m0 + ty * 2 + i, n = n0 + tx * 2 + j;
      if (m < a.M && n < a.N) out[(int64_t)m * a.N + n] = acc[i][j];
    }
}

hipError_t launch_fma_nt(int dtype, const NtArgs& a, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  dim3 grid((a.N + kFmaTile - 1) / kFmaTile, (a.M + kFmaTile - 1) / kFmaTile, a.splits);
  if (dtype == kBF16)
    fma_nt_kernel<bf16><<<grid, 256, 0, s>>>(a);
  else
    fma_nt_kernel<float><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Router selection.  One wavefront per token (a block holds the kChunkTokens
// tokens of one chunk): lane l holds experts l, l+64, ... (Q per lane).
// score = sigmoid(logit) in fp32; key = score + corr_bias (fp32) decides the
// selection; k rounds of a wave-wide arg-max over (key desc, expert asc); the
// weights are the selected unbiased scores renormalised to sum routed_scale.
// Each block also writes its chunk's per-expert histogram.
template <int Q, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void topk_kernel(const float* __restrict__ part,
                                                          int splits,
                                                          const float* __restrict__ bias,
                                                          int64_t T, int E, int k, float rs,
                                                          int32_t* __restrict__ idx_out,
                                                          float* __restrict__ w_out,
                                                          int32_t* __restrict__ chunk_cnt) {
  __shared__ int hist[1024];
  topk_chunk<Q, WAVES>(part, splits, bias, T, E, k, rs, idx_out, w_out, chunk_cnt, blockIdx.x, hist);
}

hipError_t launch_topk(const float* logit_part, int splits, const float* corr_bias, int64_t T,
                       int E, int k, float routed_scale, int32_t* topk_idx, float* topk_w,
                       int32_t* chunk_cnt, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 grid((unsigned)((T + kChunkTokens - 1) / kChunkTokens));
  const int q = (E + kWave - 1) / kWave;
#define MOE_TOPK(QQ, WW)                                                                    \
  topk_kernel<QQ, WW><<<grid, WW * 64, 0, s>>>(logit_part, splits, corr_bias, T, E, k,      \
                                               routed_scale, topk_idx, topk_w, chunk_cnt)
  if (q <= 1) MOE_TOPK(1, 16);
  else if (q <= 2) MOE_TOPK(2, 16);
  else if (q <= 4) MOE_TOPK(4, 16);
  else if (q <= 8) MOE_TOPK(8, 8);
  else MOE_TOPK(16, 4);
#undef MOE_TOPK
  return hipGetLastError();
}

// Router selection for small batches: one block of 256 threads per token.  The
// four wavefronts add the split-K partial logits of the splits z = w, w + 4, ...;
// wave 0 adds the four sums in order and selects (topk_select).  Blocks T and up
// compute the shared expert's act_s when sh.T > 0 (dev_rowdot.h).
template <int Q>
__global__ __launch_bounds__(256) void topk_small_kernel(const float* __restrict__ part, int splits,
                                                         const float* __restrict__ bias, int64_t T,
                                                         int E, int k, float rs,
                                                         int32_t* __restrict__ idx_out,
                                                         float* __restrict__ w_out, SharedSmall sh) {
  __shared__ float red[4][kWave * Q];
  __shared__ float s_rd[kRdGroupLds];
  if (blockIdx.x >= T) {
    shared_gate_up_block(sh, (int)(blockIdx.x - T), sh.blocks, s_rd);
    return;
  }
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const int64_t t = blockIdx.x;
  const int64_t zstride = T * (int64_t)E;
  const float* pt = part + t * E + lane;
  float l[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) l[q] = 0.f;
  for (int z0 = w; z0 < splits; z0 += 16) {
    float v[4][Q];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const int z = z0 + 4 * u;
        v[u][q] = (z < splits && lane + kWave * q < E) ? pt[z * zstride + kWave * q] : 0.f;
      }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int q = 0; q < Q; ++q) l[q] += v[u][q];
  }
#pragma unroll
  for (int q = 0; q < Q; ++q) red[w][lane + kWave * q] = l[q];
  __syncthreads();
  if (w != 0) return;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int e = lane + kWave * q;
    l[q] = ((red[0][e] + red[1][e]) + red[2][e]) + red[3][e];
  }
  topk_select<Q>(l, bias, t, E, k, rs, idx_out, w_out, nullptr);
}

// With the shared expert's blocks, each launch asks for more LDS than half a compute
// unit's 160 KiB (the kernels do not use the extra), so that the dispatcher puts one
// block on each compute unit rather than two on some and none on others.
constexpr size_t kSharedSmallLdsHold = 96 * 1024;

hipError_t launch_topk_small(const float* logit_part, int splits, const float* corr_bias,
                             int64_t T, int E, int k, float routed_scale, int32_t* topk_idx,
                             float* topk_w, const SharedSmall& sh, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (!shared_small_ok(sh) || (sh.T > 0 && sh.T != T)) return hipErrorInvalidValue;
  const int q = (E + kWave - 1) / kWave;
  const unsigned grid = (unsigned)T + (sh.T > 0 ? (unsigned)sh.blocks : 0u);
  const size_t lds = sh.T > 0 ? kSharedSmallLdsHold : 0;
#define MOE_TOPKS(QQ)                                                                      \
  topk_small_kernel<QQ><<<dim3(grid), 256, lds, s>>>(logit_part, splits, corr_bias, T, E, k, \
                                                     routed_scale, topk_idx, topk_w, sh)
  if (q <= 1) MOE_TOPKS(1);
  else if (q <= 2) MOE_TOPKS(2);
  else if (q <= 4) MOE_TOPKS(4);
  else if (q <= 8) MOE_TOPKS(8);
  else MOE_TOPKS(16);
#undef MOE_TOPKS
  return hipGetLastError();
}

// Inclusive scan of v over the 64 lanes of a wavefront.
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  return v;
}

// Permutation for small batches (T * k <= kRouteSmallMax assignments, one block
// of 1024 threads).  The assignments, in (token, j) order, are cut into 16 equal
// segments; per-segment expert histograms (LDS atomics) give each expert's count
// and, per segment, the count of the same expert's assignments in the segments
// before it.  Then what scan_experts_kernel writes (offsets, active list,
// M-tiles, pass prefix, header) from wave-level scans, and each assignment's row:
// its expert's offset, plus the count before its segment, plus the earlier
// assignments of the same expert inside the segment.  The same stable order as
// the chunked scatter.  Blocks 1 and up compute the shared expert's output y_s
// when sh.T > 0 (dev_rowdot.h; their LDS is s_hist's).
__global__ __launch_bounds__(1024) void route_small_kernel(
    const int32_t* __restrict__ topk_idx, int A, int E, int k, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, RouteHeader* __restrict__ hdr, int32_t* __restrict__ active,
    int2* __restrict__ mtiles, int32_t* __restrict__ pass_base, int32_t* __restrict__ perm_token,
    int32_t* __restrict__ row_of, SharedSmall sh) {
  constexpr int kSegs = 16;
  __shared__ int s_idx[kRouteSmallMax];
  __shared__ int s_hist[kSegs * 1024];  // [segment][expert]
  __shared__ int s_off[1024];
  __shared__ int s_wsum[kSegs][4];
  static_assert(sizeof(s_hist) >= 4 * kRdGroupLds * sizeof(float), "row-dot LDS");
  if (blockIdx.x > 0) {
    shared_down_block<4>(sh, (int)blockIdx.x - 1, sh.blocks, reinterpret_cast<float*>(s_hist));
    return;
  }
  const int e = threadIdx.x, lane = e & (kWave - 1), w = e / kWave;
  const int seg = (A + kSegs - 1) / kSegs;  // assignments per segment
  for (int i = e; i < kSegs * E; i += 1024) s_hist[i] = 0;
  for (int i = e; i < A; i += 1024) s_idx[i] = topk_idx[i];
  __syncthreads();
  for (int i = e; i < A; i += 1024) atomicAdd(&s_hist[(i / seg) * E + s_idx[i]], 1);
  __syncthreads();
  // expert e: exclusive prefix over segments, in place, and its count
  int c = 0;
  if (e < E) {
#pragma unroll
    for (int q = 0; q < kSegs; ++q) {
      const int v = s_hist[q * E + e];
      s_hist[q * E + e] = c;
      c += v;
    }
  }
  const int a = c > 0 ? 1 : 0;
  const int tl = (c + kGroupBM - 1) / kGroupBM;
  const int np = (c + kStreamMaxMT - 1) / kStreamMaxMT;
  // block-wide inclusive scans of (c, a, tl, np) over experts: per wave, then
  // the totals of the waves before
  int ic = wave_incl_scan(c, lane), ia = wave_incl_scan(a, lane);
  int it = wave_incl_scan(tl, lane), ip = wave_incl_scan(np, lane);
  if (lane == kWave - 1) {
    s_wsum[w][0] = ic;
    s_wsum[w][1] = ia;
    s_wsum[w][2] = it;
    s_wsum[w][3] = ip;
  }
  __syncthreads();
  for (int q = 0; q < w; ++q) {
    ic += s_wsum[q][0];
    ia += s_wsum[q][1];
    it += s_wsum[q][2];
    ip += s_wsum[q][3];
  }
  s_off[e] = ic - c;
  if (e < E) {
    counts[e] = c;
    offsets[e] = ic - c;
    if (a) {
      active[ia - 1] = e;
      pass_base[ia - 1] = ip - np;
    }
    const int t0 = it - tl;
    for (int i = 0; i < tl; ++i) mtiles[t0 + i] = make_int2(e, i * kGroupBM);
  }
  if (e == E - 1) {
    offsets[E] = ic;
    hdr->n_active = ia;
    hdr->n_mtiles = it;
    hdr->n_passes = ip;
    pass_base[ia] = ip;
  }
  __syncthreads();
  for (int i = e; i < A; i += 1024) {
    const int x = s_idx[i];
    const int q = i / seg;
    int rank = s_hist[q * E + x];
    for (int j = q * seg; j < i; ++j) rank += s_idx[j] == x;
    const int row = s_off[x] + rank;
    perm_token[row] = i / k;
    row_of[i] = row;
  }
}

hipError_t launch_route_small(const int32_t* topk_idx, int64_t T, int E, int k, int32_t* counts,
                              int32_t* offsets, RouteHeader* hdr, int32_t* active, int2* mtiles,
                              int32_t* pass_base, int32_t* perm_token, int32_t* row_of,
                              const SharedSmall& sh, hipStream_t s) {
  const int64_t A = T * k;
  if (A > kRouteSmallMax || E > 1024) return hipErrorInvalidValue;
  if (!shared_small_ok(sh) || (sh.T > 0 && sh.T != T)) return hipErrorInvalidValue;
  const unsigned grid = 1u + (sh.T > 0 ? (unsigned)sh.blocks : 0u);
  const size_t lds = sh.T > 0 ? kSharedSmallLdsHold - 64 * 1024 : 0;  // beside its ~78 KB
  route_small_kernel<<<grid, 1024, lds, s>>>(topk_idx, (int)A, E, k, counts, offsets, hdr, active,
                                           mtiles, pass_base, perm_token, row_of, sh);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Permutation, step 1: per expert, exclusive prefix of the chunk histograms over
// chunks (in place) and the expert's total.  One wavefront per expert.
__global__ __launch_bounds__(256) void scan_chunks_kernel(int32_t* __restrict__ chunk_cnt,
                                                          int nchunks, int E,
                                                          int32_t* __restrict__ counts) {
  const int lane = threadIdx.x & (kWave - 1);
  const int e = blockIdx.x * 4 + threadIdx.x / kWave;
  if (e >= E) return;
  int carry = 0;
  for (int c0 = 0; c0 < nchunks; c0 += kWave) {
    const int c = c0 + lane;
    const int v = c < nchunks ? chunk_cnt[(int64_t)c * E + e] : 0;
    int incl = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int o = __shfl_up(incl, off, kWave);
      if (lane >= off) incl += o;
    }
    if (c < nchunks) chunk_cnt[(int64_t)c * E + e] = carry + incl - v;
    carry += __shfl(incl, kWave - 1, kWave);
  }
  if (lane == 0) counts[e] = carry;
}

// Permutation, step 2 (one block): expert segment offsets (exclusive scan of the
// counts), the compacted list of active experts, the M-tile work list, and the
// first streaming pass of each active expert.
__global__ __launch_bounds__(1024) void scan_experts_kernel(const int32_t* __restrict__ counts,
                                                            int E, int32_t* __restrict__ offsets,
                                                            RouteHeader* __restrict__ hdr,
                                                            int32_t* __restrict__ active,
                                                            int2* __restrict__ mtiles,
                                                            int32_t* __restrict__ pass_base) {
  __shared__ int s_cnt[1024], s_act[1024], s_til[1024], s_pas[1024];
  const int e = threadIdx.x;
  const int c = e < E ? counts[e] : 0;
  const int a = c > 0 ? 1 : 0;
  const int tl = (c + kGroupBM - 1) / kGroupBM;
  const int np = (c + kStreamMaxMT - 1) / kStreamMaxMT;
  s_cnt[e] = c;
  s_act[e] = a;
  s_til[e] = tl;
  s_pas[e] = np;
  for (int off = 1; off < 1024; off <<= 1) {
    __syncthreads();
    const int pc = e >= off ? s_cnt[e - off] : 0;
    const int pa = e >= off ? s_act[e - off] : 0;
    const int pt = e >= off ? s_til[e - off] : 0;
    const int pp = e >= off ? s_pas[e - off] : 0;
    __syncthreads();
    s_cnt[e] += pc;
    s_act[e] += pa;
    s_til[e] += pt;
    s_pas[e] += pp;
  }
  __syncthreads();
  if (e < E) {
    offsets[e] = s_cnt[e] - c;
    if (a) {
      active[s_act[e] - 1] = e;
      pass_base[s_act[e] - 1] = s_pas[e] - np;
    }
    const int t0 = s_til[e] - tl;
    for (int i = 0; i < tl; ++i) mtiles[t0 + i] = make_int2(e, i * kGroupBM);
  }
  if (e == E - 1) {
    offsets[E] = s_cnt[e];
    hdr->n_active = s_act[e];
    hdr->n_mtiles = s_til[e];
    hdr->n_passes = s_pas[e];
    pass_base[s_act[e]] = s_pas[e];
  }
}

hipError_t launch_scan(int32_t* chunk_cnt, int nchunks, int E, int32_t* counts, int32_t* offsets,
                       RouteHeader* hdr, int32_t* active, int2* mtiles, int32_t* pass_base,
                       hipStream_t s) {
  scan_chunks_kernel<<<dim3((E + 3) / 4), 256, 0, s>>>(chunk_cnt, nchunks, E, counts);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  scan_experts_kernel<<<1, 1024, 0, s>>>(counts, E, offsets, hdr, active, mtiles, pass_base);
  return hipGetLastError();
}

// Permutation, step 3: stable scatter.  One block per chunk, one thread per
// expert: the assignments of the chunk that chose expert e get consecutive rows
// of e's segment in (token, j) order.
__global__ __launch_bounds__(256) void scatter_kernel(const int32_t* __restrict__ topk_idx,
                                                      const int32_t* __restrict__ chunk_base,
                                                      const int32_t* __restrict__ offsets,
                                                      int64_t T, int E, int k,
                                                      int32_t* __restrict__ perm_token,
                                                      int32_t* __restrict__ row_of) {
  __shared__ int s_idx[kChunkTokens * 16];
  scatter_chunk(topk_idx, chunk_base, offsets, T, E, k, perm_token, row_of, blockIdx.x, s_idx);
}

hipError_t launch_scatter(const int32_t* topk_idx, const int32_t* chunk_base,
                          const int32_t* offsets, int64_t T, int E, int k, int32_t* perm_token,
                          int32_t* row_of, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int64_t nchunks = (T + kChunkTokens - 1) / kChunkTokens;
  scatter_kernel<<<dim3((unsigned)nchunks), 256, 0, s>>>(topk_idx, chunk_base, offsets, T, E, k,
                                                         perm_token, row_of);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Shared expert: act[t][n] = D(silu(g) * u), g and u summed over the split-K
// partials of the fused [gate | up] product.
template <typename T>
__global__ __launch_bounds__(256) void swiglu_finalize_kernel(const float* __restrict__ part,
                                                              int splits, int64_t Tn, int Is,
                                                              T* __restrict__ act) {
  const int n4 = blockIdx.x * blockDim.x + threadIdx.x;  // group of 4 columns
  if (n4 * 4 >= Is) return;
  swiglu_vec<T>(part, splits, Tn, Is, act, blockIdx.y, n4);
}

hipError_t launch_swiglu_finalize(int dtype, const float* part, int splits, int64_t T, int Is,
                                  void* act, hipStream_t s) {
  if (T == 0 || Is == 0) return hipSuccess;
  dim3 grid((Is / 4 + 255) / 256, (unsigned)T);
  if (dtype == kBF16)
    swiglu_finalize_kernel<bf16><<<grid, 256, 0, s>>>(part, splits, T, Is, (bf16*)act);
  else
    swiglu_finalize_kernel<float><<<grid, 256, 0, s>>>(part, splits, T, Is, (float*)act);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Combine ("GLM-5 · Input features", excerpt block: the residual is the
// pre-norm input).  out[t] = D(x[t] + (shared[t] + sum_j w[t][j] * y[row_of[t][j]]))
// in fp32 with j ascending; one 16-byte vector per thread.
template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(const T* x, const float* __restrict__ sp,
                                                      int splits, const T* __restrict__ y,
                                                      const float* __restrict__ w,
                                                      const int32_t* __restrict__ row_of,
                                                      int64_t Tn, int d, int k, T* out) {
  constexpr int V = Elem<T>::kVec;
  const int c = (blockIdx.x * blockDim.x + threadIdx.x) * V;
  if (c >= d) return;
  combine_vec<T>(x, sp, splits, y, w, row_of, Tn, d, k, out, blockIdx.y, c);
}

hipError_t launch_combine(int dtype, const void* x, const float* shared_part, int splits,
                          const void* y, const float* topk_w, const int32_t* row_of, int64_t T,
                          int d, int k, void* out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int V = dtype == kBF16 ? 8 : 4;
  dim3 grid((d / V + 255) / 256, (unsigned)T);
  if (dtype == kBF16)
    combine_kernel<bf16><<<grid, 256, 0, s>>>((const bf16*)x, shared_part, splits,
                                               (const bf16*)y, topk_w, row_of, T, d, k,
                                               (bf16*)out);
  else
    combine_kernel<float><<<grid, 256, 0, s>>>((const float*)x, shared_part, splits,
                                                (const float*)y, topk_w, row_of, T, d, k,
                                                (float*)out);
  return hipGetLastError();
}

}  // namespace moe
