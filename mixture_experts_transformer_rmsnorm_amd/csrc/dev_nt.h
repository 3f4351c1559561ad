// Device code of the register-staged dense K-contiguous MFMA product (one
// 128 x 128 output tile, fp32 partial sums over one K range), shared by the
// stand-alone kernel and the fused decode kernel.
#pragma once

#include "common.h"
#include "kernels.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kNtBM = kMfmaBM, kNtBN = kMfmaBN, kNtBK = kMfmaBK;
constexpr int kNtLDK = kNtBK + 8;  // K-contiguous LDS rows: 72 elements (144 bytes)
constexpr int kNtTileElems = kNtBM * kNtLDK;

// LDS of one tile: A and B, double buffered.
struct NtSmem {
  uint16_t As[2 * kNtTileElems];
  uint16_t Bs[2 * kNtTileElems];
};

// out_part[z][m][n] (fp32, [splits][M][N]) for the 128 x 128 tile (m_tile, n_tile) and
// K-tiles [z * k_tiles_per_split, ...) of a.  256 threads: four wavefronts in a 2 x 2
// arrangement, each owning 64 rows x 64 columns as 2 x 2 v_mfma_f32_32x32x16_bf16
// tiles.  A and B tiles are staged in LDS with K contiguous (row stride 72
// elements, so the 16-byte fragment reads of 16 consecutive rows hit distinct
// banks) and double buffered: the global loads of K-tile t+1 are in flight while
// tile t is multiplied.  Ends with a block barrier, so sm may be reused at once.
__device__ __forceinline__ void nt_tile_128(const NtArgs& a, int n_tile, int m_tile, int z,
                                            NtSmem& sm) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int m0 = m_tile * kNtBM;
  const int rows = min(kNtBM, a.M - m0);
  const int nkt = a.K / kNtBK;
  const int kt0 = z * a.k_tiles_per_split;
  const int kt1 = min(nkt, kt0 + a.k_tiles_per_split);
  const uint16_t* A = (const uint16_t*)a.A;
  const uint16_t* B1 = (const uint16_t*)a.B1;
  const uint16_t* B2 = (const uint16_t*)a.B2;
  // B-columns of wave column wn: [wn*32, +32) (f = 0) and [64 + wn*32, +32) (f = 1)
  auto b_local_col = [&](int f) { return f * 64 + wn * 32; };

  // per-thread global load assignments: A rows and B rows tid/8 + 32*i, 16-byte
  // chunk tid%8.  Rows past the tile's valid rows (and B rows past N) load a valid
  // row instead: they only feed outputs the epilogue never stores, and
  // unconditional loads keep the wait counts of the pipeline exact.
  const uint16_t* a_src[4];
  const uint16_t* b_src[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = min(tid / 8 + 32 * i, rows - 1);
    a_src[i] = A + (int64_t)(m0 + r) * a.lda + (tid % 8) * 8;
    const int n = n_tile * kNtBN + tid / 8 + 32 * i;
    const int nn = n < a.N ? n : 0;
    const uint16_t* row = nn < a.n_split ? B1 + (int64_t)nn * a.ldb
                                         : B2 + (int64_t)(nn - a.n_split) * a.ldb;
    b_src[i] = row + (tid % 8) * 8;
  }

  uint4 ra[4], rb[4];
  auto gload = [&](int kt) {
    const int k0 = kt * kNtBK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = ldg16(a_src[i] + k0);
      rb[i] = ldg16(b_src[i] + k0);
    }
  };
  auto lstore = [&](int buf) {
    uint16_t* as = sm.As + buf * kNtTileElems;
    uint16_t* bs = sm.Bs + buf * kNtTileElems;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<uint4*>(as + (tid / 8 + 32 * i) * kNtLDK + (tid % 8) * 8) = ra[i];
      *reinterpret_cast<uint4*>(bs + (tid / 8 + 32 * i) * kNtLDK + (tid % 8) * 8) = rb[i];
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
      const uint16_t* as = sm.As + buf * kNtTileElems;
      const uint16_t* bs = sm.Bs + buf * kNtTileElems;
#pragma unroll
      for (int ks = 0; ks < kNtBK / 16; ++ks) {
        const int kof = ks * 16 + (lane >> 5) * 8;
        bf16x8_t af[2], bf[2];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
          af[mi] = *reinterpret_cast<const bf16x8_t*>(as + (wm * 64 + mi * 32 + (lane & 31)) * kNtLDK + kof);
#pragma unroll
        for (int f = 0; f < 2; ++f)
          bf[f] = *reinterpret_cast<const bf16x8_t*>(bs + (b_local_col(f) + (lane & 31)) * kNtLDK + kof);
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

  // in a 32x32 tile, accumulator element i of lane l is row 8*(i/4) + 4*(l/32) + i%4,
  // column l%32
  const int col32 = lane & 31;
  float* out = a.out + (int64_t)z * a.M * a.N;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const int n = n_tile * kNtBN + b_local_col(f) + col32;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = wm * 64 + mi * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
        if (r < rows && n < a.N) out[(int64_t)(m0 + r) * a.N + n] = acc[mi][f][i];
      }
    }
}

}  // namespace moe
