// Device code of the weight-streaming grouped expert matmuls (decode-sized
// batches), shared by the stand-alone kernels and the fused decode kernel.
#pragma once

#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kStreamThreads = 256;
constexpr int kStreamMaxMT = 8;  // tokens of one expert processed per pass over its weights

template <typename T, int CL, bool GU>
struct StreamShape {
  static constexpr int V = Elem<T>::kVec;
  static constexpr int RG = kStreamThreads / CL;           // row groups
  static constexpr int SW = GU ? (CL / 2) * V : CL * V;    // output columns per slice
  static constexpr int RED_COLS = CL * V;                  // LDS columns per (rg, m)
};

// One pass over the slice's weights for tokens [m0, m0 + mt) of the expert
// (mt <= MT).  Rows beyond mt repeat the last valid row and are never stored.
template <typename T, int CL, bool GU, int MT>
__device__ __forceinline__ void stream_pass(const GroupArgs& g, const T* __restrict__ A,
                                            int64_t lda, const T* __restrict__ W, int64_t ldw,
                                            int K, int n_out, int seg, int m0, int mt, int slice,
                                            T* __restrict__ out, int64_t ldo, float* red) {
  using S = StreamShape<T, CL, GU>;
  constexpr int V = S::V, RG = S::RG, SW = S::SW;
  const int tid = threadIdx.x, cl = tid % CL, rg = tid / CL;

  int pos, wcol;
  bool lane_ok;
  if (GU) {
    const int half = cl / (CL / 2);
    const int j = (cl % (CL / 2)) * V;
    pos = half * SW + j;
    wcol = (half ? g.I : 0) + slice * SW + j;
    lane_ok = slice * SW + j < g.I;
  } else {
    pos = cl * V;
    wcol = slice * SW + pos;
    lane_ok = wcol < n_out;
  }

  const T* arow[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int mm = m < mt ? m : mt - 1;
    const int64_t prow = seg + m0 + mm;
    const int64_t r = GU ? (int64_t)g.perm_token[prow] : prow;
    arow[m] = A + r * lda;
  }

  float acc[MT][V];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int c = 0; c < V; ++c) acc[m][c] = 0.f;

  const int kc = K / RG;
  const int kb = rg * kc, ke = kb + kc;
  if (lane_ok) {
    const T* wp = W + (int64_t)kb * ldw + wcol;
    for (int k = kb; k < ke; k += V, wp += (int64_t)V * ldw) {
      uint4 wv[V];
#pragma unroll
      for (int r = 0; r < V; ++r) wv[r] = ldg16_stream(wp + (int64_t)r * ldw);
      float a[MT][V];
#pragma unroll
      for (int m = 0; m < MT; ++m) Elem<T>::unpack(ldg16(arow[m] + k), a[m]);
#pragma unroll
      for (int r = 0; r < V; ++r) {
        float f[V];
        Elem<T>::unpack(wv[r], f);
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int c = 0; c < V; ++c) acc[m][c] += a[m][r] * f[c];
      }
    }
  }

  __syncthreads();  // the previous pass's output phase has finished reading red
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    float* dst = red + ((int64_t)rg * MT + m) * S::RED_COLS + pos;
#pragma unroll
    for (int c = 0; c < V; c += 4)
      *reinterpret_cast<float4*>(dst + c) = make_float4(acc[m][c], acc[m][c + 1], acc[m][c + 2],
                                                        acc[m][c + 3]);
  }
  __syncthreads();

  const int width = GU ? g.I : n_out;
  for (int o = tid; o < mt * SW; o += kStreamThreads) {
    const int m = o / SW, j = o % SW;
    const int col = slice * SW + j;
    if (col >= width) continue;
    float v;
    if (GU) {
      float gs = 0.f, us = 0.f;
#pragma unroll
      for (int q = 0; q < RG; ++q) {
        const float* src = red + ((int64_t)q * MT + m) * S::RED_COLS;
        gs += src[j];
        us += src[SW + j];
      }
      v = silu(gs) * us;
    } else {
      v = 0.f;
#pragma unroll
      for (int q = 0; q < RG; ++q) v += red[((int64_t)q * MT + m) * S::RED_COLS + j];
    }
    T* dst = out + (int64_t)(seg + m0 + m) * ldo + col;
    if constexpr (sizeof(T) == 2)
      reinterpret_cast<uint16_t*>(dst)[0] = (uint16_t)f32_to_bf16_bits(v);
    else
      reinterpret_cast<float*>(dst)[0] = v;
  }
}

// One work unit: expert e, column slice `slice`, every token routed to e (in
// passes of up to kStreamMaxMT tokens).  red: LDS of
// RG * kStreamMaxMT * RED_COLS floats.
// gate_up: A = h [T, d] (rows gathered by perm_token), W = gate_up[e] [d, 2I], out = act [A, I]
// down:    A = act [A, I],                            W = down[e] [I, d],  out = y [A, d]
template <typename T, int CL, bool GU>
__device__ __forceinline__ void stream_item(const GroupArgs& g, const T* __restrict__ A,
                                            const T* __restrict__ Wall, T* __restrict__ out,
                                            int e, int slice, float* red) {
  const int seg = g.offsets[e], ne = g.counts[e];
  const int K = GU ? g.d : g.I;
  const int64_t ldw = GU ? 2 * (int64_t)g.I : (int64_t)g.d;
  const int n_out = GU ? g.I : g.d;
  const T* W = Wall + (int64_t)e * K * ldw;
  const int64_t lda = K;
  const int64_t ldo = n_out;
  for (int m0 = 0; m0 < ne; m0 += kStreamMaxMT) {
    const int mt = min(kStreamMaxMT, ne - m0);
    if (mt == 1)
      stream_pass<T, CL, GU, 1>(g, A, lda, W, ldw, K, n_out, seg, m0, mt, slice, out, ldo, red);
    else if (mt == 2)
      stream_pass<T, CL, GU, 2>(g, A, lda, W, ldw, K, n_out, seg, m0, mt, slice, out, ldo, red);
    else if (mt <= 4)
      stream_pass<T, CL, GU, 4>(g, A, lda, W, ldw, K, n_out, seg, m0, mt, slice, out, ldo, red);
    else
      stream_pass<T, CL, GU, 8>(g, A, lda, W, ldw, K, n_out, seg, m0, mt, slice, out, ldo, red);
  }
}

// Column slices of one expert's output for a stream kernel of this shape.
template <typename T, int CL, bool GU>
__host__ __device__ inline int stream_slices(int I, int d) {
  constexpr int V = 16 / sizeof(T);
  constexpr int SW = GU ? (CL / 2) * V : CL * V;
  const int width = GU ? I : d;
  return (width + SW - 1) / SW;
}

}  // namespace moe
