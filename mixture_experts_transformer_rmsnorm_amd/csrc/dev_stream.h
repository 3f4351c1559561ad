// Device code of the weight-streaming grouped expert matmuls (decode-sized
// batches), shared by the stand-alone kernels and the fused decode kernel.
#pragma once

#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kStreamThreads = 256;

template <typename T, int CL, bool GU>
struct StreamShape {
  static constexpr int V = Elem<T>::kVec;
  static constexpr int RG = kStreamThreads / CL;           // row groups
  static constexpr int SW = GU ? (CL / 2) * V : CL * V;    // output columns per slice
  static constexpr int RED_COLS = CL * V;                  // LDS columns per (rg, m)
};

// Columns of this lane: its 16-byte vector sits at `pos` of the slice's LDS row
// and at column `wcol` of the weight matrix; lanes past the output width idle.
template <typename T, int CL, bool GU>
__device__ __forceinline__ bool stream_lane(const GroupArgs& g, int n_out, int slice, int cl,
                                            int* pos, int* wcol) {
  using S = StreamShape<T, CL, GU>;
  if (GU) {
    const int half = cl / (CL / 2);
    const int j = (cl % (CL / 2)) * S::V;
    *pos = half * S::SW + j;
    *wcol = (half ? g.I : 0) + slice * S::SW + j;
    return slice * S::SW + j < g.I;
  }
  *pos = cl * S::V;
  *wcol = slice * S::SW + *pos;
  return *wcol < n_out;
}

// Sums over rows [kb, ke) of W: acc[m][c] += A[row m][k] * W[k][wcol + c].  Rows
// of A beyond mt repeat the last valid row (their sums are never stored).
template <typename T, int CL, bool GU, int MT>
__device__ __forceinline__ void stream_accumulate(const GroupArgs& g, const T* __restrict__ A,
                                                  int64_t lda, const T* __restrict__ W,
                                                  int64_t ldw, int wcol, int seg, int m0, int mt,
                                                  int kb, int ke,
                                                  float (&acc)[MT][Elem<T>::kVec]) {
  constexpr int V = Elem<T>::kVec;
  const T* arow[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int mm = m < mt ? m : mt - 1;
    const int64_t prow = seg + m0 + mm;
    const int64_t r = GU ? (int64_t)g.perm_token[prow] : prow;
    arow[m] = A + r * lda;
  }
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

// Writes a row group's sums to its LDS rows: red[(rg * MT + m) * RED_COLS + pos + c].
template <typename T, int CL, bool GU, int MT>
__device__ __forceinline__ void stream_to_lds(const float (&acc)[MT][Elem<T>::kVec], int rg,
                                              int pos, float* red) {
  using S = StreamShape<T, CL, GU>;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    float* dst = red + ((int64_t)rg * MT + m) * S::RED_COLS + pos;
#pragma unroll
    for (int c = 0; c < S::V; c += 4)
      *reinterpret_cast<float4*>(dst + c) = make_float4(acc[m][c], acc[m][c + 1], acc[m][c + 2],
                                                        acc[m][c + 3]);
  }
}

// Output phase of a slice: v = silu(gate) * up (gate_up) or the sum (down), from
// the per-column sums in LDS rows red[m * RED_COLS + ...] (row group 0's rows).
template <typename T, int CL, bool GU, int MT>
__device__ __forceinline__ void stream_store(const float* red, int width, int seg, int m0, int mt,
                                             int slice, T* __restrict__ out, int64_t ldo) {
  using S = StreamShape<T, CL, GU>;
  constexpr int SW = S::SW;
  for (int o = threadIdx.x; o < mt * SW; o += kStreamThreads) {
    const int m = o / SW, j = o % SW;
    const int col = slice * SW + j;
    if (col >= width) continue;
    const float* src = red + (int64_t)m * S::RED_COLS;
    const float v = GU ? silu(src[j]) * src[SW + j] : src[j];
    T* dst = out + (int64_t)(seg + m0 + m) * ldo + col;
    if constexpr (sizeof(T) == 2)
      reinterpret_cast<uint16_t*>(dst)[0] = (uint16_t)f32_to_bf16_bits(v);
    else
      reinterpret_cast<float*>(dst)[0] = v;
  }
}

// Adds the RG row groups' sums of each (m, column) in a fixed order, in place into
// row group 0's rows.  Each sum is read and written by one thread only.
template <typename T, int CL, bool GU, int MT>
__device__ __forceinline__ void stream_reduce_rg(float* red, int mt) {
  using S = StreamShape<T, CL, GU>;
  for (int o = threadIdx.x; o < mt * S::RED_COLS; o += kStreamThreads) {
    const int m = o / S::RED_COLS, j = o % S::RED_COLS;
    float v = 0.f;
#pragma unroll
    for (int q = 0; q < S::RG; ++q) v += red[((int64_t)q * MT + m) * S::RED_COLS + j];
    red[(int64_t)m * S::RED_COLS + j] = v;
  }
}

// One pass over the slice's weights for tokens [m0, m0 + mt) of the expert
// (mt <= MT), all K rows: the row groups split K into equal contiguous ranges.
template <typename T, int CL, bool GU, int MT>
__device__ __forceinline__ void stream_pass(const GroupArgs& g, const T* __restrict__ A,
                                            int64_t lda, const T* __restrict__ W, int64_t ldw,
                                            int K, int n_out, int seg, int m0, int mt, int slice,
                                            T* __restrict__ out, int64_t ldo, float* red) {
  using S = StreamShape<T, CL, GU>;
  const int tid = threadIdx.x, cl = tid % CL, rg = tid / CL;
  int pos, wcol;
  const bool lane_ok = stream_lane<T, CL, GU>(g, n_out, slice, cl, &pos, &wcol);
  float acc[MT][S::V];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int c = 0; c < S::V; ++c) acc[m][c] = 0.f;
  const int kc = K / S::RG;
  if (lane_ok)
    stream_accumulate<T, CL, GU, MT>(g, A, lda, W, ldw, wcol, seg, m0, mt, rg * kc, rg * kc + kc,
                                     acc);
  __syncthreads();  // the previous pass's output phase has finished reading red
  stream_to_lds<T, CL, GU, MT>(acc, rg, pos, red);
  __syncthreads();
  stream_reduce_rg<T, CL, GU, MT>(red, mt);
  __syncthreads();
  stream_store<T, CL, GU, MT>(red, GU ? g.I : n_out, seg, m0, mt, slice, out, ldo);
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
