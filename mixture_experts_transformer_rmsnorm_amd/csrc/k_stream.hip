// Weight-streaming grouped kernels for the routed experts (gfx950).
//
// For decode-sized batches each active expert holds a handful of tokens, so the
// expert matmuls are bound by reading the expert weights from HBM once.  The
// weights stay in their grouped layout ("nemo_automodel ... state_dict_adapter",
// Glm4MoeStateDictAdapter: gate_and_up_projs [E, d, 2I] and down_projs [E, I, d],
// both with the output dimension contiguous), so a lane reads 16 contiguous
// bytes of one weight row and the wavefront reads whole row segments; the few
// token activations are broadcast and the products are fp32 FMAs.
//
// Work unit: (active expert, column slice).  Inside a 256-thread block, CL
// lanes cover the slice's columns (16 bytes each) and the 256/CL row groups
// split the contraction dimension into contiguous ranges; the row-group partial
// sums are reduced through LDS in a fixed order, so results are bitwise
// reproducible.  gate_up slices pair gate columns [c, c+w) with up columns
// [I+c, I+c+w) so that silu(gate)*up is formed in the block
// ("GLM-5 · Input features", excerpt mlp: the SwiGLU form).
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

template <typename T, int CL, bool GU>
__global__ __launch_bounds__(kStreamThreads) void stream_kernel(GroupArgs g, const T* __restrict__ A,
                                                                const T* __restrict__ Wall,
                                                                T* __restrict__ out,
                                                                int n_slices) {
  extern __shared__ float red[];
  const int u = blockIdx.x;
  const int ai = u / n_slices, slice = u % n_slices;
  if (ai >= g.hdr->n_active) return;
  const int e = g.active[ai];
  const int seg = g.offsets[e], ne = g.counts[e];
  // gate_up: A = h [T, d], W = gate_up[e] [d, 2I], out = act [A, I]
  // down:    A = act [A, I], W = down[e] [I, d],  out = y [A, d]
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

template <typename T, int CL, bool GU>
static hipError_t launch_stream(const GroupArgs& g, const void* A, const void* W, void* out,
                                hipStream_t s) {
  using S = StreamShape<T, CL, GU>;
  const int width = GU ? g.I : g.d;
  const int n_slices = (width + S::SW - 1) / S::SW;
  const size_t lds = (size_t)S::RG * kStreamMaxMT * S::RED_COLS * sizeof(float);
  const int64_t blocks = (int64_t)g.E * n_slices;
  stream_kernel<T, CL, GU><<<dim3((unsigned)blocks), kStreamThreads, lds, s>>>(
      g, (const T*)A, (const T*)W, (T*)out, n_slices);
  return hipGetLastError();
}

hipError_t launch_stream_gate_up(int dtype, const GroupArgs& g, const void* h,
                                 const void* gate_up, void* act, hipStream_t s) {
  if (dtype == kBF16) return launch_stream<bf16, 32, true>(g, h, gate_up, act, s);
  return launch_stream<float, 32, true>(g, h, gate_up, act, s);
}

hipError_t launch_stream_down(int dtype, const GroupArgs& g, const void* act, const void* down,
                              void* y, hipStream_t s) {
  if (dtype == kBF16) return launch_stream<bf16, 64, false>(g, act, down, y, s);
  return launch_stream<float, 64, false>(g, act, down, y, s);
}

}  // namespace moe
