// Device code of the small kernels (RMSNorm, router top-k, scatter, shared-expert
// SwiGLU, combine), shared by the stand-alone kernels and the fused decode kernel.
// The design notes are with the kernels in k_small.hip.
#pragma once

#include <math.h>

#include "common.h"
#include "kernels.h"

namespace moe {

__device__ __forceinline__ float rms_scale(double sum_sq, int d, float eps) {
  const float ms = (float)(sum_sq / (double)d);
  const float sq = (float)sqrt((double)(ms + eps));
  return (float)(1.0 / (double)sq);
}

template <typename T>
__device__ __forceinline__ double sum_sq(const uint4& v) {
  constexpr int V = Elem<T>::kVec;
  float f[V];
  Elem<T>::unpack(v, f);
  double ss = 0.0;
#pragma unroll
  for (int q = 0; q < V; ++q) ss += (double)f[q] * (double)f[q];
  return ss;
}

template <typename T>
__device__ __forceinline__ uint4 rms_vec(const uint4& xv, const T* w, int i, float r) {
  constexpr int V = Elem<T>::kVec;
  float f[V], g[V];
  Elem<T>::unpack(xv, f);
  Elem<T>::unpack(ldg16(w + (int64_t)i * V), g);
#pragma unroll
  for (int q = 0; q < V; ++q) f[q] = Elem<T>::round(g[q] * Elem<T>::round(f[q] * r));
  return Elem<T>::pack(f);
}

// One row handled by `step` threads starting at vector i0.  The first NV vectors of
// each thread stay in registers between the sum of squares and the scaling, so a
// row of up to NV * step vectors is read from memory once; longer rows read the
// rest again.  The partial sum of squares goes through `reduce`.
template <typename T, int NV, typename Reduce>
__device__ __forceinline__ void rms_row(const T* xr, const T* w, T* hr, int nvec, int i0, int step,
                                        int d, float eps, Reduce reduce) {
  constexpr int V = Elem<T>::kVec;
  uint4 xv[NV];
  double ss = 0.0;
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const int i = i0 + u * step;
    if (i < nvec) {
      xv[u] = ldg16(xr + (int64_t)i * V);
      ss += sum_sq<T>(xv[u]);
    }
  }
  for (int i = i0 + NV * step; i < nvec; i += step) ss += sum_sq<T>(ldg16(xr + (int64_t)i * V));
  const float r = rms_scale(reduce(ss), d, eps);
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const int i = i0 + u * step;
    if (i < nvec) stg16(hr + (int64_t)i * V, rms_vec(xv[u], w, i, r));
  }
  for (int i = i0 + NV * step; i < nvec; i += step)
    stg16(hr + (int64_t)i * V, rms_vec(ldg16(xr + (int64_t)i * V), w, i, r));
}

// One RMSNorm row by a whole block (blockDim.x threads); red: 4 doubles of LDS.
template <typename T>
__device__ __forceinline__ void rms_block_row(const T* xr, const T* __restrict__ w, T* hr, int d,
                                              float eps, double* red) {
  constexpr int V = Elem<T>::kVec;
  auto reduce = [&](double ss) {
    ss = wave_sum(ss);
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
    if (lane == 0) red[wid] = ss;
    __syncthreads();
    const double tot = red[0] + red[1] + red[2] + red[3];
    __syncthreads();  // red may be reused by the next row
    return tot;
  };
  rms_row<T, 4>(xr, w, hr, d / V, threadIdx.x, 256, d, eps, reduce);
}

// Selection for one token by one wavefront from its fp32 logits l[q] (expert
// lane + 64 q): score = sigmoid(logit); key = score + corr_bias decides; k
// rounds of a wave-wide arg-max over (key desc, expert asc); the weights are the
// selected unbiased scores renormalised to sum rs.  Lane j < k writes choice j of
// token t; lane 0 counts each choice in hist (LDS) when hist is not null.
template <int Q>
__device__ __forceinline__ void topk_select(const float (&l)[Q], const float* __restrict__ bias,
                                            int64_t t, int E, int k, float rs,
                                            int32_t* __restrict__ idx_out,
                                            float* __restrict__ w_out, int* hist) {
  const int lane = threadIdx.x & (kWave - 1);
  float key[Q], sc[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int e = lane + kWave * q;
    key[q] = -INFINITY;
    sc[q] = 0.f;
    if (e < E) {
      const float sg = 1.0f / (1.0f + expf(-l[q]));
      sc[q] = sg;
      key[q] = sg + bias[e];
    }
  }
  uint32_t taken = 0;
  float ssum = 0.f, my_s = 0.f;
  int my_e = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY, bs = 0.f;
    int be = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int e = lane + kWave * q;
      const bool ok = e < E && !((taken >> q) & 1u);
      if (ok && (key[q] > bv || (key[q] == bv && e < be))) {
        bv = key[q];
        be = e;
        bs = sc[q];
      }
    }
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off, kWave);
      const int oe = __shfl_xor(be, off, kWave);
      const float os = __shfl_xor(bs, off, kWave);
      if (ov > bv || (ov == bv && oe < be)) {
        bv = ov;
        be = oe;
        bs = os;
      }
    }
    if ((be & (kWave - 1)) == lane) taken |= 1u << (be / kWave);
    ssum += bs;
    if (lane == j) {
      my_s = bs;
      my_e = be;
    }
    if (hist && lane == 0) atomicAdd(&hist[be], 1);
  }
  if (lane < k) {
    idx_out[t * k + lane] = my_e;
    w_out[t * k + lane] = rs * my_s / ssum;
  }
}

template <int Q, int WAVES>
__device__ __forceinline__ void topk_chunk(const float* __restrict__ part, int splits,
                                           const float* __restrict__ bias, int64_t T, int E, int k,
                                           float rs, int32_t* __restrict__ idx_out,
                                           float* __restrict__ w_out, int32_t* __restrict__ chunk_cnt,
                                           int64_t chunk, int* hist) {
  for (int e = threadIdx.x; e < E; e += WAVES * 64) hist[e] = 0;
  __syncthreads();
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  const int64_t tbase = chunk * kChunkTokens;
  for (int tl = wid; tl < kChunkTokens; tl += WAVES) {
    const int64_t t = tbase + tl;
    if (t >= T) break;
    float l[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) l[q] = 0.f;
    const int64_t zstride = T * (int64_t)E;
    const float* pt = part + t * E + lane;
    int z = 0;
    for (; z + 4 <= splits; z += 4) {
      float v[4][Q];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int q = 0; q < Q; ++q)
          v[u][q] = (lane + kWave * q < E) ? pt[(z + u) * zstride + kWave * q] : 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int q = 0; q < Q; ++q) l[q] += v[u][q];
    }
    for (; z < splits; ++z)
#pragma unroll
      for (int q = 0; q < Q; ++q)
        if (lane + kWave * q < E) l[q] += pt[z * zstride + kWave * q];
    topk_select<Q>(l, bias, t, E, k, rs, idx_out, w_out, hist);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += WAVES * 64) chunk_cnt[chunk * E + e] = hist[e];
}

__device__ __forceinline__ void scatter_chunk(const int32_t* __restrict__ topk_idx,
                                              const int32_t* __restrict__ chunk_base,
                                              const int32_t* __restrict__ offsets, int64_t T, int E,
                                              int k, int32_t* __restrict__ perm_token,
                                              int32_t* __restrict__ row_of, int64_t chunk,
                                              int* s_idx) {
  const int64_t t0 = chunk * kChunkTokens;
  const int ntok = (int)min<int64_t>(kChunkTokens, T - t0);
  for (int i = threadIdx.x; i < ntok * k; i += blockDim.x) s_idx[i] = topk_idx[t0 * k + i];
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int row = offsets[e] + chunk_base[chunk * E + e];
    for (int i = 0; i < ntok * k; ++i) {
      if (s_idx[i] == e) {
        perm_token[row] = (int32_t)(t0 + i / k);
        row_of[t0 * k + i] = row;
        ++row;
      }
    }
  }
  __syncthreads();
}

// act[t][4*n4 .. +3] from the split partial sums of gate and up
template <typename T>
__device__ __forceinline__ void swiglu_vec(const float* __restrict__ part, int splits, int64_t Tn,
                                           int Is, T* __restrict__ act, int64_t t, int n4) {
  float g[4] = {0.f, 0.f, 0.f, 0.f}, u[4] = {0.f, 0.f, 0.f, 0.f};
  for (int z = 0; z < splits; ++z) {
    const float* p = part + ((int64_t)z * Tn + t) * (2 * (int64_t)Is);
    const float4 gv = *reinterpret_cast<const float4*>(p + n4 * 4);
    const float4 uv = *reinterpret_cast<const float4*>(p + Is + n4 * 4);
    g[0] += gv.x; g[1] += gv.y; g[2] += gv.z; g[3] += gv.w;
    u[0] += uv.x; u[1] += uv.y; u[2] += uv.z; u[3] += uv.w;
  }
  T* o = act + t * Is + n4 * 4;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float v = silu(g[q]) * u[q];
    if constexpr (sizeof(T) == 2)
      reinterpret_cast<uint16_t*>(o)[q] = (uint16_t)f32_to_bf16_bits(v);
    else
      reinterpret_cast<float*>(o)[q] = v;
  }
}

// out[t][c .. c+V) for one 16-byte vector.  The partial sums and the expert
// outputs are read once, with nontemporal loads (the combine step of a 4096-token
// batch runs 25 % faster than with plain loads).
template <typename T>
__device__ __forceinline__ void combine_vec(const T* x, const float* __restrict__ sp, int splits,
                                            const T* __restrict__ y, const float* __restrict__ w,
                                            const int32_t* __restrict__ row_of, int64_t Tn, int d,
                                            int k, T* out, int64_t t, int c) {
  constexpr int V = Elem<T>::kVec;
  float acc[V];
#pragma unroll
  for (int q = 0; q < V; ++q) acc[q] = 0.f;
  for (int z = 0; z < splits; ++z) {
    const float* p = sp + ((int64_t)z * Tn + t) * d + c;
#pragma unroll
    for (int q = 0; q < V; q += 4) {
      const uint4 v = ldg16_stream(p + q);
      acc[q] += __uint_as_float(v.x);
      acc[q + 1] += __uint_as_float(v.y);
      acc[q + 2] += __uint_as_float(v.z);
      acc[q + 3] += __uint_as_float(v.w);
    }
  }
  for (int j = 0; j < k; ++j) {
    const float wj = w[t * k + j];
    const int64_t r = row_of[t * k + j];
    float yv[V];
    Elem<T>::unpack(ldg16_stream(y + r * d + c), yv);
#pragma unroll
    for (int q = 0; q < V; ++q) acc[q] += wj * yv[q];
  }
  float xv[V];
  Elem<T>::unpack(ldg16(x + t * d + c), xv);
#pragma unroll
  for (int q = 0; q < V; ++q) xv[q] = xv[q] + acc[q];
  stg16(out + t * d + c, Elem<T>::pack(xv));
}

}  // namespace moe
