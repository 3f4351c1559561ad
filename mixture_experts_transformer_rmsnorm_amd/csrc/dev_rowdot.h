// The shared expert of a small batch (bf16), computed by extra blocks of the two
// one-block routing launches (selection, then the permutation), which otherwise
// leave all but a few compute units idle: the selection launch's extra blocks form
// act_s = silu(gate h) * up h, the permutation launch's extra blocks the shared
// output s = down act_s in fp32 ("GLM-5 · Input features", excerpt mlp: the SwiGLU
// form; the shared weights keep the nn.Linear layout [out, in], so every output is
// the dot product of one contiguous weight row with an activation row).
//
// A group of 256 lanes (4 waves) takes a batch of RB = 8 weight rows: lane g reads
// the 16-byte vectors g, g + 256, ... of every row (nontemporal; a wave reads 1 KiB
// of a row per load) and the same vectors of the MT <= 4 activation rows, and keeps
// the RB x MT products in fp32 (v_dot2c_f32_bf16 on element pairs).  A wave then
// adds its 64 lanes' values by recursive halving (after step s, lane l holds the
// sums of the values whose index agrees with l in the top s bits), and the four
// waves' sums meet in LDS.  The order of every sum is fixed by the shapes alone, so
// repeated calls give the same bits.
#pragma once

#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kRdLanes = 256;  // lanes of a group
constexpr int kRdGroupLds = kRdLanes + 64;  // floats of LDS per group

__device__ __forceinline__ float rd_dot2(uint32_t x, uint32_t y, float c) {
  typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, x), __builtin_bit_cast(v2bf, y),
                                         c, false);
}

// s[r * MT + t] = sum_k W_r[k] A_t[k] (fp32) for the rows wp[r] (null: no row) and
// the activation rows ap[t] (t < mt), each KV 16-byte vectors long, U vectors of
// each row in flight per lane.  gl: the lane's index in its group; lds: kRdGroupLds
// floats of the group's LDS, the sums land in lds[kRdLanes + r * MT + t].  Every
// lane of the block calls it the same number of times (it holds block barriers).
template <int RB, int MT, int U>
__device__ __forceinline__ void rowdot_batch(const bf16* const (&wp)[RB],
                                             const bf16* const (&ap)[MT], int mt, int KV, int gl,
                                             float* lds) {
  constexpr int NV = RB * MT;  // values per lane
  constexpr int LOGNV = NV == 4 ? 2 : NV == 8 ? 3 : NV == 16 ? 4 : NV == 32 ? 5 : 6;
  static_assert(NV == 1 << LOGNV && NV <= kWave, "a power of two, at most one per lane");
  float v[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) v[j] = 0.f;
#pragma unroll 1
  for (int v0 = gl; v0 < KV; v0 += kRdLanes * U) {
    uint4 w[RB][U], a[MT][U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int vi = v0 + u * kRdLanes;
      const bool ok = vi < KV;
      // a 32-bit byte offset from the rows' scalar base pointers
      const uint32_t off = (uint32_t)vi * 16u;
#pragma unroll
      for (int r = 0; r < RB; ++r)
        w[r][u] = ok && wp[r] ? ldg16_stream(reinterpret_cast<const char*>(wp[r]) + off)
                              : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int t = 0; t < MT; ++t)
        a[t][u] = ok && t < mt ? ldg16(reinterpret_cast<const char*>(ap[t]) + off)
                               : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          float c = v[r * MT + t];
          c = rd_dot2(w[r][u].x, a[t][u].x, c);
          c = rd_dot2(w[r][u].y, a[t][u].y, c);
          c = rd_dot2(w[r][u].z, a[t][u].z, c);
          c = rd_dot2(w[r][u].w, a[t][u].w, c);
          v[r * MT + t] = c;
        }
  }
  // recursive halving over the wave: at offset o the lanes with bit o set keep the
  // upper half of the values, the others the lower half, each plus its partner's.
  // Both halves are exchanged and the sums selected, so that no value is picked
  // by a lane-dependent index (which the compiler would turn into indexed
  // register access through memory).
  const int lane = gl & (kWave - 1);
#pragma unroll
  for (int s = 0; s < LOGNV; ++s) {
    const int h = NV >> (s + 1), o = (kWave / 2) >> s;
    const bool up = (lane & o) != 0;
#pragma unroll
    for (int q = 0; q < h; ++q) {
      const float lo = v[q] + __shfl_xor(v[q], o, kWave);
      const float hi = v[q + h] + __shfl_xor(v[q + h], o, kWave);
      v[q] = up ? hi : lo;
    }
  }
  // lane l now holds value j = l >> (6 - LOGNV), summed over the lanes that agree
  // with l in bits 6 - LOGNV and up; add the lanes that differ only below
#pragma unroll
  for (int o = (kWave >> LOGNV) / 2; o > 0; o >>= 1) v[0] += __shfl_xor(v[0], o, kWave);
  const int wv = gl / kWave;
  if ((lane & ((kWave >> LOGNV) - 1)) == 0) lds[wv * NV + (lane >> (6 - LOGNV))] = v[0];
  __syncthreads();
  if (gl < NV) lds[kRdLanes + gl] = ((lds[gl] + lds[NV + gl]) + lds[2 * NV + gl]) + lds[3 * NV + gl];
  __syncthreads();
}

// Columns [c0, c1) of act_s for the tokens of the batch: the gate and up rows of
// RB / 2 columns per row batch.
template <int RB, int MT, int U>
__device__ __forceinline__ void shared_gate_up_cols(const SharedSmall& sh, int c0, int c1, int gl,
                                                    float* lds) {
  constexpr int C = RB / 2;
  const bf16* ap[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) ap[t] = sh.h + (int64_t)(t < sh.T ? t : 0) * sh.d;
  const int KV = sh.d / 8;
#pragma unroll 1
  for (int c = c0; c < c1; c += C) {
    const bf16* wp[RB];
#pragma unroll
    for (int j = 0; j < C; ++j) {
      const bool ok = c + j < c1;
      wp[j] = ok ? sh.gate + (int64_t)(c + j) * sh.d : nullptr;
      wp[C + j] = ok ? sh.up + (int64_t)(c + j) * sh.d : nullptr;
    }
    rowdot_batch<RB, MT, U>(wp, ap, sh.T, KV, gl, lds);
    if (gl < C * MT) {
      const int j = gl / MT, t = gl % MT;
      if (c + j < c1 && t < sh.T) {
        const float g = lds[kRdLanes + j * MT + t], u = lds[kRdLanes + (C + j) * MT + t];
        sh.act_s[(int64_t)t * sh.Is + c + j].bits = (uint16_t)f32_to_bf16_bits(silu(g) * u);
      }
    }
    __syncthreads();  // lds is reused by the next batch
  }
}

// Rows [m0, m1) of the shared down weights (outputs m of s, fp32) in nb batches of
// RB rows (batches past m1 hold no rows).
template <int RB, int MT, int U>
__device__ __forceinline__ void shared_down_rows(const SharedSmall& sh, int m0, int m1, int nb,
                                                 int gl, float* lds) {
  const bf16* ap[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) ap[t] = sh.act_s + (int64_t)(t < sh.T ? t : 0) * sh.Is;
  const int KV = sh.Is / 8;
#pragma unroll 1
  for (int b = 0; b < nb; ++b) {
    const int m = m0 + b * RB;
    const bf16* wp[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r)
      wp[r] = m + r < m1 ? sh.down + (int64_t)(m + r) * sh.Is : nullptr;
    rowdot_batch<RB, MT, U>(wp, ap, sh.T, KV, gl, lds);
    if (gl < RB * MT) {
      const int r = gl / MT, t = gl % MT;
      if (m + r < m1 && t < sh.T) sh.y_s[(int64_t)t * sh.d + m + r] = lds[kRdLanes + gl];
    }
    __syncthreads();
  }
}

// Block `b` of `nb` extra blocks of 256 lanes (one wave per SIMD, registers for 3
// or 4 vectors of 8 rows in flight: at the GLM-5 width, d = 6144, every vector of
// the batch's rows at once): act_s columns [col0 + b n / nb, col0 + (b + 1) n / nb)
// of the launch's n = col1 - col0.
__device__ __forceinline__ void shared_gate_up_block(const SharedSmall& sh, int b, int nb,
                                                     float* lds) {
  const int n = sh.col1 - sh.col0;
  const int c0 = sh.col0 + (int)((int64_t)b * n / nb);
  const int c1 = sh.col0 + (int)((int64_t)(b + 1) * n / nb);
  const int gl = threadIdx.x;
  static_assert(kSharedSmallTokens <= 4, "token counts dispatched below");
  if (sh.T <= 1) shared_gate_up_cols<8, 1, 4>(sh, c0, c1, gl, lds);
  else if (sh.T <= 2) shared_gate_up_cols<8, 2, 4>(sh, c0, c1, gl, lds);
  else shared_gate_up_cols<8, 4, 3>(sh, c0, c1, gl, lds);
}

// Block `b` of `nb` extra blocks of G groups of 256 lanes (four waves per SIMD at
// G = 4, so at most 128 registers per lane: one vector of each of the 8 rows in
// flight, a whole row of the GLM-5 width Is = 2048 per group load): rows
// [b d / nb, (b + 1) d / nb) of the shared down weights, split evenly over the
// groups; every group runs the same number of batches (the block's barriers).
template <int G>
__device__ __forceinline__ void shared_down_block(const SharedSmall& sh, int b, int nb,
                                                  float* lds) {
  const int r0 = (int)((int64_t)b * sh.d / nb), r1 = (int)((int64_t)(b + 1) * sh.d / nb);
  const int per = (r1 - r0 + G - 1) / G;
  // the group index is the same in every lane of a wave: keep the row pointers scalar
  const int gi = __builtin_amdgcn_readfirstlane(threadIdx.x / kRdLanes), gl = threadIdx.x % kRdLanes;
  const int m0 = min(r1, r0 + gi * per), m1 = min(r1, m0 + per);
  float* glds = lds + gi * kRdGroupLds;
  if (sh.T <= 1) shared_down_rows<8, 1, 1>(sh, m0, m1, (per + 7) / 8, gl, glds);
  else if (sh.T <= 2) shared_down_rows<8, 2, 1>(sh, m0, m1, (per + 7) / 8, gl, glds);
  else shared_down_rows<8, 4, 1>(sh, m0, m1, (per + 7) / 8, gl, glds);
}

}  // namespace moe
