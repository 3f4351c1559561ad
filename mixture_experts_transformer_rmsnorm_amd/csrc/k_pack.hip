// Layout conversion of expert weights between the HF checkpoint layout (per expert,
// nn.Linear [out, in]: gate_proj.weight [I, d], up_proj.weight [I, d],
// down_proj.weight [d, I]) and the grouped layout of Glm4MoeStateDictAdapter
// (page "nemo_automodel.components.models.glm4_moe.state_dict_adapter",
// class documentation: gate_and_up_projs
// [E, d, 2I] with the gate columns first, down_projs [E, I, d]).  Pure data
// movement: every conversion is a set of matrix transposes, bits copied as they are.
//
// transpose_kernel: dst[c][r] = src[r][c] for an R x C matrix (rows ld_src / ld_dst
// elements apart), in 64 x 64 tiles through LDS.  A block of 256 threads reads
// the tile's 64 rows as 16-byte vectors (coalesced), writes them to an LDS tile
// whose rows are 66 elements apart (the 2-byte reads of one column by 64 lanes
// then fall in distinct banks or share a dword), and writes the transposed tile
// as 16-byte vectors of 8 (bf16) or 4 (fp32) consecutive source rows.  Up to three
// matrices of equal element count go in one launch (blockIdx.y picks one).
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kTT = 64;       // tile edge
constexpr int kTLd = kTT + 2;  // LDS row stride (elements)

template <typename E>  // uint16_t (bf16 bits) or uint32_t (fp32 bits)
__global__ __launch_bounds__(256) void transpose_kernel(TransposeBatch b) {
  constexpr int V = 16 / sizeof(E);         // elements per 16-byte vector
  constexpr int VPR = kTT / V;              // vectors per tile row
  constexpr int ITER = kTT * VPR / 256;     // vectors per thread
  __shared__ E tile[kTT * kTLd];
  const int m = blockIdx.y;
  const E* src = (const E*)b.src[m];
  E* dst = (E*)b.dst[m];
  const int R = b.rows[m], C = b.cols[m];
  const int tiles_c = C / kTT;
  const int tr = blockIdx.x / tiles_c, tc = blockIdx.x % tiles_c;
  if (tr * kTT >= R) return;
  const int64_t r0 = (int64_t)tr * kTT, c0 = (int64_t)tc * kTT;
  const int tid = threadIdx.x;
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int idx = tid + 256 * it;
    const int r = idx / VPR, v = idx % VPR;
    const uint4 q = ldg16(src + (r0 + r) * b.ld_src[m] + c0 + v * V);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    uint32_t* t32 = reinterpret_cast<uint32_t*>(tile + r * kTLd + v * V);  // 4-byte aligned
#pragma unroll
    for (int k = 0; k < 4; ++k) t32[k] = w[k];
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int idx = tid + 256 * it;
    const int c = idx / VPR, v = idx % VPR;  // output row c, source rows v*V .. v*V+V-1
    E e[V];
#pragma unroll
    for (int q = 0; q < V; ++q) e[q] = tile[(v * V + q) * kTLd + c];
    uint32_t w[4];
    if constexpr (sizeof(E) == 2) {
#pragma unroll
      for (int k = 0; k < 4; ++k) w[k] = (uint32_t)e[2 * k] | ((uint32_t)e[2 * k + 1] << 16);
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) w[k] = (uint32_t)e[k];
    }
    stg16(dst + (c0 + c) * b.ld_dst[m] + r0 + v * V, make_uint4(w[0], w[1], w[2], w[3]));
  }
}

hipError_t launch_transpose(int dtype, const TransposeBatch& b, hipStream_t s) {
  if (b.count == 0) return hipSuccess;
  const int64_t tiles = (int64_t)(b.rows[0] / kTT) * (b.cols[0] / kTT);
  dim3 grid((unsigned)tiles, (unsigned)b.count);
  if (dtype == kBF16)
    transpose_kernel<uint16_t><<<grid, 256, 0, s>>>(b);
  else
    transpose_kernel<uint32_t><<<grid, 256, 0, s>>>(b);
  return hipGetLastError();
}

}  // namespace moe
