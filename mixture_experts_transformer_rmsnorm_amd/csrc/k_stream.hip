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
#include "dev_stream.h"
#include "kernels.h"

namespace moe {

template <typename T, int CL, bool GU>
__global__ __launch_bounds__(kStreamThreads) void stream_kernel(GroupArgs g, const T* __restrict__ A,
                                                                const T* __restrict__ Wall,
                                                                T* __restrict__ out,
                                                                int n_slices) {
  extern __shared__ float red[];
  const int u = blockIdx.x;
  const int ai = u / n_slices, slice = u % n_slices;
  if (ai >= g.hdr->n_active) return;
  stream_item<T, CL, GU>(g, A, Wall, out, g.active[ai], slice, red);
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
