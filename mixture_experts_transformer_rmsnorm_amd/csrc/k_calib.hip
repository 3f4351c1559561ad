// Measurement kernels: the attainable peaks that the sublayer's kernels are
// compared with beside MI355X's published figures.
//
// calib_read_kernel: the HBM read ceiling.  Each of the launch's blocks (one per
// compute unit, 1024 lanes) reads an equal contiguous share of the buffer with
// 16-byte nontemporal loads, 4 independent loads per lane in flight per step --
// the access pattern of the decode weight streams at its best.
//
// calib_mfma_kernel: the matrix-core ceiling.  Every wave runs chains of
// v_mfma_f32_32x32x16_bf16 on register operands, four independent accumulators
// per wave so that each MFMA's latency hides behind the other three, two waves
// per SIMD.  No memory traffic.
#include "common.h"
#include "dev_nt.h"
#include "kernels.h"

namespace moe {

constexpr int kCalibReadThreads = 1024;
constexpr int kCalibMfmaThreads = 512;

__global__ __launch_bounds__(kCalibReadThreads) void calib_read_kernel(const uint4* src, int64_t n16,
                                                                       uint32_t* sink) {
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t b0 = (int64_t)blockIdx.x * per, b1 = min(n16, b0 + per);
  uint32_t x = 0;
  int64_t i = b0 + threadIdx.x;
  for (; i + 3 * kCalibReadThreads < b1; i += 4 * kCalibReadThreads) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = ldg16_stream(src + i + u * kCalibReadThreads);
#pragma unroll
    for (int u = 0; u < 4; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < b1; i += kCalibReadThreads) {
    const uint4 v = ldg16_stream(src + i);
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (x == 0x9e3779b9u) sink[0] = x;  // keeps the loads; almost never taken
}

__global__ __launch_bounds__(kCalibMfmaThreads) void calib_mfma_kernel(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  bf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)(lane + i));
    b[i] = (__bf16)(0.002f * (float)(lane - i));
  }
  f32x16_t acc[4] = {f32x16_t{}, f32x16_t{}, f32x16_t{}, f32x16_t{}};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  if (s == 12345.678f) sink[0] = s;  // keeps the MFMAs; almost never taken
}

hipError_t launch_calib_read(const void* src, size_t bytes, int blocks, uint32_t* sink,
                             hipStream_t s) {
  calib_read_kernel<<<dim3((unsigned)blocks), kCalibReadThreads, 0, s>>>(
      (const uint4*)src, (int64_t)(bytes / 16), sink);
  return hipGetLastError();
}

hipError_t launch_calib_mfma(int iters, int blocks, float* sink, double* flops, hipStream_t s) {
  calib_mfma_kernel<<<dim3((unsigned)blocks), kCalibMfmaThreads, 0, s>>>(iters, sink);
  // per wave and iteration: 4 MFMAs of 2 * 32 * 32 * 16 FLOP
  *flops = (double)blocks * (kCalibMfmaThreads / 64) * (double)iters * 4.0 * 2.0 * 32 * 32 * 16;
  return hipGetLastError();
}

}  // namespace moe
