// Measured ceilings for the roofline fractions, timed by the caller beside the datasheet
// figures: a loop of independent bf16 MFMAs over every SIMD of the chip (the dense bf16 matrix
// rate the chip sustains at its loaded clock) and a streaming read of a large buffer with
// 16-byte loads (the HBM read rate a bandwidth-bound kernel can reach).
#include "moe_internal.h"

namespace moe {

namespace {
constexpr int kChains = 8;  // independent accumulators per wave
}

// Every wave issues iters x kChains v_mfma_f32_32x32x16_bf16 (32 x 32 x 16 multiply-adds,
// 32768 flops each) on independent accumulators; the operands depend on the lane so nothing is
// folded, and the result is stored only if an impossible condition holds, so nothing is dropped.
__global__ __launch_bounds__(256) void k_mfma_loop(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  bf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (short)(0x3F80 + ((lane + i) & 7));  // bf16 values near 1
    b[i] = (short)(0x3C00 + ((lane * 3 + i) & 7));
  }
  f32x16_t acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = f32x16_t{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  if (s == -1.0f) sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

hipError_t launch_mfma_loop(int workgroups, int iters, float* sink, hipStream_t s) {
  hipLaunchKernelGGL(k_mfma_loop, dim3(workgroups), dim3(256), 0, s, iters, sink);
  return hipGetLastError();
}

double mfma_loop_flops(int workgroups, int iters) {
  return (double)workgroups * 4 * iters * kChains * 32.0 * 32.0 * 16.0 * 2.0;
}

// Every thread reads 16-byte pieces i = tid, tid + stride, ... of n16 pieces, four in flight.
__global__ __launch_bounds__(256) void k_stream_read(const uint4* __restrict__ p, size_t n16,
                                                      uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = p[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

hipError_t launch_stream_read(const void* p, size_t bytes, int workgroups, uint32_t* sink,
                              hipStream_t s) {
  hipLaunchKernelGGL(k_stream_read, dim3(workgroups), dim3(256), 0, s,
                     static_cast<const uint4*>(p), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace moe
