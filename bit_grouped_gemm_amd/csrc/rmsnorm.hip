// Residual update and RMSNorm between stacked MoE layers.
//
// "Perplexity's Lily: A Breakthrough Local Inference Engine Tailored Exclusively for Apple
// Silicon", section "The Model: Qwen3.6-35B-A3B in Focus": the model stacks 40 layers (10
// attention + 30 Gated DeltaNet), each followed by the MoE block; section "How It Works: Prefill
// and Decode Strategies": the next step's input is written into a GPU-resident slot with no CPU
// round trip. Between two MoE layers the fp32 residual stream takes the layer output and the
// next layer reads its RMS-normalised bf16 copy:
//   r <- r + y,   x <- bf16( r / sqrt(mean(r^2) + eps) )      (unit weight)
// (init 1: r <- x as fp32, then the same normalisation; init 2: r unchanged, normalisation only).
// One workgroup per token row; the row is read once, its sum of squares reduced in the
// workgroup, then written normalised.
#include "moe_internal.h"

namespace moe {

__global__ __launch_bounds__(256) void k_residual_rmsnorm(const float* __restrict__ y,
                                                          float* __restrict__ r,
                                                          uint16_t* __restrict__ x, int H,
                                                          float eps, int init) {
  __shared__ float part[4];
  const int t = blockIdx.x, tid = threadIdx.x;
  float* rr = r + (size_t)t * H;
  uint16_t* xx = x + (size_t)t * H;
  float ss = 0.0f;
  for (int i = 4 * tid; i < H; i += 1024) {
    float4 v;
    if (init == 1) {
      const uint2 b = *reinterpret_cast<const uint2*>(xx + i);
      v = make_float4(bf16_to_f32(b.x & 0xFFFFu), bf16_to_f32(b.x >> 16),
                      bf16_to_f32(b.y & 0xFFFFu), bf16_to_f32(b.y >> 16));
    } else if (init == 2) {
      v = *reinterpret_cast<const float4*>(rr + i);
    } else {
      const float4 a = *reinterpret_cast<const float4*>(rr + i);
      const float4 u = *reinterpret_cast<const float4*>(y + (size_t)t * H + i);
      v = make_float4(a.x + u.x, a.y + u.y, a.z + u.z, a.w + u.w);
    }
    if (init != 2) *reinterpret_cast<float4*>(rr + i) = v;
    ss = __builtin_fmaf(v.x, v.x, ss);
    ss = __builtin_fmaf(v.y, v.y, ss);
    ss = __builtin_fmaf(v.z, v.z, ss);
    ss = __builtin_fmaf(v.w, v.w, ss);
  }
  ss = wave_sum(ss);
  if ((tid & 63) == 0) part[tid >> 6] = ss;
  __syncthreads();
  const float tot = (part[0] + part[1]) + (part[2] + part[3]);
  const float den = sqrtf(tot / (float)H + eps);
  for (int i = 4 * tid; i < H; i += 1024) {
    const float4 v = *reinterpret_cast<const float4*>(rr + i);  // this thread's own stores
    uint2 o;
    o.x = pack_bf16x2(v.x / den, v.y / den);
    o.y = pack_bf16x2(v.z / den, v.w / den);
    *reinterpret_cast<uint2*>(xx + i) = o;
  }
}

hipError_t launch_residual_rmsnorm(const float* y, float* r, uint16_t* x, int T, int H, float eps,
                                   int init, hipStream_t s) {
  hipLaunchKernelGGL(k_residual_rmsnorm, dim3(T), dim3(256), 0, s, y, r, x, H, eps, init);
  return hipGetLastError();
}

}  // namespace moe
