// Weighted combine of the grouped expert outputs, and the dequantisation test export.
//
// The combine forms y[t] = sum_k p[t,k] * Y[slot_pos[t*K+k]] + sigmoid_gate[t] * Y_shared[t]
// from the fp32 expert outputs Y, in fp32
// ("Perplexity's Lily: A Breakthrough Local Inference Engine Tailored Exclusively for Apple
// Silicon", section "The Model: Qwen3.6-35B-A3B in Focus": eight routed experts plus one shared
// expert per token). Terms are added in rank order, then the shared term: deterministic.
#include "moe_internal.h"

namespace moe {

__device__ __forceinline__ void fma4(float4& acc, float w, const float4& v) {
  acc.x = __builtin_fmaf(w, v.x, acc.x);
  acc.y = __builtin_fmaf(w, v.y, acc.y);
  acc.z = __builtin_fmaf(w, v.z, acc.z);
  acc.w = __builtin_fmaf(w, v.w, acc.w);
}

// One workgroup per token; a thread takes 4 consecutive columns (one 16-byte piece of each
// expert-output row), all K rows requested before the first is used.
template <int KC>
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ y_perm,
                                                 const int32_t* __restrict__ slot_pos,
                                                 const float* __restrict__ topk_w,
                                                 const float* __restrict__ shared_y,
                                                 const float* __restrict__ sgate, int H, int K,
                                                 float* __restrict__ out) {
  const int t = blockIdx.x;
  const int h4n = H >> 2;
  for (int h4 = threadIdx.x; h4 < h4n; h4 += 256) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k0 = 0; k0 < K; k0 += KC) {
      float4 v[KC];
      float w[KC];
#pragma unroll
      for (int j = 0; j < KC; ++j) {
        const int k = k0 + j < K ? k0 + j : K - 1;  // past K: re-read the last row, weight 0
        const int s = t * K + k;
        v[j] = reinterpret_cast<const float4*>(y_perm + (size_t)slot_pos[s] * H)[h4];
        w[j] = k0 + j < K ? topk_w[s] : 0.0f;
      }
#pragma unroll
      for (int j = 0; j < KC; ++j)
        if (k0 + j < K) fma4(acc, w[j], v[j]);
    }
    if (shared_y != nullptr)
      fma4(acc, sgate[t], reinterpret_cast<const float4*>(shared_y + (size_t)t * H)[h4]);
    reinterpret_cast<float4*>(out + (size_t)t * H)[h4] = acc;
  }
}

hipError_t launch_combine(const float* y_perm, const int32_t* slot_pos, const float* topk_w,
                          const float* shared_y, const float* sgate, const Dims& d, float* out,
                          hipStream_t s) {
  hipLaunchKernelGGL(k_combine<8>, dim3(d.T), dim3(256), 0, s, y_perm, slot_pos, topk_w,
                     shared_y, sgate, d.H, d.K, out);
  return hipGetLastError();
}

// One row of a packed projection through the same dequant8 used by the GEMM kernels.
__global__ void k_debug_dequant(const uint32_t* __restrict__ q, const uint16_t* __restrict__ sc,
                                const uint16_t* __restrict__ bi, size_t row, int kin,
                                float* __restrict__ out_f32, uint16_t* __restrict__ out_bf16) {
  const int w = blockIdx.x * blockDim.x + threadIdx.x;
  if (w >= (kin >> 3)) return;
  const uint32_t word = q[row * (kin >> 3) + w];
  const size_t g = row * (kin >> 6) + (w >> 3);
  const float s = bf16_to_f32(sc[g]), b = bf16_to_f32(bi[g]);
  if (out_f32) {
    float f[8];
    dequant8_f32(word, s, b, f);
#pragma unroll
    for (int i = 0; i < 8; ++i) out_f32[8 * w + i] = f[i];
  }
  if (out_bf16) {
    uint32_t o[4];
    dequant8(word, s, b, o);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out_bf16[8 * w + 2 * i] = (uint16_t)(o[i] & 0xFFFFu);
      out_bf16[8 * w + 2 * i + 1] = (uint16_t)(o[i] >> 16);
    }
  }
}

hipError_t launch_debug_dequant(const moe_w4_t& w, int n_rows, int kin, int mat, int row,
                                float* out_f32, uint16_t* out_bf16, hipStream_t s) {
  const size_t r = (size_t)mat * n_rows + row;
  const int words = kin >> 3;
  hipLaunchKernelGGL(k_debug_dequant, dim3((words + 255) / 256), dim3(256), 0, s, w.q, w.scale,
                     w.bias, r, kin, out_f32, out_bf16);
  return hipGetLastError();
}

}  // namespace moe
