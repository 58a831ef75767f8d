// Weighted combine of the grouped expert outputs, and the dequantisation test export.
//
// The combine forms y[t] = sum_k p[t,k] * Y[slot_pos[t*K+k]] + sigmoid_gate[t] * Y_shared[t]
// from the bf16 expert outputs Y, in fp32
// ("Perplexity's Lily: A Breakthrough Local Inference Engine Tailored Exclusively for Apple
// Silicon", section "The Model: Qwen3.6-35B-A3B in Focus": eight routed experts plus one shared
// expert per token). Terms are added in rank order, then the shared term: deterministic.
#include "moe_internal.h"

namespace moe {

// acc[j] += w * (element j of the 8 packed bf16 values in v)
__device__ __forceinline__ void add_bf16x8(float (&acc)[8], float w, const uint4& v) {
  const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc[2 * i] = __builtin_fmaf(w, bf16_to_f32(u[i] & 0xFFFFu), acc[2 * i]);
    acc[2 * i + 1] = __builtin_fmaf(w, bf16_to_f32(u[i] >> 16), acc[2 * i + 1]);
  }
}

// One workgroup per token; a thread takes 8 consecutive columns, one 16-byte piece of each
// bf16 expert-output row.
__global__ __launch_bounds__(256) void k_combine(const uint16_t* __restrict__ y_perm,
                                                 const int32_t* __restrict__ slot_pos,
                                                 const float* __restrict__ topk_w,
                                                 const uint16_t* __restrict__ shared_y,
                                                 const float* __restrict__ sgate, int H, int K,
                                                 float* __restrict__ out) {
  const int t = blockIdx.x;
  const int h8n = H >> 3;
  for (int h8 = threadIdx.x; h8 < h8n; h8 += 256) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int k = 0; k < K; ++k) {
      const int s = t * K + k;
      const uint4 v = reinterpret_cast<const uint4*>(y_perm + (size_t)slot_pos[s] * H)[h8];
      add_bf16x8(acc, topk_w[s], v);
    }
    if (shared_y != nullptr)
      add_bf16x8(acc, sgate[t], reinterpret_cast<const uint4*>(shared_y + (size_t)t * H)[h8]);
    float4* o = reinterpret_cast<float4*>(out + (size_t)t * H) + 2 * h8;
    o[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    o[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
}

hipError_t launch_combine(const uint16_t* y_perm, const int32_t* slot_pos, const float* topk_w,
                          const uint16_t* shared_y, const float* sgate, const Dims& d, float* out,
                          hipStream_t s) {
  hipLaunchKernelGGL(k_combine, dim3(d.T), dim3(256), 0, s, y_perm, slot_pos, topk_w, shared_y,
                     sgate, d.H, d.K, out);
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
