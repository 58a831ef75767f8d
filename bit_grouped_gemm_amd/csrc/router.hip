// Router: logits, top-k with softmax renormalisation, shared-expert sigmoid gate, counts.
//
// "Perplexity's Lily: A Breakthrough Local Inference Engine Tailored Exclusively for Apple
// Silicon", section "The Model: Qwen3.6-35B-A3B in Focus": a router scores 256 experts per
// token and selects eight; one shared expert processes every token.
//
// Prefill logits run on bf16 MFMA: x is exact in bf16 and each fp32 router weight is split
// into three bf16 parts w = hi + mid + lo (24 significant bits), so x.w is formed from exact
// bf16 products with fp32 accumulation -- the same accuracy as an fp32 dot product, at MFMA
// speed (the split follows Henry, Tang and Heinecke, "Leveraging the bfloat16 artificial
// intelligence datatype for higher-precision computations", ARITH 2019). Decode logits
// (few tokens, bandwidth-bound) use fp32 FMA directly on the fp32 weights.
#include "moe_internal.h"

namespace moe {

// ------------------------------------------------------------- weight split (prefill)
// parts[p][e][h], p = 0 (hi), 1 (mid), 2 (lo), each the bf16 rounding of the remainder.
__global__ void k_router_split(const float* __restrict__ w, int n, uint16_t* __restrict__ parts) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float v = w[i];
  const uint16_t hi = f32_to_bf16(v);
  const float r1 = v - bf16_to_f32(hi);  // exact
  const uint16_t mid = f32_to_bf16(r1);
  const float r2 = r1 - bf16_to_f32(mid);  // exact
  parts[i] = hi;
  parts[n + i] = mid;
  parts[2 * n + i] = f32_to_bf16(r2);
}

hipError_t launch_router_split(const float* w, int E, int H, uint16_t* parts, hipStream_t s) {
  const int n = E * H;
  hipLaunchKernelGGL(k_router_split, dim3((n + 255) / 256), dim3(256), 0, s, w, n, parts);
  return hipGetLastError();
}

// ------------------------------------------------------------ prefill logits (MFMA)
// WG = 4 waves = 64 tokens x 64 experts; each wave a 32x32 tile on v_mfma_f32_32x32x16_bf16.
// Lane l feeds row (l & 31) of its tile and the 8 inputs k0 + 8*(l >> 5) .. +7 for both
// operands (any consistent split of K between the operands gives the same dot products).
__global__ __launch_bounds__(256) void k_router_mfma(const uint16_t* __restrict__ x,
                                                     const uint16_t* __restrict__ parts,
                                                     const float* __restrict__ bias, int T,
                                                     int E, int H, float* __restrict__ logits) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.y * 64 + (wave >> 1) * 32;
  const int e0 = blockIdx.x * 64 + (wave & 1) * 32;
  if (t0 >= T || e0 >= E) return;  // no barriers in this kernel
  const int r = lane & 31, half = lane >> 5;
  const int trow = min(t0 + r, T - 1), erow = min(e0 + r, E - 1);
  const size_t plane = (size_t)E * H;
  const uint16_t* xa = x + (size_t)trow * H + half * 8;
  const uint16_t* pb = parts + (size_t)erow * H + half * 8;
  f32x16_t acc = {};
#pragma unroll 4
  for (int k = 0; k < H; k += 16) {
    const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(xa + k);
    const bf16x8_t bh = *reinterpret_cast<const bf16x8_t*>(pb + k);
    const bf16x8_t bm = *reinterpret_cast<const bf16x8_t*>(pb + plane + k);
    const bf16x8_t bl = *reinterpret_cast<const bf16x8_t*>(pb + 2 * plane + k);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bl, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bm, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bh, acc, 0, 0, 0);
  }
  // D layout of the 32x32 tile: register i of lane l is row 8*(i/4) + 4*(l/32) + i%4,
  // column l%32.
  const int e = e0 + r;
  if (e >= E) return;
  const float bv = bias ? bias[e] : 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int t = t0 + 8 * (i >> 2) + 4 * half + (i & 3);
    if (t < T) logits[(size_t)t * E + e] = acc[i] + bv;
  }
}

hipError_t launch_router_logits_mfma(const uint16_t* x, const uint16_t* parts, const float* bias,
                                     int T, int E, int H, float* logits, hipStream_t s) {
  dim3 grid((E + 63) / 64, (T + 63) / 64);
  hipLaunchKernelGGL(k_router_mfma, grid, dim3(256), 0, s, x, parts, bias, T, E, H, logits);
  return hipGetLastError();
}

// -------------------------------------------------------------- decode logits (GEMV)
// One wave per expert row; each lane reads 16 B of the fp32 row per step (coalesced) and
// the matching 4 inputs of every token. T <= kDecodeMaxT.
template <int TC>
__global__ __launch_bounds__(64) void k_router_gemv(const uint16_t* __restrict__ x,
                                                    const float* __restrict__ w,
                                                    const float* __restrict__ bias, int T, int E,
                                                    int H, float* __restrict__ logits) {
  const int e = blockIdx.x, lane = threadIdx.x;
  const float4* wr = reinterpret_cast<const float4*>(w + (size_t)e * H);
  float acc[TC];
#pragma unroll
  for (int t = 0; t < TC; ++t) acc[t] = 0.0f;
  const int units = H / 4;
  for (int u = lane; u < units; u += 64) {
    const float4 wv = wr[u];
#pragma unroll
    for (int t = 0; t < TC; ++t) {
      if (t < T) {
        const uint2 xv = *reinterpret_cast<const uint2*>(x + (size_t)t * H + 4 * u);
        acc[t] = __builtin_fmaf(bf16_to_f32(xv.x & 0xFFFFu), wv.x, acc[t]);
        acc[t] = __builtin_fmaf(bf16_to_f32(xv.x >> 16), wv.y, acc[t]);
        acc[t] = __builtin_fmaf(bf16_to_f32(xv.y & 0xFFFFu), wv.z, acc[t]);
        acc[t] = __builtin_fmaf(bf16_to_f32(xv.y >> 16), wv.w, acc[t]);
      }
    }
  }
  const float bv = bias ? bias[e] : 0.0f;
#pragma unroll
  for (int t = 0; t < TC; ++t) {
    if (t < T) {
      const float v = wave_sum(acc[t]);
      if (lane == 0) logits[(size_t)t * E + e] = v + bv;
    }
  }
}

hipError_t launch_router_logits_gemv(const uint16_t* x, const float* w, const float* bias, int T,
                                     int E, int H, float* logits, hipStream_t s) {
  if (T <= 1)
    hipLaunchKernelGGL(k_router_gemv<1>, dim3(E), dim3(64), 0, s, x, w, bias, T, E, H, logits);
  else if (T <= 4)
    hipLaunchKernelGGL(k_router_gemv<4>, dim3(E), dim3(64), 0, s, x, w, bias, T, E, H, logits);
  else if (T <= 8)
    hipLaunchKernelGGL(k_router_gemv<8>, dim3(E), dim3(64), 0, s, x, w, bias, T, E, H, logits);
  else
    hipLaunchKernelGGL(k_router_gemv<16>, dim3(E), dim3(64), 0, s, x, w, bias, T, E, H, logits);
  return hipGetLastError();
}

// ------------------------------------------------------------------ top-k + gates
// One wave per token. Lane l holds logits e = l + 64*j. K rounds of a wave arg-max ordered
// by (larger logit, then lower expert index) give the top-k in rank order; lane r keeps the
// rank-r winner. Weights: softmax over the selected logits, which equals a softmax over all
// experts renormalised over the selected ones. The shared expert's gate is sigmoid(x . wg).
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits,
                                              const uint16_t* __restrict__ x,
                                              const float* __restrict__ wg, int T, int E, int K,
                                              int H, int32_t* __restrict__ idx,
                                              float* __restrict__ wout,
                                              float* __restrict__ sgate) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // no barriers in this kernel
  const float* lt = logits + (size_t)t * E;
  const int nj = (E + 63) >> 6;  // <= 16
  float v[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int e = lane + 64 * j;
    v[j] = (j < nj && e < E) ? lt[e] : -INFINITY;
  }
  uint32_t taken = 0;
  float my_v = -INFINITY;
  int my_i = 0;
  for (int r = 0; r < K; ++r) {
    float best = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int e = lane + 64 * j;
      if (j < nj && e < E && !((taken >> j) & 1u) && (v[j] > best || (v[j] == best && e < bi))) {
        best = v[j];
        bi = e;
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float ov = __shfl_xor(best, off, 64);
      const int oi = __shfl_xor(bi, off, 64);
      if (ov > best || (ov == best && oi < bi)) {
        best = ov;
        bi = oi;
      }
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == r) {
      my_v = best;
      my_i = bi;
    }
  }
  const float vmax = __shfl(my_v, 0, 64);
  const float z = lane < K ? __expf(my_v - vmax) : 0.0f;
  const float den = wave_sum(z);
  if (lane < K) {
    idx[(size_t)t * K + lane] = my_i;
    wout[(size_t)t * K + lane] = z / den;
  }
  if (wg != nullptr) {
    const uint16_t* xt = x + (size_t)t * H;
    float g = 0.0f;
    for (int h = lane; h < H; h += 64) g = __builtin_fmaf(bf16_to_f32(xt[h]), wg[h], g);
    g = wave_sum(g);
    if (lane == 0) sgate[t] = 1.0f / (1.0f + __expf(-g));
  }
}

hipError_t launch_topk(const float* logits, const uint16_t* x, const float* wg, int T, int E,
                       int K, int H, int32_t* idx, float* w, float* sgate, hipStream_t s) {
  hipLaunchKernelGGL(k_topk, dim3((T + 3) / 4), dim3(256), 0, s, logits, x, wg, T, E, K, H, idx,
                     w, sgate);
  return hipGetLastError();
}

// ------------------------------------------------------------- per-expert counts
// One workgroup: an LDS histogram over all T*K slots (out-of-range ids are not counted).
__global__ __launch_bounds__(1024) void k_count(const int32_t* __restrict__ idx, int TK, int E,
                                                int32_t* __restrict__ counts) {
  __shared__ int h[1024];
  for (int e = threadIdx.x; e < E; e += blockDim.x) h[e] = 0;
  __syncthreads();
  for (int s = threadIdx.x; s < TK; s += blockDim.x) {
    const int e = idx[s];
    if (e >= 0 && e < E) atomicAdd(&h[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) counts[e] = h[e];
}

hipError_t launch_count(const int32_t* idx, int TK, int E, int32_t* counts, hipStream_t s) {
  hipLaunchKernelGGL(k_count, dim3(1), dim3(1024), 0, s, idx, TK, E, counts);
  return hipGetLastError();
}

}  // namespace moe
