// Internal declarations and device helpers shared by the HIP kernels of the MoE library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_w4.h"

namespace moe {

constexpr int kBlockM = MOE_BLOCK_M;  // rows per grouped-GEMM tile (block-map granularity)
constexpr int kChunkSlots = 1024;     // slots per permutation chunk (one histogram row each)
constexpr int kDecodeMaxT = 16;       // largest T served by the decode (GEMV) kernels
constexpr int kGroup = 64;            // quantisation group along the input dimension

// Sizes of one layer call.
struct Dims {
  int H, E, K, F, Fs, T;
  int TK() const { return T * K; }
};

// Parameters of the prefill grouped GEMM (k_gemm_w4).
struct GemmParams {
  const int4* blocks;
  const int* num_blocks;
  const uint16_t* a_routed;  // gate/up: x [T,H]; down: A routed rows [TK, F]
  const uint16_t* a_shared;  // gate/up: x [T,H]; down: A shared rows [T, Fs]
  const int* sorted_slots;
  int K, E, TK;
  int kdim_routed, kdim_shared;  // input dimension of the routed / shared matrices
  int n_routed, n_shared;        // output columns of one projection (routed / shared)
  moe_w4_t w0, w1;               // routed weights (gate/up: gate, up; down: down, unused)
  moe_w4_t sw0, sw1;             // shared-expert weights
  void* out;                     // A (bf16) | Y (fp32) | y (fp32)
  int out_ld;                    // H for the down projection
  const float* topk_w;
  const float* shared_gate;
};

enum GemmMode { kGateUp = 0, kDownStore = 1, kDownAtomic = 2 };

// Launchers (return the launch status).
hipError_t launch_router_logits_mfma(const uint16_t* x, const float* w, const float* bias, int T,
                                     int E, int H, float* logits, hipStream_t s);
hipError_t launch_router_logits_gemv(const uint16_t* x, const float* w, const float* bias, int T,
                                     int E, int H, float* logits, hipStream_t s);
hipError_t launch_topk(const float* logits, const uint16_t* x, const float* wg, int T, int E,
                       int K, int H, int32_t* idx, float* w, float* sgate, hipStream_t s);
hipError_t launch_count(const int32_t* idx, int TK, int E, int32_t* counts, hipStream_t s);
hipError_t launch_route_small(const float* logits, const uint16_t* x, const float* wg,
                              const Dims& d, int32_t* idx, float* w, float* sgate,
                              const moe_plan_t& plan, hipStream_t s);
hipError_t launch_permute(const int32_t* idx, const Dims& d, bool shared, int32_t* hist,
                          const moe_plan_t& plan, hipStream_t s);
hipError_t launch_gemm_w4(int mode, const GemmParams& p, int max_blocks, hipStream_t s);
hipError_t launch_fill_zero(float* p, size_t n, hipStream_t s);
hipError_t launch_combine(const float* y_perm, const int32_t* slot_pos, const float* topk_w,
                          const float* shared_y, const float* sgate, const Dims& d, float* out,
                          hipStream_t s);
hipError_t launch_dec_gateup(const Dims& d, const moe_layer_desc_t& desc, const uint16_t* x,
                             const moe_plan_t& plan, int max_blocks, uint16_t* a_out,
                             hipStream_t s);
hipError_t launch_dec_down(const Dims& d, const moe_layer_desc_t& desc, const uint16_t* a,
                           const moe_plan_t& plan, const float* topk_w, const float* sgate,
                           float* out, hipStream_t s);
hipError_t launch_debug_dequant(const moe_w4_t& w, int n_rows, int kin, int mat, int row,
                                float* out_f32, uint16_t* out_bf16, hipStream_t s);

#ifdef __HIPCC__
// ------------------------------------------------------------------ device helpers
typedef short bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Two fp32 values -> packed bf16 pair (round to nearest even; low half = lo).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2_t v = {lo, hi};
  bf16x2_t r = __builtin_convertvector(v, bf16x2_t);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float v) {
  return (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu);
}

// Byte n of a word as fp32 (v_cvt_f32_ubyteN: one instruction).
#define MOE_CVT_UBYTE(N)                                                   \
  __device__ __forceinline__ float ubyte##N(uint32_t x) {                 \
    float r;                                                               \
    asm("v_cvt_f32_ubyte" #N " %0, %1" : "=v"(r) : "v"(x));                \
    return r;                                                              \
  }
MOE_CVT_UBYTE(0)
MOE_CVT_UBYTE(1)
MOE_CVT_UBYTE(2)
MOE_CVT_UBYTE(3)
#undef MOE_CVT_UBYTE

// Dequantise one packed word (elements 8i..8i+7 at nibbles 0..7) with its group's scale s
// and bias b: w_j = s * q_j + b in one fp32 FMA (exact whenever s*q+b fits fp32, e.g. for
// b = -8s), then rounded to bf16. out[j/2] holds elements (j, j+1), low half first, which
// is the operand order of the bf16 MFMA and dot instructions.
__device__ __forceinline__ void dequant8(uint32_t w, float s, float b, uint32_t out[4]) {
  const uint32_t lo = w & 0x0F0F0F0Fu;         // nibbles 0,2,4,6 in bytes 0..3
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;  // nibbles 1,3,5,7 in bytes 0..3
  out[0] = pack_bf16x2(__builtin_fmaf(s, ubyte0(lo), b), __builtin_fmaf(s, ubyte0(hi), b));
  out[1] = pack_bf16x2(__builtin_fmaf(s, ubyte1(lo), b), __builtin_fmaf(s, ubyte1(hi), b));
  out[2] = pack_bf16x2(__builtin_fmaf(s, ubyte2(lo), b), __builtin_fmaf(s, ubyte2(hi), b));
  out[3] = pack_bf16x2(__builtin_fmaf(s, ubyte3(lo), b), __builtin_fmaf(s, ubyte3(hi), b));
}

// The fp32 values before rounding (test export only).
__device__ __forceinline__ void dequant8_f32(uint32_t w, float s, float b, float out[8]) {
  const uint32_t lo = w & 0x0F0F0F0Fu;
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;
  out[0] = __builtin_fmaf(s, ubyte0(lo), b);
  out[1] = __builtin_fmaf(s, ubyte0(hi), b);
  out[2] = __builtin_fmaf(s, ubyte1(lo), b);
  out[3] = __builtin_fmaf(s, ubyte1(hi), b);
  out[4] = __builtin_fmaf(s, ubyte2(lo), b);
  out[5] = __builtin_fmaf(s, ubyte2(hi), b);
  out[6] = __builtin_fmaf(s, ubyte3(lo), b);
  out[7] = __builtin_fmaf(s, ubyte3(hi), b);
}

// acc += a.lo*b.lo + a.hi*b.hi for packed bf16 pairs (products exact, fp32 sum).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.0f + __expf(-g)) * u;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Top-k of one token's E logits by one wave (E <= 64*NJ): lane l holds logits e = l + 64*j.
// K rounds of a wave arg-max ordered by (larger logit, then lower expert index); lane r ends
// with the rank-r winner (my_v, my_i), lanes >= K with -inf.
template <int NJ>
__device__ __forceinline__ void wave_topk(const float* __restrict__ lt, int E, int K, int lane,
                                          float& my_v, int& my_i) {
  float v[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = lane + 64 * j;
    v[j] = e < E ? lt[e] : -INFINITY;
  }
  uint32_t taken = 0;
  my_v = -INFINITY;
  my_i = 0;
  for (int r = 0; r < K; ++r) {
    float best = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int e = lane + 64 * j;
      if (e < E && !((taken >> j) & 1u) && (v[j] > best || (v[j] == best && e < bi))) {
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
}

// x . wg for one token (bf16 x, fp32 wg), by one wave: lane l takes the contiguous inputs
// [l*H/64, (l+1)*H/64) in pieces of four, all loads issued before the FMAs. H % 64 == 0.
__device__ __forceinline__ float shared_gate_logit(const uint16_t* __restrict__ xt,
                                                   const float* __restrict__ wg, int H, int lane) {
  const int per = H >> 6;  // inputs per lane
  const int base = lane * per;
  float g0 = 0.0f, g1 = 0.0f;
  int i = 0;
  for (; i + 32 <= per; i += 32) {  // 64 B of x and 128 B of wg per step
    uint4 xv[4];
    float4 wv[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) xv[j] = *reinterpret_cast<const uint4*>(xt + base + i + 8 * j);
#pragma unroll
    for (int j = 0; j < 8; ++j) wv[j] = *reinterpret_cast<const float4*>(wg + base + i + 4 * j);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t xw[4] = {xv[j].x, xv[j].y, xv[j].z, xv[j].w};
      const float4 a = wv[2 * j], b = wv[2 * j + 1];
      g0 = __builtin_fmaf(bf16_to_f32(xw[0] & 0xFFFFu), a.x, g0);
      g1 = __builtin_fmaf(bf16_to_f32(xw[0] >> 16), a.y, g1);
      g0 = __builtin_fmaf(bf16_to_f32(xw[1] & 0xFFFFu), a.z, g0);
      g1 = __builtin_fmaf(bf16_to_f32(xw[1] >> 16), a.w, g1);
      g0 = __builtin_fmaf(bf16_to_f32(xw[2] & 0xFFFFu), b.x, g0);
      g1 = __builtin_fmaf(bf16_to_f32(xw[2] >> 16), b.y, g1);
      g0 = __builtin_fmaf(bf16_to_f32(xw[3] & 0xFFFFu), b.z, g0);
      g1 = __builtin_fmaf(bf16_to_f32(xw[3] >> 16), b.w, g1);
    }
  }
  for (; i < per; ++i) g0 = __builtin_fmaf(bf16_to_f32(xt[base + i]), wg[base + i], g0);
  return wave_sum(g0 + g1);
}
#endif  // __HIPCC__

}  // namespace moe
