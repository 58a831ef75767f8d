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
hipError_t launch_router_split(const float* w, int E, int H, uint16_t* parts, hipStream_t s);
hipError_t launch_router_logits_mfma(const uint16_t* x, const uint16_t* parts, const float* bias,
                                     int T, int E, int H, float* logits, hipStream_t s);
hipError_t launch_router_logits_gemv(const uint16_t* x, const float* w, const float* bias, int T,
                                     int E, int H, float* logits, hipStream_t s);
hipError_t launch_topk(const float* logits, const uint16_t* x, const float* wg, int T, int E,
                       int K, int H, int32_t* idx, float* w, float* sgate, hipStream_t s);
hipError_t launch_count(const int32_t* idx, int TK, int E, int32_t* counts, hipStream_t s);
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
#endif  // __HIPCC__

}  // namespace moe
