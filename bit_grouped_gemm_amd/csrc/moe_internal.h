// Internal declarations and device helpers shared by the HIP kernels of the MoE library.
#pragma once

#include <hip/hip_runtime.h>
#include <climits>
#include <stdint.h>

#include "moe_w4.h"

namespace moe {

constexpr int kBlockM = MOE_BLOCK_M;  // rows per grouped-GEMM tile (block-map granularity)
constexpr int kChunkSlots = 1024;     // slots per permutation chunk (one histogram row each)
constexpr int kPermuteOneMax = 8192;  // up to this many slots the permutation is one workgroup
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
// Prefill router logits as router_splits(T, E, H) partial slices [S][T][E+1] (split-K over the
// inputs); column E of a slice holds the partial shared-gate logit x . wg when wg != nullptr.
constexpr int kRouterMaxSplits = 8;
int router_splits(int T, int E, int H);
hipError_t launch_router_logits_mfma(const uint16_t* x, const float* w, const float* bias,
                                     const float* wg, int T, int E, int H, float* logits,
                                     hipStream_t s);
hipError_t launch_router_logits_gemv(const uint16_t* x, const float* w, const float* bias, int T,
                                     int E, int H, float* logits, hipStream_t s);
// Top-k over the sum of S logit slices [S][T][ld]; the shared gate from column E of the slices
// (gate_col) or from x . wg (wg != nullptr), else not written.
hipError_t launch_topk(const float* logits, int S, int ld, bool gate_col, const uint16_t* x,
                       const float* wg, int T, int E, int K, int H, int32_t* idx, float* w,
                       float* sgate, hipStream_t s);
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
// Decode path of moe_layer_forward in three launches (decode.hip).
struct DecodeBufs {
  float* logits;     // [T, E] router logits, then [T] shared-gate logits
  int32_t* route;    // per-expert route record handed from the gate/up to the down kernel
  uint16_t* a;       // [T*K*F] routed activations (grouped rows), then [T*Fs] shared
};
bool decode_fast_ok(const Dims& d);
size_t decode_route_bytes(const Dims& d);
// A decode layer inside the stack (moe_stack_forward): the first kernel derives the layer input
// x = bf16(RMSNorm(resid)) itself (bit for bit as k_residual_rmsnorm does) and writes it to x,
// and the last kernel adds the layer output into resid in place.
struct StackFuse {
  float* resid;  // [T, H] fp32 residual stream
  uint16_t* x;   // [T, H] bf16: written by the first kernel, read by the second
  float eps;
};
// phase < 0: all three launches; 0, 1, 2: only that one. sf == nullptr: a plain layer call
// (x in, out = the layer output); otherwise x and out are ignored and sf is used.
hipError_t launch_decode_layer(const Dims& d, const moe_layer_desc_t& desc, const uint16_t* x,
                               const DecodeBufs& b, float* out, hipStream_t s, int phase,
                               const StackFuse* sf = nullptr);
// init: 0 r <- r + y, 1 r <- x (as fp32), 2 r unchanged; then x <- bf16(RMSNorm(r)).
hipError_t launch_residual_rmsnorm(const float* y, float* r, uint16_t* x, int T, int H, float eps,
                                   int init, hipStream_t s);
hipError_t launch_debug_dequant(const moe_w4_t& w, int n_rows, int kin, int mat, int row,
                                float* out_f32, uint16_t* out_bf16, hipStream_t s);
hipError_t launch_mfma_loop(int workgroups, int iters, float* sink, hipStream_t s);
double mfma_loop_flops(int workgroups, int iters);
hipError_t launch_stream_read(const void* p, size_t bytes, int workgroups, uint32_t* sink,
                              hipStream_t s);

#ifdef __HIPCC__
// ------------------------------------------------------------------ device helpers
typedef short bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 16 bytes that a call reads once (weights, cache rows), as a non-temporal load.
__device__ __forceinline__ uint4 load_nt(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
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

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// Two nibbles of w selected by mask m (0x000F000F: nibbles 0 and 4; 0x00F000F0: nibbles 1 and
// 5) as two fp16 values in one word. A nibble q left in place is an fp16 subnormal: q * 2^-24
// at bits 0-3, q * 2^-20 at bits 4-7. The AND is written as an instruction of its own so that
// the pair stays packed and each half is selected by the widening multiply-add (op_sel)
// instead of being extracted nibble by nibble.
__device__ __forceinline__ f16x2_t nibble_pair(uint32_t w, uint32_t m) {
  uint32_t r;
  asm("v_and_b32 %0, %1, %2" : "=v"(r) : "v"(w), "v"(m));
  return __builtin_bit_cast(f16x2_t, r);
}

// Dequantise one packed word (elements 8i..8i+7 at nibbles 0..7) with its group's scale s
// and bias b: w_j = s * q_j + b in one fp32 FMA, then rounded to bf16. The FMA takes q_j as the
// fp16 subnormal q_j * 2^-24 or q_j * 2^-20 (widened exactly by v_fma_mix_f32) and s * 2^24 or
// s * 2^20, so the product is exactly s * q_j and the one rounding is that of fma(s, q_j, b),
// for every finite scale of magnitude below 2^104 (s * 2^24 exact). One shift and four ANDs
// expose the eight nibbles. out[j/2] holds elements (j, j+1), low half first, which is the
// operand order of the bf16 MFMA and dot instructions.
__device__ __forceinline__ void dequant8_f32(uint32_t w, float s, float b, float out[8]) {
  const float s24 = s * 16777216.0f, s20 = s * 1048576.0f;
  const uint32_t w8 = w >> 8;
  const f16x2_t p0 = nibble_pair(w, 0x000F000Fu), p1 = nibble_pair(w, 0x00F000F0u),
                p2 = nibble_pair(w8, 0x000F000Fu), p3 = nibble_pair(w8, 0x00F000F0u);
  out[0] = __builtin_fmaf((float)p0.x, s24, b);
  out[1] = __builtin_fmaf((float)p1.x, s20, b);
  out[2] = __builtin_fmaf((float)p2.x, s24, b);
  out[3] = __builtin_fmaf((float)p3.x, s20, b);
  out[4] = __builtin_fmaf((float)p0.y, s24, b);
  out[5] = __builtin_fmaf((float)p1.y, s20, b);
  out[6] = __builtin_fmaf((float)p2.y, s24, b);
  out[7] = __builtin_fmaf((float)p3.y, s20, b);
}

__device__ __forceinline__ void dequant8(uint32_t w, float s, float b, uint32_t out[4]) {
  float f[8];
  dequant8_f32(w, s, b, f);
  out[0] = pack_bf16x2(f[0], f[1]);
  out[1] = pack_bf16x2(f[2], f[3]);
  out[2] = pack_bf16x2(f[4], f[5]);
  out[3] = pack_bf16x2(f[6], f[7]);
}

// acc += a.lo*b.lo + a.hi*b.hi for packed bf16 pairs (products exact, fp32 sum).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// silu(g) * u = g / (1 + e^-g) * u, with the hardware reciprocal (about 1 ulp) in place of
// a full-precision division: the result is rounded to bf16 right after.
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Value of the butterfly partner lane at distance O (1, 2, 4 or 8) inside a row of 16 lanes,
// through DPP (no LDS round trip): quad_perm swaps for O = 1, 2, the half-row mirror for O = 4
// and the row mirror for O = 8. The partner always differs from the lane in bit log2(O) (the
// mirrors pair i with 7-i and 15-i), so a halving butterfly over these pairs still ends with
// lane r holding the entries selected by r's bits.
template <int O>
__device__ __forceinline__ float dpp_partner16(float v) {
  constexpr int ctrl = O == 8 ? 0x140 : (O == 4 ? 0x141 : (O == 2 ? 0x4E : 0xB1));
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), ctrl, 0xF, 0xF, false));
}

// Inclusive prefix sum of v over the 64 lanes: DPP row shifts inside rows of 16 (lanes whose
// source falls outside the row add 0), then the totals of the lower rows read from lanes 15,
// 31, 47.
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);
  const int r0 = __builtin_amdgcn_readlane(v, 15);
  const int r1 = __builtin_amdgcn_readlane(v, 31);
  const int r2 = __builtin_amdgcn_readlane(v, 47);
  const int row = lane >> 4;
  return v + (row > 0 ? r0 : 0) + (row > 1 ? r1 : 0) + (row > 2 ? r2 : 0);
}

// Maximum of v over the wave, returned to every lane (as a scalar). DPP row shifts 1, 2, 4, 8
// leave each row's maximum in its lane 15; row_bcast:15 and row_bcast:31 then carry it into
// lane 63, which is read once. Lanes with no DPP source take INT_MIN (the identity).
__device__ __forceinline__ int wave_max_i32(int v) {
  constexpr int kMin = INT_MIN;
  v = max(v, __builtin_amdgcn_update_dpp(kMin, v, 0x111, 0xF, 0xF, false));  // row_shr:1
  v = max(v, __builtin_amdgcn_update_dpp(kMin, v, 0x112, 0xF, 0xF, false));  // row_shr:2
  v = max(v, __builtin_amdgcn_update_dpp(kMin, v, 0x114, 0xF, 0xF, false));  // row_shr:4
  v = max(v, __builtin_amdgcn_update_dpp(kMin, v, 0x118, 0xF, 0xF, false));  // row_shr:8
  v = max(v, __builtin_amdgcn_update_dpp(kMin, v, 0x142, 0xA, 0xF, false));  // row_bcast:15
  v = max(v, __builtin_amdgcn_update_dpp(kMin, v, 0x143, 0xC, 0xF, false));  // row_bcast:31
  return __builtin_amdgcn_readlane(v, 63);
}

// fp32 -> int32 key with the same order (for non-NaN values): negative values have their
// magnitude bits inverted. -0 is first turned into +0 (x + 0 = +0 for x = -0), so that equal
// values have equal keys. INT_MIN lies below every key of a non-NaN value (-inf included).
__device__ __forceinline__ int order_key(float x) {
  const int b = __float_as_int(x + 0.0f);
  return b ^ ((b >> 31) & 0x7FFFFFFF);
}
__device__ __forceinline__ float key_value(int k) {
  return __int_as_float(k ^ ((k >> 31) & 0x7FFFFFFF));
}

// Top-k of one token's E logits by one wave (E <= 64*NJ) with the softmax over the selected
// logits. Lane l holds logits e = NJ*l + j in v[j] (consecutive experts per lane). The order
// (larger logit first, lower expert index first among equal logits) is a total order, so the
// selection is unique:
//   1. each lane sorts its NJ (key, index) pairs by that order once (odd-even transposition on
//      64-bit composites, so equal keys keep ascending indices);
//   2. each of the K rounds takes the wave maximum M of the lanes' heads; the winner is the
//      lowest lane whose head equals M (a lower lane holds only lower indices), read with one
//      ballot; that lane drops its head.
// Lane r < K ends with the rank-r expert my_i, its logit my_v and its renormalised weight
// my_w = exp(my_v - M_0) / sum_r exp(M_r - M_0), the sum taken in rank order; lanes >= K get
// my_w = 0. on_rank(r, I) runs on the whole wave as soon as round r has chosen expert I
// (uniform), so a caller can hand each rank on before the later rounds finish.
struct NoRankHook {
  __device__ void operator()(int, int) const {}
};
template <int NJ, typename OnRank = NoRankHook>
__device__ __forceinline__ void wave_topk_softmax(const float (&v)[NJ], int E, int K, int lane,
                                                  float& my_v, int& my_i, float& my_w,
                                                  OnRank on_rank = OnRank()) {
  // composite: order key (sign flipped to unsigned order) above the complemented index, so a
  // larger composite is earlier in the order
  uint64_t c[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = NJ * lane + j;
    const int key = e < E ? order_key(v[j]) : INT_MIN;
    c[j] = ((uint64_t)((uint32_t)key ^ 0x80000000u) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
  }
#pragma unroll
  for (int pass = 0; pass < NJ; ++pass) {
#pragma unroll
    for (int j = pass & 1; j + 1 < NJ; j += 2) {
      const uint64_t a = c[j], b = c[j + 1];
      const bool sw = b > a;
      c[j] = sw ? b : a;
      c[j + 1] = sw ? a : b;
    }
  }
  int key[NJ], idx[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    key[j] = (int)((uint32_t)(c[j] >> 32) ^ 0x80000000u);
    idx[j] = (int)(0xFFFFFFFFu - (uint32_t)c[j]);
  }
  int sel_key = INT_MIN, sel_idx = 0;
  for (int r = 0; r < K; ++r) {
    const int M = wave_max_i32(key[0]);
    const int L = (int)__builtin_ctzll(__ballot(key[0] == M));
    const int I = __builtin_amdgcn_readlane(idx[0], L);
    on_rank(r, I);
    if (lane == L) {
#pragma unroll
      for (int j = 0; j + 1 < NJ; ++j) {
        key[j] = key[j + 1];
        idx[j] = idx[j + 1];
      }
      key[NJ - 1] = INT_MIN;
    }
    if (lane == r) {
      sel_key = M;
      sel_idx = I;
    }
  }
  my_v = lane < K ? key_value(sel_key) : -INFINITY;
  my_i = sel_idx;
  const float m0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_v), 0));
  const float z = lane < K ? __expf(my_v - m0) : 0.0f;
  float den = 0.0f;
  for (int r = 0; r < K; ++r) den += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(z), r));
  my_w = lane < K ? z / den : 0.0f;
}

// Lane l takes logits NJ*l .. NJ*l + NJ - 1 (-inf past E).
template <int NJ>
__device__ __forceinline__ void load_logits(const float* __restrict__ lt, int E, int lane,
                                            float (&v)[NJ]) {
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = NJ * lane + j;
    v[j] = e < E ? lt[e] : -INFINITY;
  }
}

template <int NJ>
__device__ __forceinline__ void wave_topk(const float* __restrict__ lt, int E, int K, int lane,
                                          float& my_v, int& my_i, float& my_w) {
  float v[NJ];
  load_logits<NJ>(lt, E, lane, v);
  wave_topk_softmax<NJ>(v, E, K, lane, my_v, my_i, my_w);
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
