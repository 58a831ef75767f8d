// The gated delta-rule recurrence (the model's Gated DeltaNet layers) and its C ABI
// (delta_rule.h).
//
// "Perplexity's Lily: A Breakthrough Local Inference Engine Tailored Exclusively for Apple
// Silicon", section "The Model: Qwen3.6-35B-A3B in Focus": thirty of the forty layers run a
// recurrence with a state of fixed size. The update is the gated delta rule of Yang, Kautz and
// Hatamizadeh (Gated Delta Networks, ICLR 2025) with L2-normalised queries and keys:
//   S_t = alpha S_{t-1} + beta (v - alpha S_{t-1} kh) kh^T,   o_t = S_t qh.
//
// Layout of the work: row r of a head's [dv, dk] state changes only through its own entries
// and the token's kh, qh, v[r], alpha and beta, so rows are independent. A row of dk fp32 is
// held by dk/4 consecutive lanes (one 16-byte piece each) in registers for all T tokens: the
// state is read from HBM once and written once per call, whatever T is. Per token each lane
// group reduces three dot products of the token's q and k (their norms and q.k, independent of
// the state) and two of the state row (S kh and S qh, for the old state), with DPP and
// cross-row shuffles; the next token's inputs are requested before the current token is used.
// A decode step (T = 1) is bound by the state's bytes (2 * Hv * dv * dk * 4 per sequence).
#include <cmath>

#include "delta_rule.h"
#include "moe_internal.h"

namespace moe {

namespace {

struct DeltaArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const float* g;
  const float* beta;
  const float* s_in;
  float* s_out;
  float* o;
  int Hk, Hv, dv, T;
  float scale, eps;
};

// Sum over aligned groups of N lanes (N = 16, 32 or 64); every lane of a group ends with the
// group's total.
template <int N>
__device__ __forceinline__ float lane_group_sum(float v) {
  if constexpr (N >= 64) v += __shfl_xor(v, 32, 64);
  if constexpr (N >= 32) v += __shfl_xor(v, 16, 64);
  v += dpp_partner16<8>(v);
  v += dpp_partner16<4>(v);
  v += dpp_partner16<2>(v);
  v += dpp_partner16<1>(v);
  return v;
}

__device__ __forceinline__ float4 bf16x4_to_f32(uint2 w) {
  return make_float4(bf16_to_f32(w.x & 0xFFFFu), bf16_to_f32(w.x >> 16),
                     bf16_to_f32(w.y & 0xFFFFu), bf16_to_f32(w.y >> 16));
}

__device__ __forceinline__ float dot4(const float4& a, const float4& b) {
  return __builtin_fmaf(a.x, b.x, __builtin_fmaf(a.y, b.y, __builtin_fmaf(a.z, b.z, a.w * b.w)));
}

}  // namespace

// Workgroup of 4 waves = 4 * (64 / (DK/4)) state rows of one value head of one sequence.
template <int DK>
__global__ __launch_bounds__(256) void k_delta_rule(DeltaArgs a) {
  constexpr int LPR = DK / 4;     // lanes per state row
  constexpr int RPW = 64 / LPR;   // rows per wave
  constexpr int RPG = 4 * RPW;    // rows per workgroup
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = blockIdx.y, b = blockIdx.z;
  const int i = j / (a.Hv / a.Hk);                         // the q/k head of value head j
  const int r = blockIdx.x * RPG + wave * RPW + lane / LPR;  // this lane's state row
  const int c0 = (lane % LPR) * 4;                          // its first state column
  const bool lead = (lane % LPR) == 0;

  const size_t srow = (((size_t)b * a.Hv + j) * a.dv + r) * DK + c0;
  float4 s = a.s_in ? *reinterpret_cast<const float4*>(a.s_in + srow) : make_float4(0.f, 0.f, 0.f, 0.f);
  auto qk_at = [&](const uint16_t* p, int t) {
    return *reinterpret_cast<const uint2*>(p + (((size_t)b * a.T + t) * a.Hk + i) * DK + c0);
  };
  auto v_at = [&](int t) { return a.v[(((size_t)b * a.T + t) * a.Hv + j) * a.dv + r]; };
  auto gb = [&](int t) { return ((size_t)b * a.T + t) * a.Hv + j; };

  // token 0's inputs; then each iteration requests token t + 1's before using token t's
  uint2 kn = qk_at(a.k, 0), qn = qk_at(a.q, 0);
  uint16_t vn = v_at(0);
  float gn = a.g[gb(0)], bn = a.beta[gb(0)];
  for (int t = 0; t < a.T; ++t) {
    const uint2 kw = kn, qw = qn;
    const uint16_t vw = vn;
    const float gt = gn, bt = bn;
    if (t + 1 < a.T) {
      kn = qk_at(a.k, t + 1);
      qn = qk_at(a.q, t + 1);
      vn = v_at(t + 1);
      gn = a.g[gb(t + 1)];
      bn = a.beta[gb(t + 1)];
    }
    const float4 k4 = bf16x4_to_f32(kw), q4 = bf16x4_to_f32(qw);
    // the token's normalisation (independent of the state)
    const float kk = lane_group_sum<LPR>(dot4(k4, k4));
    const float qq = lane_group_sum<LPR>(dot4(q4, q4));
    const float kq = lane_group_sum<LPR>(dot4(k4, q4));
    const float nk = 1.0f / sqrtf(kk + a.eps);
    const float nq = a.scale / sqrtf(qq + a.eps);
    const float4 kh = make_float4(k4.x * nk, k4.y * nk, k4.z * nk, k4.w * nk);
    const float4 qh = make_float4(q4.x * nq, q4.y * nq, q4.z * nq, q4.w * nq);
    const float khqh = kq * nk * nq;
    // the old state against kh and qh
    const float u = lane_group_sum<LPR>(dot4(s, kh));
    const float sq = lane_group_sum<LPR>(dot4(s, qh));
    const float alpha = __expf(gt);
    const float coef = bt * (bf16_to_f32(vw) - alpha * u);
    s.x = __builtin_fmaf(coef, kh.x, alpha * s.x);
    s.y = __builtin_fmaf(coef, kh.y, alpha * s.y);
    s.z = __builtin_fmaf(coef, kh.z, alpha * s.z);
    s.w = __builtin_fmaf(coef, kh.w, alpha * s.w);
    if (lead) a.o[(((size_t)b * a.T + t) * a.Hv + j) * a.dv + r] = __builtin_fmaf(alpha, sq, coef * khqh);
  }
  *reinterpret_cast<float4*>(a.s_out + srow) = s;
}

}  // namespace moe

using namespace moe;

extern "C" int delta_rule_forward(const delta_rule_desc_t* desc, const uint16_t* q,
                                  const uint16_t* k, const uint16_t* v, const float* g,
                                  const float* beta, const float* state_in, float* state_out,
                                  float* o, int32_t batch, int32_t T, void* stream) {
  if (!desc) return MOE_INVALID_ARG;
  const int Hk = desc->num_k_heads, Hv = desc->num_v_heads, dk = desc->dk, dv = desc->dv;
  if (Hk <= 0 || Hv <= 0 || dv <= 0) return MOE_INVALID_ARG;
  if (Hv % Hk || dv % 16 || (dk != 64 && dk != 128 && dk != 256)) return MOE_UNSUPPORTED;
  if (!(desc->eps >= 0.0f)) return MOE_INVALID_ARG;
  if (batch < 0 || T < 0) return MOE_INVALID_ARG;
  if (batch == 0) return MOE_OK;
  if (!state_out || ((uintptr_t)state_out & 15) || (state_in && ((uintptr_t)state_in & 15)))
    return MOE_INVALID_ARG;
  if (T > 0 && (!q || !k || !v || !g || !beta || !o || ((uintptr_t)q & 15) || ((uintptr_t)k & 15)))
    return MOE_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (T == 0) {  // no token: the state passes through (a zero state if none is given)
    const size_t n = (size_t)batch * Hv * dv * dk;
    if (state_in == state_out) return MOE_OK;
    if (state_in)
      return hipMemcpyAsync(state_out, state_in, n * 4, hipMemcpyDeviceToDevice, s) == hipSuccess
                 ? MOE_OK : MOE_HIP_ERROR;
    return launch_fill_zero(state_out, n, s) == hipSuccess ? MOE_OK : MOE_HIP_ERROR;
  }
  DeltaArgs a{q, k, v, g, beta, state_in, state_out, o, Hk, Hv, dv, T, desc->scale, desc->eps};
  const int rpg = 4 * (64 / (dk / 4));
  const dim3 grid(dv / rpg, Hv, batch);
  if (dk == 64) hipLaunchKernelGGL((k_delta_rule<64>), grid, dim3(256), 0, s, a);
  else if (dk == 128) hipLaunchKernelGGL((k_delta_rule<128>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((k_delta_rule<256>), grid, dim3(256), 0, s, a);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_HIP_ERROR;
}
