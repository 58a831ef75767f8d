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
// and the token's kh, qh, v[r], alpha and beta, so rows are independent, and each row stays in
// registers of a group of lanes for all T tokens of a call: the state is read from HBM once and
// written once, whatever T is. Two kernels:
//  * k_delta_rule_tok (T < kDeltaBlockFrom, decode): 4 waves; dk/4 lanes per row (4 values
//    each). Per token each lane group reduces the token's |q|^2, |k|^2 and q.k and the two dot
//    products of the old state row with kh and qh; the next token's inputs are requested before
//    the current token is used. A decode step is bound by the state's bytes.
//  * k_delta_rule_blk (longer T): dk/32 waves own 16 rows of one value head; dk/8 lanes per row
//    (8 values each). Tokens go through in blocks of 32: the block's q and k are normalised once
//    per workgroup (16 lanes per token, DPP reductions) and kept in LDS as fp32 kh and qh with
//    the token's alpha, beta, kh.qh and its v for the 16 rows; the next block's inputs are
//    requested before the current block's tokens run, and each token's LDS values are read one
//    token ahead, so the serial chain of a token is the two dot products, their reductions
//    inside rows of 16 lanes (DPP) and the row update.
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

// Sum over aligned groups of N lanes (N = 8, 16, 32 or 64); every lane of a group ends with the
// group's total.
template <int N>
__device__ __forceinline__ float lane_group_sum(float v) {
  if constexpr (N >= 64) v += __shfl_xor(v, 32, 64);
  if constexpr (N >= 32) v += __shfl_xor(v, 16, 64);
  if constexpr (N >= 16) v += dpp_partner16<8>(v);
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

constexpr int kDeltaBlockFrom = 16;  // T from which the block kernel runs
constexpr int kDeltaTB = 32;         // tokens per block staged in LDS
constexpr int kDeltaRows = 16;       // state rows per workgroup of the block kernel

}  // namespace

// Workgroup of 4 waves = 4 * (64 / (DK/4)) state rows of one value head of one sequence.
template <int DK>
__global__ __launch_bounds__(256) void k_delta_rule_tok(DeltaArgs a) {
  constexpr int LPR = DK / 4;     // lanes per state row
  constexpr int RPW = 64 / LPR;   // rows per wave
  constexpr int RPG = 4 * RPW;    // rows per workgroup
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = blockIdx.x, b = blockIdx.z;  // head fastest: with Hv a multiple of 8 a head's row blocks share an XCD (and its L2)
  const int i = j / (a.Hv / a.Hk);                         // the q/k head of value head j
  const int r = blockIdx.y * RPG + wave * RPW + lane / LPR;  // this lane's state row
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

// Workgroup of DK/32 waves = 16 state rows of one value head of one sequence.
template <int DK>
__global__ __launch_bounds__(2 * DK) void k_delta_rule_blk(DeltaArgs a) {
  constexpr int NW = DK / 32;          // waves
  constexpr int NT = 64 * NW;          // threads
  constexpr int LPR = DK / 8;          // lanes per state row
  constexpr int RPW = 64 / LPR;        // rows per wave
  constexpr int TB = kDeltaTB;
  constexpr int E = DK / 16;           // q / k values per lane in the staging (16 lanes a token)
  constexpr int TPW = TB / NW;         // tokens per wave in the staging
  constexpr int PASS = TPW / 4;        // staging passes (a wave normalises 4 tokens per pass)
  constexpr int VPT = (TB * kDeltaRows + NT - 1) / NT;  // v values per thread in the staging
  static_assert(NW * RPW == kDeltaRows && PASS * 4 == TPW && E % 4 == 0, "tiling");
  __shared__ __attribute__((aligned(16))) float kh[TB * DK];
  __shared__ __attribute__((aligned(16))) float qh[TB * DK];
  __shared__ __attribute__((aligned(16))) float sc4[TB * 4];  // alpha, beta, kh.qh, -
  __shared__ float vs[TB * kDeltaRows];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = blockIdx.x, b = blockIdx.z;  // head fastest: with Hv a multiple of 8 a head's row blocks share an XCD (and its L2)
  const int i = j / (a.Hv / a.Hk);                 // the q/k head of value head j
  const int r0 = blockIdx.y * kDeltaRows;
  const int rl = wave * RPW + lane / LPR;          // this lane's row in the workgroup
  const int r = r0 + rl;
  const int c0 = (lane % LPR) * 8;                 // its first state column
  const bool lead = (lane % LPR) == 0;

  const size_t srow = (((size_t)b * a.Hv + j) * a.dv + r) * DK + c0;
  float4 s0 = make_float4(0.f, 0.f, 0.f, 0.f), s1 = s0;
  if (a.s_in) {
    s0 = *reinterpret_cast<const float4*>(a.s_in + srow);
    s1 = *reinterpret_cast<const float4*>(a.s_in + srow + 4);
  }

  // ---- staging: token (wave*TPW + 4*p + lane/16) of a block, dimensions E*(lane%16) .. + E
  uint2 rq[PASS][E / 4], rk[PASS][E / 4];
  float rv[VPT];
  float rgb = 0.0f;   // threads 0..TB-1: the token's g; TB..2TB-1: its beta
  const int sr = lane >> 4, sc = lane & 15;
  auto tok_of = [&](int t0, int t) { return min(t0 + t, a.T - 1); };
  auto load_block = [&](int t0) {
#pragma unroll
    for (int p = 0; p < PASS; ++p) {
      const int t = tok_of(t0, wave * TPW + 4 * p + sr);
      const size_t base = (((size_t)b * a.T + t) * a.Hk + i) * DK + E * sc;
#pragma unroll
      for (int e = 0; e < E / 4; ++e) {
        rq[p][e] = *reinterpret_cast<const uint2*>(a.q + base + 4 * e);
        rk[p][e] = *reinterpret_cast<const uint2*>(a.k + base + 4 * e);
      }
    }
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int idx = tid + u * NT;
      const int t = tok_of(t0, idx / kDeltaRows);
      rv[u] = idx < TB * kDeltaRows
                  ? bf16_to_f32(a.v[(((size_t)b * a.T + t) * a.Hv + j) * a.dv + r0 + idx % kDeltaRows])
                  : 0.0f;
    }
    if (tid < 2 * TB) {
      const float* src = tid < TB ? a.g : a.beta;
      rgb = src[((size_t)b * a.T + tok_of(t0, tid % TB)) * a.Hv + j];
    }
  };
  // normalise the staged block into LDS (16 lanes per token, four tokens per wave at a time)
  auto stage_block = [&]() {
#pragma unroll
    for (int p = 0; p < PASS; ++p) {
      float4 kf[E / 4], qf[E / 4];
      float kk = 0.0f, qq = 0.0f, kq = 0.0f;
#pragma unroll
      for (int e = 0; e < E / 4; ++e) {
        kf[e] = bf16x4_to_f32(rk[p][e]);
        qf[e] = bf16x4_to_f32(rq[p][e]);
        kk += dot4(kf[e], kf[e]);
        qq += dot4(qf[e], qf[e]);
        kq += dot4(kf[e], qf[e]);
      }
      kk = lane_group_sum<16>(kk);
      qq = lane_group_sum<16>(qq);
      kq = lane_group_sum<16>(kq);
      const int t = wave * TPW + 4 * p + sr;
      const float nk = 1.0f / sqrtf(kk + a.eps);
      const float nq = a.scale / sqrtf(qq + a.eps);
#pragma unroll
      for (int e = 0; e < E / 4; ++e) {
        *reinterpret_cast<float4*>(kh + t * DK + E * sc + 4 * e) =
            make_float4(kf[e].x * nk, kf[e].y * nk, kf[e].z * nk, kf[e].w * nk);
        *reinterpret_cast<float4*>(qh + t * DK + E * sc + 4 * e) =
            make_float4(qf[e].x * nq, qf[e].y * nq, qf[e].z * nq, qf[e].w * nq);
      }
      if (sc == 0) sc4[t * 4 + 2] = kq * nk * nq;
    }
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int idx = tid + u * NT;
      if (idx < TB * kDeltaRows) vs[idx] = rv[u];
    }
    if (tid < TB) sc4[tid * 4 + 0] = __expf(rgb);
    else if (tid < 2 * TB) sc4[(tid - TB) * 4 + 1] = rgb;
  };

  // one token's LDS values
  struct Tok {
    float4 k0, k1, q0, q1, sc;
    float v;
  };
  auto read_tok = [&](int t) {
    Tok x;
    x.k0 = *reinterpret_cast<const float4*>(kh + t * DK + c0);
    x.k1 = *reinterpret_cast<const float4*>(kh + t * DK + c0 + 4);
    x.q0 = *reinterpret_cast<const float4*>(qh + t * DK + c0);
    x.q1 = *reinterpret_cast<const float4*>(qh + t * DK + c0 + 4);
    x.sc = *reinterpret_cast<const float4*>(sc4 + t * 4);
    x.v = vs[t * kDeltaRows + rl];
    return x;
  };

  load_block(0);
  stage_block();
  __syncthreads();
  for (int t0 = 0; t0 < a.T; t0 += TB) {
    const int nt = min(TB, a.T - t0);
    const bool more = t0 + TB < a.T;
    if (more) load_block(t0 + TB);   // in flight while this block's tokens run
    // one token: the two dot products of the old row with kh and qh (two chains of four
    // products each), their row sums (DPP inside rows of 16 lanes), the row update
    auto step = [&](const Tok& x, int t) {
      const float u = lane_group_sum<LPR>(dot4(s0, x.k0) + dot4(s1, x.k1));  // S_old kh
      const float sq = lane_group_sum<LPR>(dot4(s0, x.q0) + dot4(s1, x.q1));  // S_old qh
      const float alpha = x.sc.x, bt = x.sc.y, khqh = x.sc.z;
      const float coef = bt * (x.v - alpha * u);
      s0.x = __builtin_fmaf(coef, x.k0.x, alpha * s0.x);
      s0.y = __builtin_fmaf(coef, x.k0.y, alpha * s0.y);
      s0.z = __builtin_fmaf(coef, x.k0.z, alpha * s0.z);
      s0.w = __builtin_fmaf(coef, x.k0.w, alpha * s0.w);
      s1.x = __builtin_fmaf(coef, x.k1.x, alpha * s1.x);
      s1.y = __builtin_fmaf(coef, x.k1.y, alpha * s1.y);
      s1.z = __builtin_fmaf(coef, x.k1.z, alpha * s1.z);
      s1.w = __builtin_fmaf(coef, x.k1.w, alpha * s1.w);
      if (lead)
        a.o[(((size_t)b * a.T + t0 + t) * a.Hv + j) * a.dv + r] = __builtin_fmaf(alpha, sq, coef * khqh);
    };
    // two tokens per iteration, each token's LDS values read one token ahead into the other
    // register set
    Tok xa = read_tok(0);
    for (int t = 0; t < nt; t += 2) {
      const Tok xb = read_tok(min(t + 1, nt - 1));
      step(xa, t);
      if (t + 1 >= nt) break;
      xa = read_tok(min(t + 2, nt - 1));
      step(xb, t + 1);
    }
    if (more) {
      __syncthreads();   // every wave is done with this block's LDS
      stage_block();
      __syncthreads();
    }
  }
  *reinterpret_cast<float4*>(a.s_out + srow) = s0;
  *reinterpret_cast<float4*>(a.s_out + srow + 4) = s1;
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
  if (T < kDeltaBlockFrom) {
    const int rpg = 4 * (64 / (dk / 4));
    const dim3 grid(Hv, dv / rpg, batch);
    if (dk == 64) hipLaunchKernelGGL((k_delta_rule_tok<64>), grid, dim3(256), 0, s, a);
    else if (dk == 128) hipLaunchKernelGGL((k_delta_rule_tok<128>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_delta_rule_tok<256>), grid, dim3(256), 0, s, a);
  } else {
    const dim3 grid(Hv, dv / kDeltaRows, batch);  // workgroups of 2 * dk threads
    if (dk == 64) hipLaunchKernelGGL((k_delta_rule_blk<64>), grid, dim3(128), 0, s, a);
    else if (dk == 128) hipLaunchKernelGGL((k_delta_rule_blk<128>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_delta_rule_blk<256>), grid, dim3(512), 0, s, a);
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_HIP_ERROR;
}
