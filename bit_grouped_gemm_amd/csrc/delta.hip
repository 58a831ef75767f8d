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

// ================================================================ chunked form (long T)
// The same recurrence over chunks of kDeltaChunk = 32 tokens, as in the chunkwise form of
// Gated Delta Networks (section 3 of Yang, Kautz and Hatamizadeh): within a chunk that starts
// from state S0, with G_s the chunk's running sum of g (so exp(G_s - G_r) is the decay from
// token r to token s) and gamma_s = exp(G_s),
//   delta_s = beta_s (v_s - gamma_s S0 kh_s) - sum_{r<s} M[s,r] delta_r,
//       M[s,r] = beta_s exp(G_s - G_r) (kh_s . kh_r), i.e. delta = (I + M)^-1 R = T R,
//   o_t = gamma_t S0 qh_t + sum_{s<=t} P[t,s] delta_s,  P[t,s] = exp(G_t - G_s) (qh_t . kh_s),
//   S   = exp(G_last) S0 + sum_s exp(G_last - G_s) delta_s kh_s^T,
// which unrolls the per-token update exactly (fp32 rounding aside). Written as matrices over
// the chunk's tokens (rows) and the state's rows (columns), with U = T diag(beta gamma) Kh,
// Vb = T diag(beta) V, Q' = diag(gamma) Qh - P U and O' = P Vb:
//   delta = Vb - U S0^T,   o = O' + Q' S0^T,
// where U, Vb, Q' and O' depend only on the chunk's inputs, so one pass forms them for all
// chunks at once and the serial part is one product with the state per chunk.
//  * k_delta_prep: one workgroup per (value head, chunk, sequence): normalises the chunk's
//    keys and queries (as k_delta_rule_blk does), the running sums of g, the dot products
//    kh_s . kh_r and qh_t . kh_s on fp32 MFMA, M and P, T by a blocked inverse (8 x 8
//    diagonal blocks by forward substitution, then two doubling steps), then U, Q', Vb and O'
//    on fp32 MFMA, 32 columns per wave at a time; writes them, kh transposed and the decays
//    to the chunk's record. Tokens past T are zero keys and queries with beta = 0, so they
//    add nothing.
//  * k_delta_chunk: one workgroup per 16 state rows of a value head, dk/16 waves (at most 8);
//    the state stays in registers for the whole call, wave w holding columns
//    [w*dk/NW, (w+1)*dk/NW) of the 16 rows in the accumulator layout of
//    v_mfma_f32_16x16x4_f32. A wave loads its own columns of U, Q' and kh^T straight into
//    registers, one chunk ahead. Per chunk: U S0^T and Q' S0^T on MFMA over each wave's
//    columns (the state registers are the B operand as they are), the waves' shares added
//    through LDS into delta and o, then the rank-32 state update on MFMA into the same
//    registers: two workgroup barriers per chunk.
constexpr int kDeltaChunk = 32;
constexpr int kDeltaChunkRows = 16;  // state rows per workgroup of k_delta_chunk

// Record of one (sequence, value head, chunk), in floats: U [32][dk] | Q' [32][dk] |
// kh^T [dk][32] | Vb [32][dv] | O' [32][dv] | exp(G_last - G_s) [32], exp(G_last), pad [31].
__host__ __device__ constexpr size_t delta_rec_floats(int dk, int dv) {
  return 3 * (size_t)kDeltaChunk * dk + 2 * (size_t)kDeltaChunk * dv + 64;
}

// LDS writes of one wave made visible to its own later reads, with no workgroup barrier
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int DK>
__global__ __launch_bounds__(256) void k_delta_prep(DeltaArgs a, float* __restrict__ ws, int nchunks) {
  constexpr int C = kDeltaChunk;
  constexpr int KP = DK + 4;             // padded LDS row of kh / qh
  constexpr int E = DK / 16;             // values per lane in the normalisation (16 lanes a token)
  static_assert(E % 4 == 0, "whole 4-value pieces");
  __shared__ __attribute__((aligned(16))) float kl[C * KP];
  __shared__ __attribute__((aligned(16))) float ql[C * KP];
  constexpr int LD = C + 1;              // LDS row of the 32 x 32 matrices read by columns
  constexpr int TP = C + 4;              // LDS row of T and P, read in 16-byte pieces
  __shared__ float Ml[C * LD];           // M of the chunk (strictly lower triangular)
  __shared__ __attribute__((aligned(16))) float Tl[C * TP];  // (I + M)^-1, built block by block
  __shared__ __attribute__((aligned(16))) float Pl[C * TP];  // P (lower triangular)
  __shared__ float Xl[2][C * LD];        // the dot products' second halves
  __shared__ __attribute__((aligned(16))) float Sw[4][C * TP];  // per wave: a 32 x 32 result,
                                                                // transposed, on its way to a B operand
  __shared__ float Wl[16 * 16];
  __shared__ float Gs[C], bl[C], gam[C];
  __shared__ __attribute__((aligned(16))) float bgl[C];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = blockIdx.x, c = blockIdx.y, b = blockIdx.z;
  const int i = j / (a.Hv / a.Hk);
  const int t0 = c * C, n = min(C, a.T - t0);
  const int dv = a.dv;
  float* rec = ws + (((size_t)b * a.Hv + j) * nchunks + c) * delta_rec_floats(DK, dv);
  const size_t oQ = (size_t)C * DK, oKT = 2 * oQ, oVB = 3 * oQ, oOB = oVB + (size_t)C * dv,
               oSC = oOB + (size_t)C * dv;
  // g and beta of the chunk's tokens (lanes 0..31 of wave 0), requested first
  const bool gvalid = wave == 0 && lane < n;
  const size_t gi = ((size_t)b * a.T + t0 + (gvalid ? lane : 0)) * a.Hv + j;
  float G = gvalid ? a.g[gi] : 0.0f;
  const float bv = gvalid ? a.beta[gi] : 0.0f;

  // v of this wave's first 32 state rows (lane l: row 32 w + l % 32, tokens 16 (l / 32) + jj),
  // requested now and used after the inverse
  const int vm = lane & 31, vhs = lane >> 5;
  uint16_t vr[16];
  auto load_v = [&](int vt) __attribute__((always_inline)) {
    const int r = min(32 * vt + vm, a.dv - 1);
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      const int t = min(t0 + 16 * vhs + jj, a.T - 1);
      vr[jj] = a.v[(((size_t)b * a.T + t) * a.Hv + j) * a.dv + r];
    }
  };
  load_v(wave);
  for (int e = tid; e < C * TP; e += 256) Tl[e] = 0.0f;  // the inverse is zero above its diagonal
  // normalised keys and queries: 16 lanes per token, tokens wave*8 + 4*pass + lane/16; both
  // passes' raw bf16 words are requested before any is converted
  const int sc = lane & 15;
  uint2 kw[2][E / 4], qw[2][E / 4];
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int tt = min(t0 + wave * 8 + 4 * pass + (lane >> 4), a.T - 1);
    const size_t base = (((size_t)b * a.T + tt) * a.Hk + i) * DK + E * sc;
#pragma unroll
    for (int e = 0; e < E / 4; ++e) {
      kw[pass][e] = *reinterpret_cast<const uint2*>(a.k + base + 4 * e);
      qw[pass][e] = *reinterpret_cast<const uint2*>(a.q + base + 4 * e);
    }
  }
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int t = wave * 8 + 4 * pass + (lane >> 4);
    float4 kf[E / 4], qf[E / 4];
    float kk = 0.0f, qq = 0.0f;
#pragma unroll
    for (int e = 0; e < E / 4; ++e) {
      kf[e] = bf16x4_to_f32(kw[pass][e]);
      qf[e] = bf16x4_to_f32(qw[pass][e]);
      kk += dot4(kf[e], kf[e]);
      qq += dot4(qf[e], qf[e]);
    }
    kk = lane_group_sum<16>(kk);
    qq = lane_group_sum<16>(qq);
    const bool valid = t < n;
    const float nk = valid ? 1.0f / sqrtf(kk + a.eps) : 0.0f;
    const float nq = valid ? a.scale / sqrtf(qq + a.eps) : 0.0f;
#pragma unroll
    for (int e = 0; e < E / 4; ++e) {
      *reinterpret_cast<float4*>(kl + t * KP + E * sc + 4 * e) =
          make_float4(kf[e].x * nk, kf[e].y * nk, kf[e].z * nk, kf[e].w * nk);
      *reinterpret_cast<float4*>(ql + t * KP + E * sc + 4 * e) =
          make_float4(qf[e].x * nq, qf[e].y * nq, qf[e].z * nq, qf[e].w * nq);
    }
  }
  // running sums of g over the chunk (lanes 0..31 of wave 0)
  if (wave == 0) {
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) {
      const float up = __shfl_up(G, o, 64);
      if ((lane & 31) >= o) G += up;
    }
    if (lane < C) {
      Gs[lane] = G;
      bl[lane] = bv;
      gam[lane] = __expf(G);
      bgl[lane] = bv * __expf(G);
    }
  }
  __syncthreads();
  // kh_s . kh_r (waves 0, 1) and qh_s . kh_r (waves 2, 3) on v_mfma_f32_32x32x2_f32, each wave
  // over one half of the key dimension. Lane l holds row l & 31 of both operands; of each
  // 8-column piece it holds columns 4 * (l >> 5) .. + 3, which four MFMAs take in turn (both
  // operands pair the same columns, so every column enters the sums once).
  {
    const float* A = (wave >> 1) ? ql : kl;
    const int kh = (wave & 1) * (DK / 2), m = lane & 31, hs = lane >> 5;
    f32x16_t acc = {};
#pragma unroll
    for (int p = 0; p < DK / 16; ++p) {
      const f32x4_t av = *reinterpret_cast<const f32x4_t*>(A + m * KP + kh + 8 * p + 4 * hs);
      const f32x4_t bv = *reinterpret_cast<const f32x4_t*>(kl + m * KP + kh + 8 * p + 4 * hs);
#pragma unroll
      for (int u = 0; u < 4; ++u) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[u], bv[u], acc, 0, 0, 0);
    }
    // result register i of lane l: row 8 (i / 4) + 4 (l / 32) + i % 4, column l % 32
    float* part = Xl[wave >> 1];
    if (wave & 1) {
#pragma unroll
      for (int i = 0; i < 16; ++i) part[(8 * (i >> 2) + 4 * hs + (i & 3)) * LD + m] = acc[i];
    }
    __syncthreads();
    if (!(wave & 1)) {  // column r = m of rows s2(i); every LDS read first, then no branches
      float pv[16], gs[16], bs[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int s2 = 8 * (i >> 2) + 4 * hs + (i & 3);
        pv[i] = part[s2 * LD + m];
        gs[i] = Gs[s2];
        bs[i] = bl[s2];
      }
      const float gr = Gs[m];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int s2 = 8 * (i >> 2) + 4 * hs + (i & 3);
        const float v = (acc[i] + pv[i]) * __expf(gs[i] - gr);  // used only where r <= s2
        if (wave == 0) Ml[s2 * LD + m] = m < s2 ? bs[i] * v : 0.0f;
        else Pl[s2 * TP + m] = m <= s2 ? v : 0.0f;
      }
    }
    __syncthreads();
  }
  // T = (I + M)^-1, blocked: the four 8 x 8 diagonal blocks by forward substitution (lane
  // 8b + c solves column c of block b), then [[A, 0], [B, D]]^-1 = [[A^-1, 0], [-D^-1 B A^-1,
  // D^-1]] on pairs of 8 x 8 blocks and then on the two 16 x 16 halves.
  if (tid < C) {
    const int b8 = tid & ~7, c8 = tid & 7;
    float tc[8];
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2) {
      float acc = s2 == c8 ? 1.0f : 0.0f;
#pragma unroll
      for (int r = 0; r < s2; ++r) acc = __builtin_fmaf(-Ml[(b8 + s2) * LD + b8 + r], tc[r], acc);
      tc[s2] = acc;
    }
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2) Tl[(b8 + s2) * TP + b8 + c8] = tc[s2];
  }
  __syncthreads();
  const int pq = tid >> 6, i8 = (tid >> 3) & 7, j8 = tid & 7, o8 = 16 * pq;
  if (tid < 128) {  // W = M_10 T_00 of the pair of blocks starting at row o8
    float w = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) w = __builtin_fmaf(Ml[(o8 + 8 + i8) * LD + o8 + k], Tl[(o8 + k) * TP + o8 + j8], w);
    Wl[pq * 64 + i8 * 8 + j8] = w;
  }
  __syncthreads();
  if (tid < 128) {  // T_10 = -T_11 W
    float t = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) t = __builtin_fmaf(Tl[(o8 + 8 + i8) * TP + o8 + 8 + k], Wl[pq * 64 + k * 8 + j8], t);
    Tl[(o8 + 8 + i8) * TP + o8 + j8] = -t;
  }
  __syncthreads();
  const int i16 = tid >> 4, j16 = tid & 15;
  {  // the same on the two halves of 16 rows
    float w = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) w = __builtin_fmaf(Ml[(16 + i16) * LD + k], Tl[k * TP + j16], w);
    Wl[i16 * 16 + j16] = w;
  }
  __syncthreads();
  {
    float t = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) t = __builtin_fmaf(Tl[(16 + i16) * TP + 16 + k], Wl[k * 16 + j16], t);
    Tl[(16 + i16) * TP + j16] = -t;
  }
  __syncthreads();
  // U = T diag(beta gamma) Kh, then Q' = diag(gamma) Qh - P U, 32 columns per wave at a time on
  // v_mfma_f32_32x32x2_f32. Step j of 16 takes k = 16 (l / 32) + j: lane l supplies T[l % 32][k]
  // (or P) and the k-th row's entry in column l % 32 (the intermediate products are kept
  // transposed, so both operands are read as 16-byte pieces); result register i of lane l is row
  // 8 (i / 4) + 4 (l / 32) + i % 4, column l % 32.
  const int m = lane & 31, hs = lane >> 5;
  f32x4_t ta[4], pa[4], bg[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    ta[q] = *reinterpret_cast<const f32x4_t*>(Tl + m * TP + 16 * hs + 4 * q);
    pa[q] = *reinterpret_cast<const f32x4_t*>(Pl + m * TP + 16 * hs + 4 * q);
    bg[q] = *reinterpret_cast<const f32x4_t*>(bgl + 16 * hs + 4 * q);
  }
  float* sw = Sw[wave];
  // a 32 x 32 result into sw transposed: register 4g + x is row 8g + 4 (l / 32) + x, column l % 32
  auto stash_t = [&](const f32x16_t& u) __attribute__((always_inline)) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4)
      *reinterpret_cast<f32x4_t*>(sw + m * TP + 8 * g4 + 4 * hs) =
          f32x4_t{u[4 * g4], u[4 * g4 + 1], u[4 * g4 + 2], u[4 * g4 + 3]};
  };
  for (int ct = wave; ct < DK / 32; ct += 4) {
    const int c0 = 32 * ct;
    f32x4_t kt[4];  // kh[16 (l / 32) + 4q .. + 3][c0 + l % 32], which is also its record row
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int x = 0; x < 4; ++x) kt[q][x] = kl[(16 * hs + 4 * q + x) * KP + c0 + m];
      *reinterpret_cast<f32x4_t*>(rec + oKT + (size_t)(c0 + m) * C + 16 * hs + 4 * q) = kt[q];
    }
    f32x16_t u = {};
#pragma unroll
    for (int jj = 0; jj < 16; ++jj)
      u = __builtin_amdgcn_mfma_f32_32x32x2f32(ta[jj >> 2][jj & 3], bg[jj >> 2][jj & 3] * kt[jj >> 2][jj & 3],
                                              u, 0, 0, 0);
    stash_t(u);
    f32x16_t y;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int s2 = 8 * (i >> 2) + 4 * hs + (i & 3);
      rec[(size_t)s2 * DK + c0 + m] = u[i];
      y[i] = gam[s2] * ql[s2 * KP + c0 + m];
    }
    wave_lds_sync();
    f32x4_t ub[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) ub[q] = *reinterpret_cast<const f32x4_t*>(sw + m * TP + 16 * hs + 4 * q);
#pragma unroll
    for (int jj = 0; jj < 16; ++jj)
      y = __builtin_amdgcn_mfma_f32_32x32x2f32(-pa[jj >> 2][jj & 3], ub[jj >> 2][jj & 3], y, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) rec[oQ + (size_t)(8 * (i >> 2) + 4 * hs + (i & 3)) * DK + c0 + m] = y[i];
    wave_lds_sync();  // sw is rewritten by the next block
  }
  // Vb = T diag(beta) V and O' = P Vb, 32 state rows per wave at a time (rows past dv are zero
  // and not stored)
  for (int vt = wave; vt < (dv + 31) / 32; vt += 4) {
    const int r = 32 * vt + m;
    const bool rok = r < dv;
    if (vt != wave) load_v(vt);
    f32x16_t u = {};
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      const int k = 16 * hs + jj;  // beta is zero past the last token
      u = __builtin_amdgcn_mfma_f32_32x32x2f32(ta[jj >> 2][jj & 3], rok ? bl[k] * bf16_to_f32(vr[jj]) : 0.0f,
                                              u, 0, 0, 0);
    }
    stash_t(u);
    if (rok) {
#pragma unroll
      for (int i = 0; i < 16; ++i) rec[oVB + (size_t)(8 * (i >> 2) + 4 * hs + (i & 3)) * dv + r] = u[i];
    }
    wave_lds_sync();
    f32x4_t ub[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) ub[q] = *reinterpret_cast<const f32x4_t*>(sw + m * TP + 16 * hs + 4 * q);
    f32x16_t y = {};
#pragma unroll
    for (int jj = 0; jj < 16; ++jj)
      y = __builtin_amdgcn_mfma_f32_32x32x2f32(pa[jj >> 2][jj & 3], ub[jj >> 2][jj & 3], y, 0, 0, 0);
    if (rok) {
#pragma unroll
      for (int i = 0; i < 16; ++i) rec[oOB + (size_t)(8 * (i >> 2) + 4 * hs + (i & 3)) * dv + r] = y[i];
    }
    wave_lds_sync();
  }
  // the decays
  if (tid < C) rec[oSC + tid] = tid < n ? __expf(Gs[n - 1] - Gs[tid]) : 0.0f;
  if (tid == 0) rec[oSC + C] = __expf(Gs[n - 1]);
}

template <int DK>
constexpr int delta_chunk_waves() { return DK / 16 < 8 ? DK / 16 : 8; }

// One chunk's record entries held by a lane of k_delta_chunk
template <int NTL, int NPR>
struct DeltaChunkRegs {
  f32x4_t ua[NTL][2], qa[NTL][2];  // U and Q': rows 16 h + l % 16, columns c0 + 4 (l / 16) .. + 3
  f32x4_t kt[NTL][2];              // kh^T: column c0 + l % 16, tokens 8 (l / 16) .. + 7
  float vb[NPR], ob[NPR], dc[NPR];  // Vb, O' and the decay of this thread's (token, row) pairs
  float gl;                         // exp(G_last)
};

template <int DK>
__global__ __launch_bounds__(64 * delta_chunk_waves<DK>()) void k_delta_chunk(DeltaArgs a, const float* __restrict__ ws,
                                                                             int nchunks) {
  constexpr int C = kDeltaChunk, RW = kDeltaChunkRows;
  constexpr int NW = delta_chunk_waves<DK>();   // wave w owns state columns [w*DK/NW, (w+1)*DK/NW)
  constexpr int NTH = 64 * NW;
  constexpr int NTL = DK / 16 / NW;             // 16-column state tiles per wave
  constexpr int CP = C + 4;                     // LDS row of W ([row][token])
  constexpr int NPR = RW * C / NTH;             // (token, row) pairs per thread
  static_assert(RW == 16 && NTL >= 1 && NPR >= 1 && RW * C % NTH == 0, "16 rows, whole tiles");
  __shared__ float part[NW][2][C * RW];  // each wave's share of U S0^T and Q' S0^T, [token][row]
  __shared__ __attribute__((aligned(16))) float Wt[RW * CP];  // exp(G_last - G_s) delta, [row][token]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = blockIdx.x, b = blockIdx.z, r0 = blockIdx.y * RW;
  const int m16 = lane & 15, q4 = lane >> 4;
  const int dv = a.dv;
  const size_t RF = delta_rec_floats(DK, dv);
  const size_t oQ = (size_t)C * DK, oKT = 2 * oQ, oVB = 3 * oQ, oOB = oVB + (size_t)C * dv,
               oSC = oOB + (size_t)C * dv;

  // The state in the accumulator layout of v_mfma_f32_16x16x4_f32, as S^T tiles [column][row]:
  // register i of lane l in tile u holds S[r0 + l % 16][c0 + 4 (l / 16) + i], c0 = 16 (w NTL + u).
  f32x4_t st[NTL];
#pragma unroll
  for (int u = 0; u < NTL; ++u) {
    const int c0 = 16 * (wave * NTL + u);
    const size_t src = (((size_t)b * a.Hv + j) * dv + r0 + m16) * DK + c0 + 4 * q4;
    st[u] = a.s_in ? *reinterpret_cast<const f32x4_t*>(a.s_in + src) : f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  using Regs = DeltaChunkRegs<NTL, NPR>;
  auto fetch = [&](int cc, Regs& R) __attribute__((always_inline)) {
    const float* rec = ws + (((size_t)b * a.Hv + j) * nchunks + cc) * RF;
#pragma unroll
    for (int u = 0; u < NTL; ++u) {
      const int c0 = 16 * (wave * NTL + u);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        R.ua[u][h] = *reinterpret_cast<const f32x4_t*>(rec + (size_t)(16 * h + m16) * DK + c0 + 4 * q4);
        R.qa[u][h] = *reinterpret_cast<const f32x4_t*>(rec + oQ + (size_t)(16 * h + m16) * DK + c0 + 4 * q4);
        R.kt[u][h] = *reinterpret_cast<const f32x4_t*>(rec + oKT + (size_t)(c0 + m16) * C + 8 * q4 + 4 * h);
      }
    }
#pragma unroll
    for (int e = 0; e < NPR; ++e) {
      const int p = tid + NTH * e, s2 = p / RW, r = p % RW;
      R.vb[e] = rec[oVB + (size_t)s2 * dv + r0 + r];
      R.ob[e] = rec[oOB + (size_t)s2 * dv + r0 + r];
      R.dc[e] = rec[oSC + s2];
    }
    R.gl = rec[oSC + C];
  };
  auto body = [&](int cc, const Regs& R) __attribute__((always_inline)) {
    const int t0 = cc * C;
    // U S0^T and Q' S0^T over this wave's columns, two 16-token tiles each: lanes l / 16 = 0..3
    // supply columns c0 + 4 (l / 16) + i in step i, the same columns their state registers hold
    f32x4_t ad[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    f32x4_t ao[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int u = 0; u < NTL; ++u) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ad[h] = __builtin_amdgcn_mfma_f32_16x16x4f32(R.ua[u][h][i], st[u][i], ad[h], 0, 0, 0);
          ao[h] = __builtin_amdgcn_mfma_f32_16x16x4f32(R.qa[u][h][i], st[u][i], ao[h], 0, 0, 0);
        }
      }
    }
    // result register i of lane l: token 16 h + 4 (l / 16) + i, row l % 16
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        part[wave][0][(16 * h + 4 * q4 + i) * RW + m16] = ad[h][i];
        part[wave][1][(16 * h + 4 * q4 + i) * RW + m16] = ao[h][i];
      }
    }
    __syncthreads();
    // delta = Vb - U S0^T and o = O' + Q' S0^T, the waves' shares added in wave order
#pragma unroll
    for (int e = 0; e < NPR; ++e) {
      const int p = tid + NTH * e, s2 = p / RW, r = p % RW;
      float x = 0.0f, y = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        x += part[w][0][p];
        y += part[w][1][p];
      }
      if (t0 + s2 < a.T) a.o[(((size_t)b * a.T + t0 + s2) * a.Hv + j) * dv + r0 + r] = R.ob[e] + y;
      Wt[r * CP + s2] = R.dc[e] * (R.vb[e] - x);
    }
    __syncthreads();
    // S^T = exp(G_last) S0^T + kh^T W on the state tiles: A = kh^T [column][token], B = W
    // [token][row]; lanes l / 16 = 0..3 supply tokens 8 (l / 16) + k in step k
#pragma unroll
    for (int u = 0; u < NTL; ++u) {
      st[u] *= R.gl;
#pragma unroll
      for (int k = 0; k < 8; ++k)
        st[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(R.kt[u][k >> 2][k & 3], Wt[m16 * CP + 8 * q4 + k],
                                                     st[u], 0, 0, 0);
    }
  };
  // two register sets, so that a chunk's entries are requested while the previous one runs;
  // the requests are unconditional (past the end they repeat the last chunk's), so that the
  // wait before each chunk counts only the other set's requests (three sets, two chunks
  // ahead, were no faster)
  Regs ra, rb;
  fetch(0, ra);
  for (int cc = 0;; cc += 2) {
    fetch(min(cc + 1, nchunks - 1), rb);
    body(cc, ra);
    if (cc + 1 >= nchunks) break;
    fetch(min(cc + 2, nchunks - 1), ra);
    body(cc + 1, rb);
    if (cc + 2 >= nchunks) break;
  }
#pragma unroll
  for (int u = 0; u < NTL; ++u) {
    const int c0 = 16 * (wave * NTL + u);
    const size_t dst = (((size_t)b * a.Hv + j) * dv + r0 + m16) * DK + c0 + 4 * q4;
    *reinterpret_cast<f32x4_t*>(a.s_out + dst) = st[u];
  }
}

}  // namespace moe

using namespace moe;

namespace {

// Checks shared by both entry points; T = 0 passes the state through. Returns MOE_OK with
// *done = false when the caller should launch its kernels.
int delta_prologue(const delta_rule_desc_t* desc, const uint16_t* q, const uint16_t* k,
                   const uint16_t* v, const float* g, const float* beta, const float* state_in,
                   float* state_out, float* o, int32_t batch, int32_t T, hipStream_t s, bool* done) {
  *done = true;
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
  if (T == 0) {  // no token: the state passes through (a zero state if none is given)
    const size_t n = (size_t)batch * Hv * dv * dk;
    if (state_in == state_out) return MOE_OK;
    if (state_in)
      return hipMemcpyAsync(state_out, state_in, n * 4, hipMemcpyDeviceToDevice, s) == hipSuccess
                 ? MOE_OK : MOE_HIP_ERROR;
    return launch_fill_zero(state_out, n, s) == hipSuccess ? MOE_OK : MOE_HIP_ERROR;
  }
  *done = false;
  return MOE_OK;
}

}  // namespace

extern "C" int delta_rule_forward(const delta_rule_desc_t* desc, const uint16_t* q,
                                  const uint16_t* k, const uint16_t* v, const float* g,
                                  const float* beta, const float* state_in, float* state_out,
                                  float* o, int32_t batch, int32_t T, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  bool done;
  const int st = delta_prologue(desc, q, k, v, g, beta, state_in, state_out, o, batch, T, s, &done);
  if (done) return st;
  const int Hk = desc->num_k_heads, Hv = desc->num_v_heads, dk = desc->dk, dv = desc->dv;
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

extern "C" size_t delta_rule_chunked_workspace_bytes(const delta_rule_desc_t* desc,
                                                     int32_t batch, int32_t T) {
  if (!desc || batch <= 0 || T <= 0 || desc->num_v_heads <= 0 || desc->dv <= 0) return 0;
  const int dk = desc->dk;
  if (dk != 64 && dk != 128 && dk != 256) return 0;
  const size_t nch = ((size_t)T + kDeltaChunk - 1) / kDeltaChunk;
  return (size_t)batch * desc->num_v_heads * nch * delta_rec_floats(dk, desc->dv) * sizeof(float);
}

extern "C" int delta_rule_forward_chunked(const delta_rule_desc_t* desc, const uint16_t* q,
                                          const uint16_t* k, const uint16_t* v, const float* g,
                                          const float* beta, const float* state_in,
                                          float* state_out, float* o, int32_t batch, int32_t T,
                                          void* workspace, size_t ws_bytes, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  bool done;
  const int st = delta_prologue(desc, q, k, v, g, beta, state_in, state_out, o, batch, T, s, &done);
  if (done) return st;
  if (!workspace || ((uintptr_t)workspace & 15)) return MOE_INVALID_ARG;
  if (ws_bytes < delta_rule_chunked_workspace_bytes(desc, batch, T)) return MOE_WORKSPACE_TOO_SMALL;
  const int Hk = desc->num_k_heads, Hv = desc->num_v_heads, dk = desc->dk, dv = desc->dv;
  DeltaArgs a{q, k, v, g, beta, state_in, state_out, o, Hk, Hv, dv, T, desc->scale, desc->eps};
  float* ws = static_cast<float*>(workspace);
  const int nch = (T + kDeltaChunk - 1) / kDeltaChunk;
  const dim3 gp(Hv, nch, batch), gm(Hv, dv / kDeltaChunkRows, batch);
  if (dk == 64) {
    hipLaunchKernelGGL((k_delta_prep<64>), gp, dim3(256), 0, s, a, ws, nch);
    hipLaunchKernelGGL((k_delta_chunk<64>), gm, dim3(64 * delta_chunk_waves<64>()), 0, s, a, ws, nch);
  } else if (dk == 128) {
    hipLaunchKernelGGL((k_delta_prep<128>), gp, dim3(256), 0, s, a, ws, nch);
    hipLaunchKernelGGL((k_delta_chunk<128>), gm, dim3(64 * delta_chunk_waves<128>()), 0, s, a, ws, nch);
  } else {
    hipLaunchKernelGGL((k_delta_prep<256>), gp, dim3(256), 0, s, a, ws, nch);
    hipLaunchKernelGGL((k_delta_chunk<256>), gm, dim3(64 * delta_chunk_waves<256>()), 0, s, a, ws, nch);
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_HIP_ERROR;
}
