// Router: logits, top-k with softmax renormalisation, shared-expert sigmoid gate, counts.
//
// "Perplexity's Lily: A Breakthrough Local Inference Engine Tailored Exclusively for Apple
// Silicon", section "The Model: Qwen3.6-35B-A3B in Focus": a router scores 256 experts per
// token and selects eight; one shared expert processes every token.
//
// Prefill logits run on bf16 MFMA: x is exact in bf16 and each fp32 router weight is split
// into three bf16 parts w = hi + mid + lo (together all 24 significant bits), so x.w is formed
// from exact bf16 products with fp32 accumulation -- the accuracy of an fp32 dot product, at
// MFMA speed (the split follows Henry, Tang and Heinecke, "Leveraging the bfloat16 artificial
// intelligence datatype for higher-precision computations", ARITH 2019). Decode logits
// (few tokens, bandwidth-bound) use fp32 FMA directly on the fp32 weights.
#include "moe_internal.h"

namespace moe {

// ------------------------------------------------------------ prefill logits (MFMA)
// WG = 4 waves = 64 tokens x 64 experts; each wave a 32x32 tile on v_mfma_f32_32x32x16_bf16.
// Per K-chunk of 64 inputs the workgroup stages x (bf16) and the fp32 router rows into LDS,
// splitting every weight into its three bf16 parts while storing (double-buffered, rows padded
// to 144 B). Lane l feeds row (l & 31) of its tile and inputs 8*(l >> 5) .. +7 of the 16-input
// step for both operands (any consistent split of K between the operands gives the same dot
// products). Per step the low, middle and high parts are accumulated in that order.
//
// The global loads run two chunks ahead of the MFMAs (two register sets), and the barrier
// between chunks waits only for the LDS stores, so the prefetch stays in flight across it.
// When there are few token tiles the inputs are split into S ranges (split-K), so that the
// chip has enough workgroups: split s writes its partial logits to slice s of an [S, T, E+1]
// array, and the top-k kernel adds the S slices in a fixed order.
// Workgroups are dispatched round-robin over the 8 XCDs; XCD i takes a contiguous range of
// tiles, so the expert tiles of one token tile (and split) read x through the same L2.
// The workgroups of the first expert tile also form the partial shared-expert gate logit
// x . wg in fp32 from the x chunks they hold in LDS (column E of the slice).
namespace {
constexpr int kRK = 64;        // inputs per K-chunk
constexpr int kRRow = kRK + 8; // padded LDS row (bf16 elements)
constexpr int kXcds = 8;
}  // namespace

// (v0, v1) -> three packed bf16 pairs whose sums are exact splits of v0 and v1.
__device__ __forceinline__ void split3(float v0, float v1, uint32_t& hi, uint32_t& mid,
                                       uint32_t& lo) {
  hi = pack_bf16x2(v0, v1);
  const float r0 = v0 - __uint_as_float(hi << 16);          // exact
  const float r1 = v1 - __uint_as_float(hi & 0xFFFF0000u);  // exact
  mid = pack_bf16x2(r0, r1);
  lo = pack_bf16x2(r0 - __uint_as_float(mid << 16), r1 - __uint_as_float(mid & 0xFFFF0000u));
}

__global__ __launch_bounds__(256, 2) void k_router_mfma(const uint16_t* __restrict__ x,
                                                        const float* __restrict__ w,
                                                        const float* __restrict__ bias,
                                                        const float* __restrict__ wg, int T,
                                                        int E, int H, int n_etiles,
                                                        int n_ttiles, int ntiles, int cps,
                                                        float* __restrict__ logits) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][64 * kRRow];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][3][64 * kRRow];
  __shared__ __attribute__((aligned(16))) float Gs[2][kRK];
  const int per = gridDim.x / kXcds;
  const int tile = (blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
  if (tile >= ntiles) return;  // whole workgroup, before any barrier
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int split = tile / (n_ttiles * n_etiles), rem = tile % (n_ttiles * n_etiles);
  const int t0 = (rem / n_etiles) * 64, e0 = (rem % n_etiles) * 64;
  const bool gate = wg != nullptr && e0 == 0;
  const float* wgp = wg != nullptr ? wg : w;  // loads stay unconditional; unused without a gate
  const int c0 = split * cps;                      // this split's first K-chunk
  const int nchunks = min(cps, H / kRK - c0);      // and its chunk count (>= 1)

  // one chunk's registers: x (64 rows x 8 segments of 8 bf16, two per thread), router rows
  // (64 rows x 16 float4, four per thread) and the shared gate weight k0 + (tid & 63)
  auto load = [&](bf16x8_t (&ra)[2], float4 (&rb)[4], float& rg, int c) {
    const int k0 = (c0 + min(c, nchunks - 1)) * kRK;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int v = tid + 256 * i, row = v >> 3, seg = v & 7;
      const int t = min(t0 + row, T - 1);
      ra[i] = *reinterpret_cast<const bf16x8_t*>(x + (size_t)t * H + k0 + seg * 8);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int v = tid + 256 * i, row = v >> 4, c4 = v & 15;
      const int e = min(e0 + row, E - 1);
      rb[i] = *reinterpret_cast<const float4*>(w + (size_t)e * H + k0 + c4 * 4);
    }
    rg = wgp[k0 + lane];
  };
  auto store = [&](const bf16x8_t (&ra)[2], const float4 (&rb)[4], float rg, int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int v = tid + 256 * i, row = v >> 3, seg = v & 7;
      *reinterpret_cast<bf16x8_t*>(&As[buf][row * kRRow + seg * 8]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int v = tid + 256 * i, row = v >> 4, c4 = v & 15;
      uint2 h, m, l;
      split3(rb[i].x, rb[i].y, h.x, m.x, l.x);
      split3(rb[i].z, rb[i].w, h.y, m.y, l.y);
      const int o = row * kRRow + c4 * 4;
      *reinterpret_cast<uint2*>(&Bs[buf][0][o]) = h;
      *reinterpret_cast<uint2*>(&Bs[buf][1][o]) = m;
      *reinterpret_cast<uint2*>(&Bs[buf][2][o]) = l;
    }
    if (wave == 0) Gs[buf][lane] = rg;
  };
  // LDS stores of this wave are complete, then the workgroup meets; outstanding global loads
  // (the prefetch) are not waited for: vmcnt 63 in bits 3:0 and 15:14, expcnt 7, lgkmcnt 0.
  auto barrier = [&]() {
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  const int r = lane & 31, half = lane >> 5;
  const int arow = (wave >> 1) * 32 + r, brow = (wave & 1) * 32 + r;
  const int grow = tid >> 2, gq = tid & 3;  // gate: token row, quarter of the chunk
  f32x16_t acc = {};
  float gacc = 0.0f;
  auto compute = [&](int buf) {
#pragma unroll
    for (int st = 0; st < kRK / 16; ++st) {
      const int ko = st * 16 + half * 8;
      const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(&As[buf][arow * kRRow + ko]);
      const bf16x8_t bl = *reinterpret_cast<const bf16x8_t*>(&Bs[buf][2][brow * kRRow + ko]);
      const bf16x8_t bm = *reinterpret_cast<const bf16x8_t*>(&Bs[buf][1][brow * kRRow + ko]);
      const bf16x8_t bh = *reinterpret_cast<const bf16x8_t*>(&Bs[buf][0][brow * kRRow + ko]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bl, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bm, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bh, acc, 0, 0, 0);
    }
    if (gate) {
      const uint4* xs = reinterpret_cast<const uint4*>(&As[buf][grow * kRRow + gq * 16]);
      const float4* gs = reinterpret_cast<const float4*>(&Gs[buf][gq * 16]);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint4 xv = xs[i];
        const float4 g0 = gs[2 * i], g1 = gs[2 * i + 1];
        gacc = __builtin_fmaf(bf16_to_f32(xv.x & 0xFFFFu), g0.x, gacc);
        gacc = __builtin_fmaf(bf16_to_f32(xv.x >> 16), g0.y, gacc);
        gacc = __builtin_fmaf(bf16_to_f32(xv.y & 0xFFFFu), g0.z, gacc);
        gacc = __builtin_fmaf(bf16_to_f32(xv.y >> 16), g0.w, gacc);
        gacc = __builtin_fmaf(bf16_to_f32(xv.z & 0xFFFFu), g1.x, gacc);
        gacc = __builtin_fmaf(bf16_to_f32(xv.z >> 16), g1.y, gacc);
        gacc = __builtin_fmaf(bf16_to_f32(xv.w & 0xFFFFu), g1.z, gacc);
        gacc = __builtin_fmaf(bf16_to_f32(xv.w >> 16), g1.w, gacc);
      }
    }
  };

  // LDS buffer c & 1 holds chunk c; the registers of chunk c + 1 are in flight meanwhile
  bf16x8_t xa0[2], xa1[2];
  float4 wb0[4], wb1[4];
  float g0, g1;
  load(xa0, wb0, g0, 0);
  load(xa1, wb1, g1, 1);
  store(xa0, wb0, g0, 0);
  barrier();
  int c = 0;
  for (; c + 1 < nchunks; c += 2) {
    load(xa0, wb0, g0, c + 2);
    compute(0);
    store(xa1, wb1, g1, 1);
    barrier();
    load(xa1, wb1, g1, c + 3);
    compute(1);
    store(xa0, wb0, g0, 0);
    barrier();
  }
  if (c < nchunks) compute(0);  // odd chunk count: the last chunk is in buffer 0
  // drain the clamped tail loads before the workgroup ends
  __builtin_amdgcn_s_waitcnt(0);

  const int ld = E + 1;
  float* slice = logits + (size_t)split * T * ld;
  if (gate) {
    gacc += __shfl_xor(gacc, 1, 64);
    gacc += __shfl_xor(gacc, 2, 64);
    const int t = t0 + grow;
    if (gq == 0 && t < T) slice[(size_t)t * ld + E] = gacc;
  }
  // D layout of the 32x32 tile: register i of lane l is row 8*(i/4) + 4*(l/32) + i%4,
  // column l%32. The bias goes into split 0 only.
  const int e = e0 + (wave & 1) * 32 + r;
  if (e >= E) return;
  const float bv = (bias != nullptr && split == 0) ? bias[e] : 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int t = t0 + (wave >> 1) * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
    if (t < T) slice[(size_t)t * ld + e] = acc[i] + bv;
  }
}

int router_splits(int T, int E, int H) {
  const int base = ((E + 63) / 64) * ((T + 63) / 64);
  const int nchunks = H / kRK;
  int S = 1;
  while (S < kRouterMaxSplits && base * S * 2 <= 512 && nchunks % (2 * S) == 0) S *= 2;
  return S;
}

hipError_t launch_router_logits_mfma(const uint16_t* x, const float* w, const float* bias,
                                     const float* wg, int T, int E, int H, float* logits,
                                     hipStream_t s) {
  const int S = router_splits(T, E, H);
  const int n_etiles = (E + 63) / 64, n_ttiles = (T + 63) / 64;
  const int ntiles = n_etiles * n_ttiles * S;
  const int grid = (ntiles + kXcds - 1) / kXcds * kXcds;
  hipLaunchKernelGGL(k_router_mfma, dim3(grid), dim3(256), 0, s, x, w, bias, wg, T, E, H,
                     n_etiles, n_ttiles, ntiles, (H / kRK) / S, logits);
  return hipGetLastError();
}

// -------------------------------------------------------------- decode logits (GEMV)
// One wave per expert row; each lane reads 16 B of the fp32 row per step (coalesced) and
// the matching 4 inputs of every token. T <= kDecodeMaxT. All of a lane's loads are issued
// before the first FMA (one memory round trip per row).
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
  constexpr int kU = TC <= 2 ? 8 : (TC <= 4 ? 4 : 2);  // units per lane per batch
  for (int u0 = 0; u0 < units; u0 += 64 * kU) {
    float4 wv[kU];
    uint2 xv[kU][TC];
#pragma unroll
    for (int i = 0; i < kU; ++i) {
      const int u = u0 + lane + 64 * i;
      wv[i] = u < units ? wr[u] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int t = 0; t < TC; ++t)
        xv[i][t] = (u < units && t < T) ? *reinterpret_cast<const uint2*>(x + (size_t)t * H + 4 * u)
                                        : make_uint2(0, 0);
    }
#pragma unroll
    for (int i = 0; i < kU; ++i) {
#pragma unroll
      for (int t = 0; t < TC; ++t) {
        acc[t] = __builtin_fmaf(bf16_to_f32(xv[i][t].x & 0xFFFFu), wv[i].x, acc[t]);
        acc[t] = __builtin_fmaf(bf16_to_f32(xv[i][t].x >> 16), wv[i].y, acc[t]);
        acc[t] = __builtin_fmaf(bf16_to_f32(xv[i][t].y & 0xFFFFu), wv[i].z, acc[t]);
        acc[t] = __builtin_fmaf(bf16_to_f32(xv[i][t].y >> 16), wv[i].w, acc[t]);
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
  else if (T <= 2)
    hipLaunchKernelGGL(k_router_gemv<2>, dim3(E), dim3(64), 0, s, x, w, bias, T, E, H, logits);
  else if (T <= 4)
    hipLaunchKernelGGL(k_router_gemv<4>, dim3(E), dim3(64), 0, s, x, w, bias, T, E, H, logits);
  else if (T <= 8)
    hipLaunchKernelGGL(k_router_gemv<8>, dim3(E), dim3(64), 0, s, x, w, bias, T, E, H, logits);
  else
    hipLaunchKernelGGL(k_router_gemv<16>, dim3(E), dim3(64), 0, s, x, w, bias, T, E, H, logits);
  return hipGetLastError();
}

// ------------------------------------------------------------------ top-k + gates
// One wave per token. Lane l holds logits e = NJ*l + j (the sum of the S split slices, added in
// slice order). K rounds of a wave arg-max ordered by (larger logit, then lower expert index)
// give the top-k in rank order; lane r keeps the rank-r winner. Weights: softmax over the
// selected logits, which equals a softmax over all experts renormalised over the selected
// ones. The shared expert's gate is sigmoid(x . wg): from column E of the slices when
// gate_col, otherwise formed here from x and wg (when wg is given).
template <int NJ>
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits, int S, int ld,
                                              int gate_col, const uint16_t* __restrict__ x,
                                              const float* __restrict__ wg, int T, int E, int K,
                                              int H, int32_t* __restrict__ idx,
                                              float* __restrict__ wout,
                                              float* __restrict__ sgate) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // no barriers in this kernel
  const size_t slice = (size_t)T * ld;
  const float* lt = logits + (size_t)t * ld;
  float v[NJ];
  load_logits<NJ>(lt, E, lane, v);
  for (int s = 1; s < S; ++s) {
    float u[NJ];
    load_logits<NJ>(lt + s * slice, E, lane, u);
#pragma unroll
    for (int j = 0; j < NJ; ++j) v[j] += u[j];
  }
  float my_v, my_w;
  int my_i;
  wave_topk_softmax<NJ>(v, E, K, lane, my_v, my_i, my_w);
  if (lane < K) {
    idx[(size_t)t * K + lane] = my_i;
    wout[(size_t)t * K + lane] = my_w;
  }
  if (gate_col) {
    if (lane == 0) {
      float g = lt[E];
      for (int s = 1; s < S; ++s) g += lt[s * slice + E];
      sgate[t] = 1.0f / (1.0f + __expf(-g));
    }
  } else if (wg != nullptr) {
    const float g = shared_gate_logit(x + (size_t)t * H, wg, H, lane);
    if (lane == 0) sgate[t] = 1.0f / (1.0f + __expf(-g));
  }
}

hipError_t launch_topk(const float* logits, int S, int ld, bool gate_col, const uint16_t* x,
                       const float* wg, int T, int E, int K, int H, int32_t* idx, float* w,
                       float* sgate, hipStream_t s) {
  const dim3 grid((T + 3) / 4);
  const int gc = gate_col ? 1 : 0;
#define MOE_TOPK(NJ)                                                                            \
  hipLaunchKernelGGL(k_topk<NJ>, grid, dim3(256), 0, s, logits, S, ld, gc, x, wg, T, E, K, H, \
                     idx, w, sgate)
  if (E <= 64)
    MOE_TOPK(1);
  else if (E <= 256)
    MOE_TOPK(4);
  else if (E <= 512)
    MOE_TOPK(8);
  else
    MOE_TOPK(16);
#undef MOE_TOPK
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
