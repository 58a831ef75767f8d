// Grouped-query decode attention over a block-paged KV cache, and its C ABI (attn_gqa.h).
//
// "Perplexity's Lily: A Breakthrough Local Inference Engine Tailored Exclusively for Apple
// Silicon": section "The Model: Qwen3.6-35B-A3B in Focus" (grouped-query attention, 16 query
// heads sharing two KV heads, over a growing key-value cache) and section "How It Works: Prefill
// and Decode Strategies" (coalesced key and value cache reads; GQA packing, i.e. the query heads
// of a KV head sharing its reads; a fixed-block cache layout). Decode attention reads every cached
// key and value once per token and is bound by HBM bandwidth; with G query heads packed per
// workgroup it does 2G multiply-adds per cached value, which for G = 8 keeps the VALUs about as
// busy as HBM. So packed workgroups run both products on MFMA (v_mfma_f32_16x16x32_bf16, the G
// heads as 16 columns): q.K per 16-token tile, 32 dimensions per step (exact bf16 products, fp32
// sums), and P.V per 16-dimension tile, 32 tokens per step, with the fp32 probabilities entering
// as two bf16 parts (hi = RNE(p), lo = RNE(p - hi)) so that about 16 of their significant bits
// take part; the softmax stays fp32 VALU work.
//
// Layout of the work (split over the context, then a merge):
//  * k_attn_split: one workgroup of 4 waves per (sequence, KV head, span of the context) with
//    all G query heads of that KV head (packed). A span is a run of chunks; a token's key row of
//    D bf16 is read by D/8 consecutive lanes, 16 bytes each, so one wave instruction reads whole
//    rows (64 * 16 bytes); the block table is read per token, so chunks may span blocks of any
//    placement (for MFMA scores a lane reads 16 bytes of a token row per MFMA step instead:
//    four lanes cover 64 contiguous bytes of each of 16 rows). Per chunk: scores to LDS, each
//    head's running maximum and the chunk's exponentials (fp32, online softmax: earlier sums are
//    rescaled by exp(m_old - m_new)), then P.V: on MFMA (packed) each wave owns D/4 dimensions
//    of every head, with the chunk's value rows staged in LDS; on VALU each lane accumulates 8
//    dimensions of the workgroup's heads, summed over lanes and waves at the end. A chunk is
//    sized so that every
//    lane requests all its key and value rows of the chunk at once, and the next chunk's keys
//    (values) are requested as soon as the current ones have been used, so a workgroup keeps a
//    chunk's rows in flight while it computes. The span's (max, sum, acc) per head is stored.
//    The spans are sized so that a set number of workgroups covers the call.
//  * k_attn_combine: per (sequence, query head, 32 of its dimensions), the spans' records are
//    merged, rescaled by exp(max_s - max): the first accumulator rows and every span's (max,
//    sum) are requested at once, then weights, then 8 lanes per record with 16-byte loads over
//    interleaved records (256 records per request round), summed over the lanes' partial sums
//    in a fixed order, so the output does not depend on scheduling.
#include <algorithm>
#include <cmath>

#include "attn_gqa.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kAttnThreads = 256;

// Split workgroups a call is spread over: 512 with packed heads (a packed workgroup does G
// heads' arithmetic per byte and already keeps the chip busy), 1024 with one head per workgroup.
constexpr int kAttnTargetWorkgroups = 512;
constexpr int kAttnTargetWorkgroupsUnpacked = 1024;
constexpr int kAttnMaxSpans = 1024;  // spans per (sequence, head): bounds the merge's LDS

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  const int32_t* table;
  const int32_t* lens;
  float* part;  // [B, Hq, nspans, D + 4]: max, sum, -, -, acc[D]
  float* out;   // [B, Hq, D]
  int Hq, Hkv, bs_shift, MB, nblocks, max_len;
  int span;     // tokens per span: a multiple of the chunk
  int nspans;   // spans of the longest sequence (the record stride)
  float scale;
};

__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// Sum over aligned groups of N lanes (N = 8, 16 or 32); every lane of a group ends with the
// group's total. Distances below 16 use DPP partners inside a row of 16 lanes.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 32) v += __shfl_xor(v, 16, 64);
  if constexpr (N >= 16) v += dpp_partner16<8>(v);
  v += dpp_partner16<4>(v);
  v += dpp_partner16<2>(v);
  v += dpp_partner16<1>(v);
  return v;
}

}  // namespace

// Tokens of one chunk: U wave-instruction steps of the workgroup, so that each lane requests all
// of its key and value rows of the chunk at once (one memory round trip per chunk). U = 8 for
// long contexts; when the long chunks would leave the grid short of workgroups, U = 4 for
// packed workgroups (64 tokens at D = 128, still whole 16-token MFMA tiles per wave) and U = 2
// otherwise.
template <int D, int U>
__host__ __device__ constexpr int attn_chunk() {
  return U * 4 * (64 / (D / 8));   // U steps of 4 waves x (64 / (D/8)) tokens
}

// HPW query heads per workgroup (G when packed, 1 when not); D head size; U steps per chunk.
template <int D, int HPW, int U>
__global__ __launch_bounds__(kAttnThreads) void k_attn_split(AttnArgs a) {
  constexpr int LPT = D / 8;     // lanes per token row (16 bytes each)
  constexpr int TPI = 64 / LPT;  // tokens per wave instruction
  constexpr int TPB = 4 * TPI;   // tokens per workgroup step
  constexpr int C = attn_chunk<D, U>();  // U steps: every row of a chunk requested up front
  // q.K on MFMA (16 x 16 x 32 bf16, HPW of the 16 columns used) for packed workgroups with
  // long chunks; the VALU dot products otherwise
  constexpr int NJ = D / 32;     // MFMAs per 16-token tile (32 dimensions each)
  constexpr bool kMM = HPW >= 4 && C % 64 == 0 && (C / 64) * NJ == U;  // same loads per lane
  // MFMA path: the chunk's value rows in LDS, row-major with a pitch of D + 4 bf16, so that the
  // transposed operand reads of P.V (8 rows apart per lane group) fall in distinct banks
  constexpr int VP = D + 4;
  __shared__ __attribute__((aligned(16))) float sc[HPW * C];       // scores, then probabilities
  __shared__ __attribute__((aligned(16))) float wacc[kMM ? 1 : 4 * HPW * D];  // per-wave sums
  __shared__ __attribute__((aligned(16))) uint16_t vl[kMM ? C * VP : 1];      // value rows
  __shared__ float st[3 * HPW];   // per head: running max, running sum, this chunk's rescale
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = blockIdx.z;
  const int h0 = blockIdx.y * HPW;           // first query head of the workgroup
  const int g = h0 / (a.Hq / a.Hkv);         // its KV head
  int len = a.lens[b];
  len = len < 0 ? 0 : (len > a.max_len ? a.max_len : len);
  const int t0 = blockIdx.x * a.span;
  const int t1 = min(len, t0 + a.span);      // this span: tokens [t0, t1)
  if (t1 <= t0) return;                      // past the sequence: the merge reads no record here

  const int dsl = lane % LPT, tsub = lane / LPT;
  const int32_t* trow = a.table + (size_t)b * a.MB;
  const int bs_mask = (1 << a.bs_shift) - 1;
  // this lane's 16 bytes of token j (j < t1)
  auto row = [&](const uint16_t* cache, int j) -> const uint4* {
    int blk = trow[j >> a.bs_shift];
    blk = blk < 0 ? 0 : (blk >= a.nblocks ? a.nblocks - 1 : blk);
    return reinterpret_cast<const uint4*>(
        cache + ((((size_t)blk * a.Hkv + g) << a.bs_shift) + (j & bs_mask)) * D + dsl * 8);
  };
  // token of step u of the chunk at c0, clamped into the span (the clamped rows are not used)
  auto tok = [&](int c0, int u) { return min(c0 + u * TPB + wave * TPI + tsub, t1 - 1); };
  // MFMA scores (kMM): wave w takes tokens [w*C/4, (w+1)*C/4) of a chunk as 16-token tiles;
  // key load u = tile * NJ + j is this lane's 16 bytes of token (lane % 16) of the tile at
  // dimensions 32j + 8*(lane / 16): the A operand of v_mfma_f32_16x16x32_bf16 (rows = tokens,
  // k = 32 dimensions), whose B operand is q^T (columns = the HPW heads, the rest zero).
  auto krow_mm = [&](int c0, int u) -> const uint4* {
    const int tt = u / NJ, j = u % NJ;
    const int jt = min(c0 + wave * (C / 4) + tt * 16 + (lane & 15), t1 - 1);
    int blk = trow[jt >> a.bs_shift];
    blk = blk < 0 ? 0 : (blk >= a.nblocks ? a.nblocks - 1 : blk);
    return reinterpret_cast<const uint4*>(
        a.kc + ((((size_t)blk * a.Hkv + g) << a.bs_shift) + (jt & bs_mask)) * D + 32 * j +
        8 * (lane >> 4));
  };
  auto krow = [&](int c0, int u) -> const uint4* {
    if constexpr (kMM) return krow_mm(c0, u);
    else return row(a.kc, tok(c0, u));
  };
  uint4 kv[U], vv[U];
#pragma unroll
  for (int u = 0; u < U; ++u) kv[u] = load_nt(krow(t0, u));
#pragma unroll
  for (int u = 0; u < U; ++u) vv[u] = load_nt(row(a.vc, tok(t0, u)));
  uint4 qv[kMM ? NJ : HPW];
  if constexpr (kMM) {
    const int hq = lane & 15;  // B operand: head hq, dimensions 32j + 8*(lane / 16) .. + 8
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      qv[j] = hq < HPW ? *reinterpret_cast<const uint4*>(a.q + ((size_t)b * a.Hq + h0 + hq) * D +
                                                         32 * j + 8 * (lane >> 4))
                       : make_uint4(0u, 0u, 0u, 0u);
  } else {
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh)
      qv[hh] = *reinterpret_cast<const uint4*>(a.q + ((size_t)b * a.Hq + h0 + hh) * D + dsl * 8);
  }
  if (tid < HPW) {
    st[tid] = -INFINITY;
    st[HPW + tid] = 0.0f;
  }
  // VALU P.V: 8 dimensions of the HPW heads per lane. MFMA P.V: the wave's D/64 tiles of 16
  // dimensions, O^T[dim][head] (lane l: head l % 16, dimensions 4*(l / 16) + i of the tile)
  constexpr int ND = kMM ? D / 64 : 1;
  float acc[kMM ? 1 : HPW][8];
  f32x4_t oacc[ND];
  if constexpr (kMM) {
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) oacc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  } else {
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[hh][e] = 0.0f;
  }

  for (int c0 = t0; c0 < t1; c0 += C) {
    const int n = min(C, t1 - c0);           // tokens of this chunk
    const bool more = c0 + C < t1;
    // ---- scores: q_h . k_j for the chunk's tokens, scaled
    if constexpr (kMM) {
      // D[token][head] of each 16-token tile: lane l holds head l % 16 for tokens
      // 4*(l / 16) + i of the tile, i < 4
#pragma unroll
      for (int tt = 0; tt < C / 64; ++tt) {
        f32x4_t d4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          d4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kv[tt * NJ + j]),
                                                       __builtin_bit_cast(bf16x8_t, qv[j]), d4, 0, 0, 0);
        const int hq = lane & 15;
        const int s0 = wave * (C / 4) + tt * 16 + 4 * (lane >> 4);
        if (hq < HPW) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (s0 + i < n) sc[hq * C + s0 + i] = d4[i] * a.scale;
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int s = u * TPB + wave * TPI + tsub;
        float t[HPW];
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) {
          float d = dot2_bf16(kv[u].x, qv[hh].x, 0.0f);
          d = dot2_bf16(kv[u].y, qv[hh].y, d);
          d = dot2_bf16(kv[u].z, qv[hh].z, d);
          d = dot2_bf16(kv[u].w, qv[hh].w, d);
          t[hh] = group_sum<LPT>(d);
        }
        float val = 0.0f;
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh)
          if (dsl == hh) val = t[hh];
        if (s < n && dsl < HPW) sc[dsl * C + s] = val * a.scale;
      }
    }
    if (more) {   // the keys are used: request the next chunk's
#pragma unroll
      for (int u = 0; u < U; ++u) kv[u] = load_nt(krow(c0 + C, u));
    }
    if constexpr (kMM) {  // the value rows to LDS, then the next chunk's requested
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int s = u * TPB + wave * TPI + tsub;
        uint2* dst = reinterpret_cast<uint2*>(vl + s * VP + dsl * 8);
        dst[0] = make_uint2(vv[u].x, vv[u].y);
        dst[1] = make_uint2(vv[u].z, vv[u].w);
      }
      if (more) {
#pragma unroll
        for (int u = 0; u < U; ++u) vv[u] = load_nt(row(a.vc, tok(c0 + C, u)));
      }
    }
    __syncthreads();

    // ---- per head: new running maximum, exponentials (kept in place), sums
    for (int hh = wave; hh < HPW; hh += 4) {
      float* sh = sc + hh * C;
      float m = -INFINITY;
      for (int i = lane; i < n; i += 64) m = fmaxf(m, sh[i]);
      m = fmaxf(wave_max_f(m), st[hh]);
      float l = 0.0f;
      for (int i = lane; i < n; i += 64) {
        const float p = __expf(sh[i] - m);
        sh[i] = p;
        l += p;
      }
      l = wave_sum(l);
      if (lane == 0) {
        const float f = __expf(st[hh] - m);  // 0 for the first chunk (old max -inf)
        st[hh] = m;
        st[HPW + hh] = __builtin_fmaf(st[HPW + hh], f, l);
        st[2 * HPW + hh] = f;
      }
    }
    __syncthreads();

    if constexpr (kMM) {
      // ---- P.V on MFMA: O^T[dim][head] += V^T[dim][tokens] P^T[tokens][head] over 32-token
      // blocks; P (fp32) enters as two bf16 parts, hi = RNE(p) and lo = RNE(p - hi), so that the
      // products keep about 16 significant bits of p
      const int hq = lane & 15;
      const float f = hq < HPW ? st[2 * HPW + hq] : 0.0f;
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) oacc[dt] *= f;
#pragma unroll
      for (int tb = 0; tb < C / 32; ++tb) {
        const int t8 = tb * 32 + 8 * (lane >> 4);   // this lane's 8 tokens of the block
        uint32_t ph[4], pl[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float p0 = 0.0f, p1 = 0.0f;
          if (hq < HPW) {
            p0 = t8 + 2 * e < n ? sc[hq * C + t8 + 2 * e] : 0.0f;
            p1 = t8 + 2 * e + 1 < n ? sc[hq * C + t8 + 2 * e + 1] : 0.0f;
          }
          ph[e] = pack_bf16x2(p0, p1);
          pl[e] = pack_bf16x2(p0 - bf16_to_f32(ph[e] & 0xFFFFu), p1 - bf16_to_f32(ph[e] >> 16));
        }
        const bf16x8_t bh = __builtin_bit_cast(bf16x8_t, make_uint4(ph[0], ph[1], ph[2], ph[3]));
        const bf16x8_t bl = __builtin_bit_cast(bf16x8_t, make_uint4(pl[0], pl[1], pl[2], pl[3]));
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) {
          const int dim = (wave * ND + dt) * 16 + hq;   // A operand: row = this dimension
          uint32_t vw[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            vw[e] = (uint32_t)vl[(t8 + 2 * e) * VP + dim] |
                    ((uint32_t)vl[(t8 + 2 * e + 1) * VP + dim] << 16);
          const bf16x8_t av = __builtin_bit_cast(bf16x8_t, make_uint4(vw[0], vw[1], vw[2], vw[3]));
          oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bh, oacc[dt], 0, 0, 0);
          oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bl, oacc[dt], 0, 0, 0);
        }
      }
      __syncthreads();   // the next chunk's scores and values overwrite sc, st and vl
      continue;
    }
    // ---- P.V: each lane accumulates its 8 dimensions for the HPW heads
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      const float f = st[2 * HPW + hh];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[hh][e] *= f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = u * TPB + wave * TPI + tsub;
      if (s < n) {
        const uint32_t w[4] = {vv[u].x, vv[u].y, vv[u].z, vv[u].w};
        float v8[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v8[2 * e] = bf16_to_f32(w[e] & 0xFFFFu);
          v8[2 * e + 1] = bf16_to_f32(w[e] >> 16);
        }
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) {
          const float p = sc[hh * C + s];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[hh][e] = __builtin_fmaf(p, v8[e], acc[hh][e]);
        }
      }
    }
    if (more) {   // the values are used: request the next chunk's
#pragma unroll
      for (int u = 0; u < U; ++u) vv[u] = load_nt(row(a.vc, tok(c0 + C, u)));
    }
    __syncthreads();   // the next chunk's scores overwrite sc and st
  }

  const size_t rec = (size_t)(D + 4);
  if constexpr (kMM) {   // each wave holds whole dimensions of every head: no reduction
    const int hq = lane & 15;
    float* part = a.part + (((size_t)b * a.Hq + h0) * a.nspans + blockIdx.x) * rec;
    if (hq < HPW) {
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) {
        const int d0 = (wave * ND + dt) * 16 + 4 * (lane >> 4);
        *reinterpret_cast<float4*>(part + hq * a.nspans * rec + 4 + d0) =
            make_float4(oacc[dt][0], oacc[dt][1], oacc[dt][2], oacc[dt][3]);
      }
    }
    if (tid < HPW) {
      part[tid * a.nspans * rec + 0] = st[tid];
      part[tid * a.nspans * rec + 1] = st[HPW + tid];
    }
    return;
  }
  // sum over the wave's token groups (lanes with the same dimensions), then over the waves
#pragma unroll
  for (int off = LPT; off < 64; off <<= 1)
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[hh][e] += __shfl_xor(acc[hh][e], off, 64);
  if (tsub == 0) {
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) wacc[(wave * HPW + hh) * D + dsl * 8 + e] = acc[hh][e];
  }
  __syncthreads();
  float* part = a.part + (((size_t)b * a.Hq + h0) * a.nspans + blockIdx.x) * rec;
  for (int i = tid; i < HPW * D; i += kAttnThreads) {
    const int hh = i / D, d = i % D;
    const float s = ((wacc[hh * D + d] + wacc[(HPW + hh) * D + d]) + wacc[(2 * HPW + hh) * D + d]) +
                    wacc[(3 * HPW + hh) * D + d];
    part[hh * a.nspans * rec + 4 + d] = s;
  }
  if (tid < HPW) {
    part[tid * a.nspans * rec + 0] = st[tid];
    part[tid * a.nspans * rec + 1] = st[HPW + tid];
  }
}

// One workgroup per (query head, sequence): the spans' records merged. The weights
// exp(max_s - max) go to LDS; then lanes take 4 dimensions of a record each (D/4 lanes per
// record, 256 / (D/4) records per step over interleaved records) and the per-slot sums are
// added in slot order, so the result does not depend on scheduling.
template <int D, int DS>
__global__ __launch_bounds__(kAttnThreads) void k_attn_combine(AttnArgs a) {
  // a workgroup merges DS dimensions of one head (D / DS workgroups per head)
  static_assert(D % DS == 0 && DS % 32 == 0, "whole 32-dimension slices");
  constexpr int TPR = DS / 4;             // lanes per record
  constexpr int RPS = kAttnThreads / TPR; // records per step
  constexpr int UNR = 8;                  // records per lane requested together
  __shared__ float wts[kAttnMaxSpans];
  __shared__ float red[8];
  __shared__ __attribute__((aligned(16))) float part_sum[RPS * DS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.x / (D / DS), ds0 = (blockIdx.x % (D / DS)) * DS;
  const int b = blockIdx.y;
  int len = a.lens[b];
  len = len < 0 ? 0 : (len > a.max_len ? a.max_len : len);
  const int ns = (len + a.span - 1) / a.span;
  float* o = a.out + ((size_t)b * a.Hq + h) * D + ds0;
  if (ns == 0) {
    for (int i = tid; i < DS; i += kAttnThreads) o[i] = 0.0f;
    return;
  }
  const size_t rec = (size_t)(D + 4);
  const float* r = a.part + ((size_t)b * a.Hq + h) * a.nspans * rec;
  // lane slot `sl` takes records sl, sl + RPS, ...; its first UNR records are requested before
  // the maximum is known, so their round trip overlaps that of the (max, sum) pairs
  const int sl = tid / TPR, d4 = (tid % TPR) * 4;
  float4 v[UNR];
#pragma unroll
  for (int u = 0; u < UNR; ++u) {
    const int cc = min(sl + u * RPS, ns - 1);
    v[u] = *reinterpret_cast<const float4*>(r + cc * rec + 4 + ds0 + d4);
  }
  // the (max, sum) pairs of this thread's spans, read once
  constexpr int kPer = kAttnMaxSpans / kAttnThreads;
  static_assert(kAttnMaxSpans % kAttnThreads == 0, "whole spans per thread");
  float mv[kPer], lv[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int c = tid + kAttnThreads * i;
    mv[i] = c < ns ? r[c * rec] : -INFINITY;
    lv[i] = c < ns ? r[c * rec + 1] : 0.0f;
  }
  // the maximum over the spans
  float M = mv[0];
#pragma unroll
  for (int i = 1; i < kPer; ++i) M = fmaxf(M, mv[i]);
  M = wave_max_f(M);
  if (lane == 0) red[wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  // weights and the total sum
  float L = 0.0f;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int c = tid + kAttnThreads * i;
    if (c < ns) {
      const float w = __expf(mv[i] - M);
      wts[c] = w;
      L = __builtin_fmaf(w, lv[i], L);
    }
  }
  L = wave_sum(L);
  if (lane == 0) red[4 + wave] = L;
  __syncthreads();
  L = ((red[4] + red[5]) + red[6]) + red[7];
  // weighted sum of the accumulators, records in increasing order per lane slot
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int c = sl; c < ns; c += UNR * RPS) {
    if (c != sl) {
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int cc = min(c + u * RPS, ns - 1);
        v[u] = *reinterpret_cast<const float4*>(r + cc * rec + 4 + ds0 + d4);
      }
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      if (c + u * RPS < ns) {
        const float w = wts[c + u * RPS];
        acc.x = __builtin_fmaf(w, v[u].x, acc.x);
        acc.y = __builtin_fmaf(w, v[u].y, acc.y);
        acc.z = __builtin_fmaf(w, v[u].z, acc.z);
        acc.w = __builtin_fmaf(w, v[u].w, acc.w);
      }
    }
  }
  *reinterpret_cast<float4*>(part_sum + sl * DS + d4) = acc;
  __syncthreads();
  if (tid < DS) {
    float tot = 0.0f;
#pragma unroll
    for (int k = 0; k < RPS; ++k) tot += part_sum[k * DS + tid];
    o[tid] = tot / L;
  }
}

// ------------------------------------------------------------------------------ host side
namespace {

bool attn_desc_ok(const attn_gqa_desc_t* d) {
  if (!d || d->num_q_heads <= 0 || d->num_kv_heads <= 0) return false;
  if (d->num_q_heads % d->num_kv_heads) return false;
  const int G = d->num_q_heads / d->num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return false;
  if (d->head_dim != 64 && d->head_dim != 128 && d->head_dim != 256) return false;
  const int bs = d->block_size;
  return bs == 16 || bs == 32 || bs == 64 || bs == 128 || bs == 256;
}

struct AttnPlan {
  int hpw, u, chunk, span, nspans;
  size_t part_bytes;
};

int chunk_tokens(int D, int u) {
  if (u == 8) return D == 64 ? attn_chunk<64, 8>() : D == 128 ? attn_chunk<128, 8>() : attn_chunk<256, 8>();
  if (u == 4) return D == 64 ? attn_chunk<64, 4>() : D == 128 ? attn_chunk<128, 4>() : attn_chunk<256, 4>();
  return D == 64 ? attn_chunk<64, 2>() : D == 128 ? attn_chunk<128, 2>() : attn_chunk<256, 2>();
}

// Chunks of attn_chunk<D, 8>() tokens (256, 128 or 64 for D = 64, 128, 256), or shorter ones
// when those would give fewer than kAttnTargetWorkgroups workgroups: half as long for packed
// workgroups with D <= 128 (the MFMA path), a quarter otherwise. Spans take as many chunks as it
// needs to keep the grid near the target (packed or unpacked) in workgroups.
AttnPlan attn_plan(const attn_gqa_desc_t* d, int B, int max_len, bool unpacked) {
  AttnPlan p{};
  const int G = d->num_q_heads / d->num_kv_heads;
  p.hpw = unpacked ? 1 : G;
  const int D = d->head_dim;
  const int64_t groups = (int64_t)(B > 0 ? B : 1) * (d->num_q_heads / p.hpw);
  const int64_t len = max_len > 0 ? max_len : 1;
  p.u = 8;
  if (groups * ((len + chunk_tokens(D, 8) - 1) / chunk_tokens(D, 8)) < kAttnTargetWorkgroups)
    p.u = (p.hpw >= 4 && D <= 128) ? 4 : 2;   // packed: 64-token chunks keep the MFMA path
  p.chunk = chunk_tokens(D, p.u);
  const int64_t nchunks = (len + p.chunk - 1) / p.chunk;
  const int64_t target = p.hpw == 1 ? kAttnTargetWorkgroupsUnpacked : kAttnTargetWorkgroups;
  const int64_t want = std::max<int64_t>(1, (target + groups - 1) / groups);
  const int64_t cps = std::max<int64_t>(1, (nchunks + want - 1) / want);   // chunks per span
  p.span = (int)std::min<int64_t>(cps * p.chunk, 1 << 30);
  p.nspans = (int)((nchunks + cps - 1) / cps);
  p.part_bytes = (size_t)(B > 0 ? B : 0) * d->num_q_heads * p.nspans * (D + 4) * 4;
  return p;
}

int ilog2(int v) {
  int s = 0;
  while ((1 << s) < v) ++s;
  return s;
}

}  // namespace

}  // namespace moe

using namespace moe;

extern "C" size_t attn_gqa_decode_workspace_bytes(const attn_gqa_desc_t* desc, int32_t batch,
                                                  int32_t max_seq_len) {
  if (!attn_desc_ok(desc) || batch < 0 || max_seq_len < 0) return 0;
  const AttnPlan p1 = attn_plan(desc, batch, max_seq_len, false);
  const AttnPlan p2 = attn_plan(desc, batch, max_seq_len, true);
  const size_t b = p1.part_bytes > p2.part_bytes ? p1.part_bytes : p2.part_bytes;
  return ((b > 0 ? b : 16) + 255) / 256 * 256;
}

extern "C" int attn_gqa_decode(const attn_gqa_desc_t* desc, const uint16_t* q,
                               const uint16_t* k_cache, const uint16_t* v_cache,
                               int32_t num_blocks, const int32_t* block_table,
                               int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t batch,
                               int32_t max_seq_len, float* out, int32_t flags, void* workspace,
                               size_t ws_bytes, void* stream) {
  if (!desc) return MOE_INVALID_ARG;
  if (!attn_desc_ok(desc)) return MOE_UNSUPPORTED;
  if (batch < 0 || max_seq_len < 0 || (flags & ~ATTN_FLAG_UNPACKED)) return MOE_INVALID_ARG;
  if (batch == 0) return MOE_OK;
  if (!q || !out || !seq_lens || ((uintptr_t)q & 15) || ((uintptr_t)out & 15)) return MOE_INVALID_ARG;
  if (max_seq_len > 0) {
    if (!k_cache || !v_cache || !block_table || num_blocks <= 0 || max_blocks_per_seq <= 0 ||
        ((uintptr_t)k_cache & 15) || ((uintptr_t)v_cache & 15))
      return MOE_INVALID_ARG;
    if ((int64_t)max_blocks_per_seq * desc->block_size < max_seq_len) return MOE_INVALID_ARG;
  }
  if (!workspace || ((uintptr_t)workspace & 255)) return MOE_INVALID_ARG;
  if (ws_bytes < attn_gqa_decode_workspace_bytes(desc, batch, max_seq_len))
    return MOE_WORKSPACE_TOO_SMALL;
  const bool unpacked = (flags & ATTN_FLAG_UNPACKED) != 0;
  const AttnPlan p = attn_plan(desc, batch, max_seq_len, unpacked);
  if (p.nspans > kAttnMaxSpans) return MOE_UNSUPPORTED;   // cannot happen: nspans <= target
  AttnArgs a;
  a.q = q;
  a.kc = k_cache;
  a.vc = v_cache;
  a.table = block_table;
  a.lens = seq_lens;
  a.part = static_cast<float*>(workspace);
  a.out = out;
  a.Hq = desc->num_q_heads;
  a.Hkv = desc->num_kv_heads;
  a.bs_shift = ilog2(desc->block_size);
  a.MB = max_blocks_per_seq;
  a.nblocks = num_blocks;
  a.max_len = max_seq_len;
  a.span = p.span;
  a.nspans = p.nspans;
  a.scale = desc->scale;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int D = desc->head_dim;
  if (max_seq_len > 0) {
    const dim3 grid(p.nspans, desc->num_q_heads / p.hpw, batch);
#define ATTN_SPLIT(DV, HV, UV) \
  hipLaunchKernelGGL((k_attn_split<DV, HV, UV>), grid, dim3(kAttnThreads), 0, s, a)
#define ATTN_SPLIT_U(DV, HV)                    \
  do {                                          \
    if (p.u == 8) ATTN_SPLIT(DV, HV, 8);        \
    else if (p.u == 4) ATTN_SPLIT(DV, HV, 4);   \
    else ATTN_SPLIT(DV, HV, 2);                 \
  } while (0)
#define ATTN_SPLIT_D(HV)                        \
  do {                                          \
    if (D == 64) ATTN_SPLIT_U(64, HV);          \
    else if (D == 128) ATTN_SPLIT_U(128, HV);   \
    else ATTN_SPLIT_U(256, HV);                 \
  } while (0)
    switch (p.hpw) {
      case 1: ATTN_SPLIT_D(1); break;
      case 2: ATTN_SPLIT_D(2); break;
      case 4: ATTN_SPLIT_D(4); break;
      default: ATTN_SPLIT_D(8); break;
    }
#undef ATTN_SPLIT_D
#undef ATTN_SPLIT_U
#undef ATTN_SPLIT
    if (hipGetLastError() != hipSuccess) return MOE_HIP_ERROR;
  }
  // Whole heads per workgroup when every span's record fits one request round of its lanes
  // (kAttnThreads / (D / 4) records per step, 8 steps); otherwise 32 dimensions per
  // workgroup, so that a long context's records are requested by D / 32 workgroups per head,
  // 256 records per round.
  const bool whole = a.nspans <= 8 * kAttnThreads / (D / 4);
  const dim3 gridc(desc->num_q_heads * (whole ? 1 : D / 32), batch);
  if (D == 64) {
    if (whole) hipLaunchKernelGGL((k_attn_combine<64, 64>), gridc, dim3(kAttnThreads), 0, s, a);
    else hipLaunchKernelGGL((k_attn_combine<64, 32>), gridc, dim3(kAttnThreads), 0, s, a);
  } else if (D == 128) {
    if (whole) hipLaunchKernelGGL((k_attn_combine<128, 128>), gridc, dim3(kAttnThreads), 0, s, a);
    else hipLaunchKernelGGL((k_attn_combine<128, 32>), gridc, dim3(kAttnThreads), 0, s, a);
  } else {
    if (whole) hipLaunchKernelGGL((k_attn_combine<256, 256>), gridc, dim3(kAttnThreads), 0, s, a);
    else hipLaunchKernelGGL((k_attn_combine<256, 32>), gridc, dim3(kAttnThreads), 0, s, a);
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_HIP_ERROR;
}
