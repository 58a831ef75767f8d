// The greedy decode step: LM head, argmax over the vocabulary, the chosen token's embedding as
// the next input, and its C ABI (greedy_head.h).
//
// "Perplexity's Lily: A Breakthrough Local Inference Engine Tailored Exclusively for Apple
// Silicon", section "How It Works: Prefill and Decode Strategies": the selected token is written
// straight into the next step's GPU-resident input slot; section "Frequently Asked Questions":
// greedy decoding only. The head is a V x H matrix in the 4-bit format: streaming it once per
// step is a bandwidth-bound GEMV (about 175 MB at V = 151,936, H = 2048).
//
// Layout of the work:
//  * k_head_logits: a grid-stride loop of waves over the vocabulary rows. A row of H packed
//    inputs is read by the 64 lanes of a wave with one load of H/512 words each (16 bytes at
//    H = 2048), the next row requested before the current one is used; dequantisation as in the
//    expert GEMVs (bf16-rounded weights, bf16 x pairs, fp32 sums), a DPP wave sum per token, and
//    a running (maximum, lowest index) per token. The workgroup's waves merge theirs in LDS and
//    write one partial per workgroup and token; the logits are stored as well.
//  * k_head_pick: one workgroup per token merges the partials (ties to the lowest index) and
//    writes the token and its embedding row, dequantised and rounded to bf16.
#include <climits>

#include "greedy_head.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kHeadWaves = 4;
constexpr int kHeadMaxWG = 2048;   // a multiple of 256 (k_head_pick reads kHeadMaxWG / 256 each)
constexpr int kHeadMaxT = 16;

struct HeadArgs {
  moe_w4_t head, embed;
  const uint16_t* x;
  int32_t* token;
  uint16_t* x_next;
  float* logits;      // [T, V]
  int2* part;         // [nwg, T]: (max bits, index)
  int V, H, T;
};

// Sum over the 64 lanes through DPP (row shifts, then row broadcasts into lane 63).
__device__ __forceinline__ float wave_sum_dpp(float v) {
  int b = __float_as_int(v);
  b = __float_as_int(__int_as_float(b) + __int_as_float(__builtin_amdgcn_update_dpp(0, b, 0x111, 0xF, 0xF, false)));
  b = __float_as_int(__int_as_float(b) + __int_as_float(__builtin_amdgcn_update_dpp(0, b, 0x112, 0xF, 0xF, false)));
  b = __float_as_int(__int_as_float(b) + __int_as_float(__builtin_amdgcn_update_dpp(0, b, 0x114, 0xF, 0xF, false)));
  b = __float_as_int(__int_as_float(b) + __int_as_float(__builtin_amdgcn_update_dpp(0, b, 0x118, 0xF, 0xF, false)));
  b = __float_as_int(__int_as_float(b) + __int_as_float(__builtin_amdgcn_update_dpp(0, b, 0x142, 0xA, 0xF, false)));
  b = __float_as_int(__int_as_float(b) + __int_as_float(__builtin_amdgcn_update_dpp(0, b, 0x143, 0xC, 0xF, false)));
  return __int_as_float(__builtin_amdgcn_readlane(b, 63));
}

// (value, index) ordering of the argmax: larger value first, then the lower index
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

template <int WPL>
struct HeadRow {
  uint32_t w[WPL];
  uint16_t s, b;
};

}  // namespace

// WPL packed words per lane (H = 512 * WPL); TC tokens at most (T <= TC).
template <int WPL, int TC>
__global__ __launch_bounds__(64 * kHeadWaves) void k_head_logits(HeadArgs a) {
  __shared__ float bv_s[kHeadWaves][TC];
  __shared__ int bi_s[kHeadWaves][TC];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int T = a.T, H = a.H, V = a.V;
  const int gw = blockIdx.x * kHeadWaves + wave, nw = gridDim.x * kHeadWaves;
  const int wpr = H >> 3, gpr = H >> 6;
  // this lane's inputs: words lane*WPL .. + WPL of a row (all in group lane*WPL/8)
  const int g = (lane * WPL) >> 3;
  uint32_t xw[TC][4 * WPL];  // the lane's x as bf16 pairs, per token
#pragma unroll
  for (int t = 0; t < TC; ++t)
#pragma unroll
    for (int i = 0; i < 4 * WPL; ++i) xw[t][i] = 0u;
#pragma unroll
  for (int t = 0; t < TC; ++t) {
    if (t < T) {
      const uint4* xp = reinterpret_cast<const uint4*>(a.x + (size_t)t * H + lane * WPL * 8);
#pragma unroll
      for (int i = 0; i < WPL; ++i) {
        const uint4 v = xp[i];
        xw[t][4 * i + 0] = v.x; xw[t][4 * i + 1] = v.y; xw[t][4 * i + 2] = v.z; xw[t][4 * i + 3] = v.w;
      }
    }
  }
  auto load_row = [&](HeadRow<WPL>& r, int v) {
    const uint32_t* q = a.head.q + (size_t)v * wpr + lane * WPL;
    if constexpr (WPL >= 4) {
#pragma unroll
      for (int i = 0; i < WPL / 4; ++i) {
        const uint4 u = load_nt(q + 4 * i);
        r.w[4 * i] = u.x; r.w[4 * i + 1] = u.y; r.w[4 * i + 2] = u.z; r.w[4 * i + 3] = u.w;
      }
    } else if constexpr (WPL == 2) {
      const uint2 u = *reinterpret_cast<const uint2*>(q);
      r.w[0] = u.x; r.w[1] = u.y;
    } else {
      r.w[0] = q[0];
    }
    r.s = __builtin_nontemporal_load(a.head.scale + (size_t)v * gpr + g);
    r.b = __builtin_nontemporal_load(a.head.bias + (size_t)v * gpr + g);
  };
  float best[TC];
  int bidx[TC];
#pragma unroll
  for (int t = 0; t < TC; ++t) {
    best[t] = -INFINITY;
    bidx[t] = INT_MAX;
  }
  HeadRow<WPL> cur, nxt;
  int v = gw;
  if (v < V) load_row(cur, v);
  for (; v < V; v += nw) {
    if (v + nw < V) load_row(nxt, v + nw);   // the next row in flight
    const float s = bf16_to_f32(cur.s), b = bf16_to_f32(cur.b);
    float acc[TC];
#pragma unroll
    for (int t = 0; t < TC; ++t) acc[t] = 0.0f;
#pragma unroll
    for (int i = 0; i < WPL; ++i) {
      uint32_t d[4];
      dequant8(cur.w[i], s, b, d);
#pragma unroll
      for (int t = 0; t < TC; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[t] = dot2_bf16(d[e], xw[t][4 * i + e], acc[t]);
    }
#pragma unroll
    for (int t = 0; t < TC; ++t) {
      if (t < T) {
        const float l = wave_sum_dpp(acc[t]);
        if (lane == 0) a.logits[(size_t)t * V + v] = l;
        if (better(l, v, best[t], bidx[t])) {
          best[t] = l;
          bidx[t] = v;
        }
      }
    }
    cur = nxt;
  }
  if (lane == 0) {
#pragma unroll
    for (int t = 0; t < TC; ++t) {
      bv_s[wave][t] = best[t];
      bi_s[wave][t] = bidx[t];
    }
  }
  __syncthreads();
  if (threadIdx.x < T) {
    const int t = threadIdx.x;
    float bv = bv_s[0][t];
    int bi = bi_s[0][t];
#pragma unroll
    for (int w = 1; w < kHeadWaves; ++w)
      if (better(bv_s[w][t], bi_s[w][t], bv, bi)) {
        bv = bv_s[w][t];
        bi = bi_s[w][t];
      }
    a.part[(size_t)blockIdx.x * T + t] = make_int2(__float_as_int(bv), bi);
  }
}

// One workgroup per token: the partials merged, then the embedding row of the token.
__global__ __launch_bounds__(256) void k_head_pick(HeadArgs a, int nwg) {
  __shared__ float bv_s[256];
  __shared__ int bi_s[256];
  __shared__ int tok_s;
  const int t = blockIdx.x, tid = threadIdx.x;
  float bv = -INFINITY;
  int bi = INT_MAX;
  constexpr int kPer = kHeadMaxWG / 256;   // partials per thread, all requested at once
  int2 pv[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int w = tid + 256 * i;
    pv[i] = w < nwg ? a.part[(size_t)w * a.T + t] : make_int2(__float_as_int(-INFINITY), INT_MAX);
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    if (better(__int_as_float(pv[i].x), pv[i].y, bv, bi)) {
      bv = __int_as_float(pv[i].x);
      bi = pv[i].y;
    }
  bv_s[tid] = bv;
  bi_s[tid] = bi;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {   // pairwise, in a fixed pattern
    if (tid < off && better(bv_s[tid + off], bi_s[tid + off], bv_s[tid], bi_s[tid])) {
      bv_s[tid] = bv_s[tid + off];
      bi_s[tid] = bi_s[tid + off];
    }
    __syncthreads();
  }
  if (tid == 0) {
    int tok = bi_s[0];
    tok = tok < 0 ? 0 : (tok >= a.V ? a.V - 1 : tok);   // every row was seen: never clamps
    tok_s = tok;
    a.token[t] = tok;
  }
  __syncthreads();
  const int tok = tok_s;
  const int wpr = a.H >> 3, gpr = a.H >> 6;
  for (int w = tid; w < wpr; w += 256) {
    const uint32_t word = a.embed.q[(size_t)tok * wpr + w];
    const size_t gi = (size_t)tok * gpr + (w >> 3);
    uint32_t d[4];
    dequant8(word, bf16_to_f32(a.embed.scale[gi]), bf16_to_f32(a.embed.bias[gi]), d);
    *reinterpret_cast<uint4*>(a.x_next + (size_t)t * a.H + 8 * w) = make_uint4(d[0], d[1], d[2], d[3]);
  }
}

}  // namespace moe

using namespace moe;

namespace {

int head_wgs(int V) {
  const int want = (V + kHeadWaves * 8 - 1) / (kHeadWaves * 8);   // at least 8 rows per wave
  return want < 1 ? 1 : (want > kHeadMaxWG ? kHeadMaxWG : want);
}

size_t align256(size_t n) { return (n + 255) / 256 * 256; }

}  // namespace

extern "C" size_t moe_greedy_workspace_bytes(int32_t V, int32_t T) {
  if (V < 1 || T < 1 || T > kHeadMaxT) return 0;
  return align256((size_t)T * V * 4) + align256((size_t)head_wgs(V) * T * 8);
}

extern "C" int moe_greedy_next_input(const moe_w4_t* head, const moe_w4_t* embed, int32_t V,
                                     int32_t H, const uint16_t* x, int32_t T, int32_t* token,
                                     uint16_t* x_next, void* workspace, size_t ws_bytes,
                                     void* stream) {
  if (!head || !embed) return MOE_INVALID_ARG;
  if (H != 512 && H != 1024 && H != 2048 && H != 4096) return MOE_UNSUPPORTED;
  if (V < 1 || T < 1 || T > kHeadMaxT) return MOE_INVALID_ARG;
  if (H == 4096 && T > 8) return MOE_UNSUPPORTED;   // the lane's x would not fit its registers
  if (!head->q || !head->scale || !head->bias || !embed->q || !embed->scale || !embed->bias)
    return MOE_INVALID_ARG;
  if (!x || !token || !x_next || ((uintptr_t)x & 15) || ((uintptr_t)x_next & 15) ||
      ((uintptr_t)head->q & 15) || ((uintptr_t)embed->q & 3))
    return MOE_INVALID_ARG;
  if (!workspace || ((uintptr_t)workspace & 255)) return MOE_INVALID_ARG;
  if (ws_bytes < moe_greedy_workspace_bytes(V, T)) return MOE_WORKSPACE_TOO_SMALL;
  HeadArgs a;
  a.head = *head;
  a.embed = *embed;
  a.x = x;
  a.token = token;
  a.x_next = x_next;
  a.logits = static_cast<float*>(workspace);
  a.part = reinterpret_cast<int2*>(static_cast<char*>(workspace) + align256((size_t)T * V * 4));
  a.V = V;
  a.H = H;
  a.T = T;
  const int nwg = head_wgs(V);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(nwg), block(64 * kHeadWaves);
#define HEAD_T(WPL, TMAX)                                                                     \
  do {                                                                                        \
    if (T == 1) hipLaunchKernelGGL((k_head_logits<WPL, 1>), grid, block, 0, s, a);            \
    else if (T <= 2) hipLaunchKernelGGL((k_head_logits<WPL, 2>), grid, block, 0, s, a);       \
    else if (T <= 4) hipLaunchKernelGGL((k_head_logits<WPL, 4>), grid, block, 0, s, a);       \
    else if (T <= 8) hipLaunchKernelGGL((k_head_logits<WPL, 8>), grid, block, 0, s, a);       \
    else hipLaunchKernelGGL((k_head_logits<WPL, TMAX>), grid, block, 0, s, a);                \
  } while (0)
  if (H == 512) HEAD_T(1, 16);
  else if (H == 1024) HEAD_T(2, 16);
  else if (H == 2048) HEAD_T(4, 16);
  else HEAD_T(8, 8);
#undef HEAD_T
  if (hipGetLastError() != hipSuccess) return MOE_HIP_ERROR;
  hipLaunchKernelGGL(k_head_pick, dim3(T), dim3(256), 0, s, a, nwg);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_HIP_ERROR;
}
