// Decode path of moe_layer_forward (T <= 16 tokens): the whole MoE layer in three launches.
//
// "Perplexity's Lily: A Breakthrough Local Inference Engine Tailored Exclusively for Apple
// Silicon", section "How It Works: Prefill and Decode Strategies": batch-1 decode barely reuses
// weights, so it is bound by the bytes moved per token, and a decode step made of many small
// dependent kernels is dominated by their sequencing; routing stays on the GPU with no CPU
// synchronisation. Section "The Model: Qwen3.6-35B-A3B in Focus": a router scores the experts
// and picks eight, one shared expert sees every token, and the 4-bit group-64 weights are
// rebuilt into bf16 for the tensor operations with fp32 accumulation.
//
// The layer has two all-to-all dependencies (every routed expert needs all router logits;
// every output row needs the complete SwiGLU activation of each selected expert), so it is cut
// into exactly three kernels; on gfx950 a kernel boundary inside a HIP graph costs less than a
// software grid barrier with the agent-scope fences that cross-XCD visibility needs.
//   A (k_dec_a): the routing-independent work: router logits (one wave per expert row, fp32 FMA
//     on the fp32 weights), the shared expert's gate logit, and the shared expert's gate/up rows
//     with SwiGLU (one wave per row pair);
//   B (k_dec_b): every workgroup selects each token's top-k from the logits (the same result in
//     all of them), groups the (token, rank) slots by expert in LDS (stable grouped rows by
//     counting; a single token's experts are its ranks), and its waves stream the selected
//     experts' gate/up rows (a 1 KiB row per wave, 16 bytes per lane), dequantise them in
//     registers and store A = bf16(silu(G) * U); workgroup 0 also stores the per-expert route
//     record for C. For a single token a wave requests its expert's rows as soon as the
//     selection has chosen that rank, while the later ranks are still being selected;
//   C (k_dec_c): down projection fused with the weighted combine of the fp32 expert outputs
//     (fp32 accumulation, never rounded). A workgroup owns four output rows (one per 16-lane group) and has one wave
//     per entry (the selected experts, the shared expert last; at most 16 waves, which then
//     take several entries each); the waves' partial sums are added in LDS in wave order,
//     so the result is deterministic.
// Every selected weight byte is read from HBM once per call.
#include "moe_internal.h"

namespace moe {

namespace {
constexpr int kNB = 2;  // k_dec_c, batches of more than one token: entries requested per batch
// k_dec_b runs one 16-wave workgroup per CU: a single wave per CU derives the top-k, so the
// selection rounds of different workgroups do not share a SIMD's issue slots.
constexpr int kDecBWaves = 16;
// k_dec_c: output rows per 16-lane group (two: one workgroup per eight rows, all resident at
// once on the full-size layer)
__host__ __device__ constexpr int dec_c_rows(int) { return 2; }
}  // namespace

struct DecodeArgs {
  const uint16_t* x;
  const float* router_w;
  const float* router_bias;
  const float* wg;  // shared-gate weights, or null when there is no shared expert
  moe_w4_t gate, up, down, sh_gate, sh_up, sh_down;
  int T, H, E, K, F, Fs;
  DecodeBufs b;
  float* out;       // [T, H]
  // inside the stack: A derives x from the residual stream rin (workgroup 0 writes it to xw),
  // and C adds the layer output into out (= the residual stream) instead of storing it
  const float* rin;
  uint16_t* xw;
  float eps;
  int acc_out;
};

// Butterfly sum of v[0..N) over aligned groups of W lanes (W = 16 or 64, N a power of two).
// Afterwards lane r of a group (r = lane % W) holds in v[0 .. N/W) the totals of entries
// (N/W)*r ... when N >= W, and otherwise in v[0] the total of entry r*N/W. Steps inside a row
// of 16 lanes use DPP; the steps across rows (distance 16, 32) use ds_bpermute.
template <int N, int W, int O>
__device__ __forceinline__ void group_reduce_step(float (&v)[N], int r) {
  if constexpr (O >= 1) {
    constexpr int live = (N * 2 * O / W) > 1 ? (N * 2 * O / W) : 1;
    if constexpr (live >= 2) {
      constexpr int h = live / 2;
      const bool up = (r & O) != 0;
#pragma unroll
      for (int j = 0; j < h; ++j) {
        const float keep = up ? v[j + h] : v[j];
        const float send = up ? v[j] : v[j + h];
        v[j] = keep + (O <= 8 ? dpp_partner16<O>(send) : __shfl_xor(send, O, 64));
      }
    } else {
      v[0] += O <= 8 ? dpp_partner16<O>(v[0]) : __shfl_xor(v[0], O, 64);
    }
    group_reduce_step<N, W, O / 2>(v, r);
  }
}

template <int N, int W>
__device__ __forceinline__ void group_reduce(float (&v)[N], int r) {
  group_reduce_step<N, W, W / 2>(v, r);
}

// One lane's share of a gate row and an up row: the 32-input chunk c = lane (H <= 2048: one
// 16-byte load per row and lane, a 1 KiB row per wave).
struct PairW {
  uint4 g, u;
  // raw bf16 bits, kept 16-bit so that the loaded value is the register itself (a widening at
  // a loop-carried copy would make the wave wait for the load); converted when used
  uint16_t gs, gb, us, ub;
};

// Every load is unconditional (lanes past the row re-read its last chunk, whose products are
// never used): a load whose destination is merged with a value from another branch has to be
// copied, and the copy makes the wave wait for the load right away.
// NT: non-temporal loads, for the routed experts' rows, which a decode step reads once and
// which would otherwise displace from the caches the weights that every step reads again (the
// router rows and the shared expert, about 3.5 MB per layer, loaded with ordinary loads).
template <bool NT>
__device__ __forceinline__ void load_pair(PairW& w, const moe_w4_t& G, const moe_w4_t& U,
                                          size_t row, int H, int lane) {
  const int c = lane < (H >> 5) ? lane : (H >> 5) - 1;
  const size_t sidx = row * (size_t)(H >> 6) + (c >> 1);
  if constexpr (NT) {
    w.g = load_nt(G.q + row * (size_t)(H >> 3) + 4 * c);
    w.u = load_nt(U.q + row * (size_t)(H >> 3) + 4 * c);
    w.gs = __builtin_nontemporal_load(G.scale + sidx);
    w.gb = __builtin_nontemporal_load(G.bias + sidx);
    w.us = __builtin_nontemporal_load(U.scale + sidx);
    w.ub = __builtin_nontemporal_load(U.bias + sidx);
  } else {
    w.g = reinterpret_cast<const uint4*>(G.q + row * (size_t)(H >> 3))[c];
    w.u = reinterpret_cast<const uint4*>(U.q + row * (size_t)(H >> 3))[c];
    w.gs = G.scale[sidx];
    w.gb = G.bias[sidx];
    w.us = U.scale[sidx];
    w.ub = U.bias[sidx];
  }
}

// Partial gate and up dot products of the lane's chunk with the m tokens listed in tok (token
// ids into the LDS copy of x; null = tokens 0..m-1). The chunk is dequantised once and used for
// all tokens. v[2j], v[2j+1] = gate, up partial of entry j.
template <int TC>
__device__ __forceinline__ void pair_dots(const PairW& w, const uint16_t* xs, int H, int lane,
                                          const int* tok, int m, float (&v)[2 * TC]) {
#pragma unroll
  for (int j = 0; j < 2 * TC; ++j) v[j] = 0.0f;
  if (lane >= (H >> 5)) return;
  uint32_t dg[16], du[16];
  const float gs = bf16_to_f32(w.gs), gb = bf16_to_f32(w.gb);
  const float us = bf16_to_f32(w.us), ub = bf16_to_f32(w.ub);
  dequant8(w.g.x, gs, gb, dg + 0);
  dequant8(w.g.y, gs, gb, dg + 4);
  dequant8(w.g.z, gs, gb, dg + 8);
  dequant8(w.g.w, gs, gb, dg + 12);
  dequant8(w.u.x, us, ub, du + 0);
  dequant8(w.u.y, us, ub, du + 4);
  dequant8(w.u.z, us, ub, du + 8);
  dequant8(w.u.w, us, ub, du + 12);
  auto token_dots = [&](int j, int t) __attribute__((always_inline)) {
    const uint4* xr = reinterpret_cast<const uint4*>(xs + (size_t)t * H + 32 * lane);
    float ag = 0.0f, au = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 xv = xr[q];
      ag = dot2_bf16(xv.x, dg[4 * q + 0], ag);
      ag = dot2_bf16(xv.y, dg[4 * q + 1], ag);
      ag = dot2_bf16(xv.z, dg[4 * q + 2], ag);
      ag = dot2_bf16(xv.w, dg[4 * q + 3], ag);
      au = dot2_bf16(xv.x, du[4 * q + 0], au);
      au = dot2_bf16(xv.y, du[4 * q + 1], au);
      au = dot2_bf16(xv.z, du[4 * q + 2], au);
      au = dot2_bf16(xv.w, du[4 * q + 3], au);
    }
    v[2 * j] = ag;
    v[2 * j + 1] = au;
  };
  if (!tok) {
    // tokens 0..m-1 of the staged batch (m is the batch, usually TC): every entry is formed
    // without a branch, entries past m from token 0 (never stored), so that the LDS reads of
    // all tokens are issued together instead of one branch and one wait per token
#pragma unroll
    for (int j = 0; j < TC; ++j) token_dots(j, j < m ? j : 0);
  } else {
#pragma unroll
    for (int j = 0; j < TC; ++j)
      if (j < m) token_dots(j, tok[j]);
  }
}

// Reduce the gate/up partials over the wave and store A = bf16(silu(g) * u) of entry j at
// a[a_row(j) + f]. After the reduction lane r holds entry r*2TC/64; u_j sits 32/TC lanes above
// g_j.
template <int TC, typename RowFn>
__device__ __forceinline__ void pair_finish(float (&v)[2 * TC], int lane, int m, int f,
                                            uint16_t* a, RowFn a_row) {
  group_reduce<2 * TC, 64>(v, lane);
  constexpr int s = 32 / TC;
  const float u = __shfl_xor(v[0], s, 64);
  const int j = lane / (2 * s);
  if (lane % (2 * s) == 0 && j < m) a[a_row(j) + f] = f32_to_bf16(silu_mul(v[0], u));
}

// Routing of one call as per-expert entries, in LDS. Entry d (d < D; ascending expert id, or
// rank order for a single token) is expert ent_e[d] with ent_m[d] tokens, whose grouped rows start at ent_row0[d]; bit t of
// ent_mask[d] is set if token t routes to it. Grouped row r belongs to token row_tok[r] with
// routing weight row_w[r] (tokens ascending inside an expert). The words from `nd` through sgs
// are also the route record that B hands to C.
struct Route {
  int* nd;            // [1] D
  int* ent_e;         // [TK]
  int* ent_m;         // [TK]
  int* ent_row0;      // [TK]
  unsigned* ent_mask; // [TK]
  float* row_w;       // [TK]
  float* sgs;         // [T] shared-expert gate
  int* row_tok;       // [TK] (B only)
};

__host__ __device__ __forceinline__ size_t route_words(int TK, int T) { return 1 + 5 * (size_t)TK + T; }

__device__ __forceinline__ Route carve_route(void* base, int TK, int T) {
  Route R;
  R.nd = reinterpret_cast<int*>(base);
  R.ent_e = R.nd + 1;
  R.ent_m = R.ent_e + TK;
  R.ent_row0 = R.ent_m + TK;
  R.ent_mask = reinterpret_cast<unsigned*>(R.ent_row0 + TK);
  R.row_w = reinterpret_cast<float*>(R.ent_mask + TK);
  R.sgs = R.row_w + TK;
  R.row_tok = reinterpret_cast<int*>(R.sgs + T);
  return R;
}

// Entries from the slots' experts sel_idx[TK] and weights sel_w[TK] (slot s = t*K + k); cnt and
// tmask [E] were filled while the top-k was written (each token routes to an expert at most
// once). Wave 0 scans the counts with DPP (E/64 consecutive experts per lane) and writes the
// entries in ascending expert order and each expert's first grouped row into off[E]; then slot
// s goes to grouped row off[e] + #{tokens t' < t routed to e} (stable). Ends with a barrier.
__device__ void build_route(const Route& R, const int* sel_idx, const float* sel_w,
                            const int* cnt, const unsigned* tmask, int* off, int T, int E, int K) {
  const int tid = threadIdx.x;
  if (tid < 64) {
    const int per = (E + 63) >> 6;  // experts per lane (<= 16)
    const int e0 = tid * per;
    int rows = 0, nz = 0;
    for (int i = 0; i < per; ++i) {
      const int e = e0 + i;
      const int c = e < E ? cnt[e] : 0;
      rows += c;
      nz += c > 0;
    }
    const int packed = (rows << 16) | nz;  // grouped rows < 2^15
    const int incl = wave_incl_scan(packed, tid);
    int row = (incl - packed) >> 16, d = (incl - packed) & 0xFFFF;
    for (int i = 0; i < per; ++i) {
      const int e = e0 + i;
      if (e < E) {
        const int c = cnt[e];
        off[e] = row;
        if (c > 0) {
          R.ent_e[d] = e;
          R.ent_m[d] = c;
          R.ent_row0[d] = row;
          R.ent_mask[d] = tmask[e];
          ++d;
        }
        row += c;
      }
    }
    if (tid == 63) *R.nd = incl & 0xFFFF;
  }
  __syncthreads();
  const int TK = T * K;
  for (int s = tid; s < TK; s += blockDim.x) {
    const int e = sel_idx[s], t = s / K;
    const int r = off[e] + __popc(tmask[e] & ((1u << t) - 1u));
    R.row_tok[r] = t;
    R.row_w[r] = sel_w[s];
  }
  __syncthreads();
}

// Copy n 16-byte pieces from global memory to LDS with the nt threads of the workgroup, NB
// pieces per thread in flight: each batch issues all its loads (indices past the end re-read
// the last piece) before the first LDS write, so a batch costs one memory round trip.
template <int NB>
__device__ __forceinline__ void stage_pieces(uint4* dst, const uint4* __restrict__ src, int n,
                                             int nt) {
  for (int v0 = threadIdx.x; v0 < n; v0 += NB * nt) {
    uint4 t[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int v = v0 + b * nt;
      t[b] = src[v < n ? v : n - 1];
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int v = v0 + b * nt;
      if (v < n) dst[v] = t[b];
    }
  }
}

// x = bf16(RMSNorm(r)) of T <= TC tokens (H <= 2048), by the 256 threads of the workgroup, into
// xs and, if xw is not null, to global memory: the same loads, fused multiply-adds, wave
// reduction, combination of the four wave sums, correctly rounded division and square root and
// bf16 rounding as k_residual_rmsnorm, so both give the same bits. part: 4 floats of LDS.
__device__ __forceinline__ void norm_x(uint16_t* xs, const float* __restrict__ r, int T, int H,
                                       float eps, uint16_t* xw, float* part) {
  const int tid = threadIdx.x;
  for (int t = 0; t < T; ++t) {
    const float* rr = r + (size_t)t * H;
    float4 v[2];
    float ss = 0.0f;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int i = 4 * tid + 1024 * k;
      if (i < H) {
        v[k] = *reinterpret_cast<const float4*>(rr + i);
        ss = __builtin_fmaf(v[k].x, v[k].x, ss);
        ss = __builtin_fmaf(v[k].y, v[k].y, ss);
        ss = __builtin_fmaf(v[k].z, v[k].z, ss);
        ss = __builtin_fmaf(v[k].w, v[k].w, ss);
      }
    }
    ss = wave_sum(ss);
    if ((tid & 63) == 0) part[tid >> 6] = ss;
    __syncthreads();
    const float tot = (part[0] + part[1]) + (part[2] + part[3]);
    const float den = sqrtf(tot / (float)H + eps);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int i = 4 * tid + 1024 * k;
      if (i < H) {
        uint2 o;
        o.x = pack_bf16x2(v[k].x / den, v[k].y / den);
        o.y = pack_bf16x2(v[k].z / den, v[k].w / den);
        *reinterpret_cast<uint2*>(xs + (size_t)t * H + i) = o;
        if (xw) *reinterpret_cast<uint2*>(xw + (size_t)t * H + i) = o;
      }
    }
    __syncthreads();  // part is reused by the next token
  }
}

// x of up to TC tokens with NT threads (H <= 2048: at most TC*256/NT pieces per thread)
template <int TC, int NT>
__device__ __forceinline__ void stage_x(uint16_t* xs, const uint16_t* __restrict__ x, int n8) {
  constexpr int per = (TC * 256 + NT - 1) / NT;
  stage_pieces<(per < 8 ? per : 8)>(reinterpret_cast<uint4*>(xs),
                                    reinterpret_cast<const uint4*>(x), n8, NT);
}

// ============================================================================ A
// Tasks (one per wave): [0, E) router rows, E: shared-gate logit, then one task per row f of the
// shared expert's gate and up matrices.
template <int TC>
__global__ __launch_bounds__(256) void k_dec_a(DecodeArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint4 smem[];
  const int T = p.T, H = p.H, E = p.E, F = p.F, Fs = p.Fs, TK = T * p.K;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  const int task = blockIdx.x * 4 + wave;
  const int nA = E + (Fs > 0 ? 1 + Fs : 0);
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);  // [T, H]

  const bool router = task <= E && task < nA;  // wave-uniform
  const float* wrow = task < E ? p.router_w + (size_t)task * H : p.wg;
  const int n4 = H >> 2;
  const int f = task - E - 1;
  const bool shared_task = !router && task < nA;
  float4 w[8];
  PairW pw;
  auto load_w = [&]() __attribute__((always_inline)) {
    if (router) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int j = lane + 64 * i;
        w[i] = j < n4 ? reinterpret_cast<const float4*>(wrow)[j] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    } else if (shared_task) {
      load_pair<false>(pw, p.sh_gate, p.sh_up, (size_t)f, H, lane);
    }
  };
  if (p.rin) {
    // inside the stack: the task's weights first, then x from the residual stream (workgroup 0
    // also writes it for B)
    load_w();
    float* part = reinterpret_cast<float*>(xs + (size_t)T * H);
    norm_x(xs, p.rin, T, H, p.eps, blockIdx.x == 0 ? p.xw : nullptr, part);
  } else {
    // x first (at most TC 16-byte pieces per thread, H <= 2048), then the task's weights: the
    // staging then waits for x only, and the dot products take the weights as they arrive.
    // The LDS writes sit inside each task branch so that the wait before them counts exactly
    // that branch's weight requests.
    const int n8 = (T * H) >> 3;
    u32x4_t xt[TC];  // a native vector type: an array of it stays in registers
#pragma unroll
    for (int b = 0; b < TC; ++b) {
      const int v = tid + 256 * b;
      xt[b] = reinterpret_cast<const u32x4_t*>(p.x)[v < n8 ? v : n8 - 1];
    }
    auto store_x = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int b = 0; b < TC; ++b) {
        const int v = tid + 256 * b;
        if (v < n8) reinterpret_cast<u32x4_t*>(xs)[v] = xt[b];
      }
    };
    if (router) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int j = lane + 64 * i;
        w[i] = j < n4 ? reinterpret_cast<const float4*>(wrow)[j] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
      store_x();
    } else if (shared_task) {
      load_pair<false>(pw, p.sh_gate, p.sh_up, (size_t)f, H, lane);
      store_x();
    } else {
      store_x();
    }
    __syncthreads();
  }

  if (router) {
    float acc[TC];
#pragma unroll
    for (int t = 0; t < TC; ++t) acc[t] = 0.0f;
    for (int j0 = 0; j0 < n4; j0 += 512) {
      if (j0 > 0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int j = j0 + lane + 64 * i;
          w[i] = j < n4 ? reinterpret_cast<const float4*>(wrow)[j] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
      // no branch per input piece or token: pieces past the row have zero weights and read
      // the row's last piece of x, tokens past T read token 0 (their sums are never stored),
      // so the LDS reads of all tokens are issued together
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int j = min(j0 + lane + 64 * i, n4 - 1);
#pragma unroll
        for (int t = 0; t < TC; ++t) {
          const int tt = t < T ? t : 0;
          const uint2 xv = *reinterpret_cast<const uint2*>(xs + (size_t)tt * H + 4 * j);
          float a = acc[t];
          a = __builtin_fmaf(bf16_to_f32(xv.x & 0xFFFFu), w[i].x, a);
          a = __builtin_fmaf(bf16_to_f32(xv.x >> 16), w[i].y, a);
          a = __builtin_fmaf(bf16_to_f32(xv.y & 0xFFFFu), w[i].z, a);
          a = __builtin_fmaf(bf16_to_f32(xv.y >> 16), w[i].w, a);
          acc[t] = a;
        }
      }
    }
    group_reduce<TC, 64>(acc, lane);
    constexpr int stride = 64 / TC;  // lane l holds token l / stride
    const int t = lane / stride;
    if (lane % stride == 0 && t < T) {
      if (task < E)
        p.b.logits[(size_t)t * E + task] = acc[0] + (p.router_bias ? p.router_bias[task] : 0.0f);
      else
        p.b.logits[(size_t)T * E + t] = acc[0];
    }
  } else if (shared_task) {
    float v[2 * TC];
    pair_dots<TC>(pw, xs, H, lane, nullptr, T, v);
    uint16_t* ash = p.b.a + (size_t)TK * F;
    pair_finish<TC>(v, lane, T, f, ash, [&](int j) { return (size_t)j * Fs; });
  }
}

// ============================================================================ B
// Grid-stride tasks (entry d, row f): one wave per gate row + up row, with the next task's rows
// requested before the current one is used.
template <int TC, int NJ>
__global__ __launch_bounds__(64 * kDecBWaves) void k_dec_b(DecodeArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint4 smem[];
  const int T = p.T, H = p.H, E = p.E, K = p.K, F = p.F, Fs = p.Fs, TK = T * K;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  const int NW = gridDim.x * kDecBWaves, gw = blockIdx.x * kDecBWaves + wave;
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);                  // [T, H]
  int* sel_idx = reinterpret_cast<int*>(xs + (size_t)T * H);        // [TK]
  float* sel_w = reinterpret_cast<float*>(sel_idx + TK);            // [TK]
  int* cnt = reinterpret_cast<int*>(sel_w + TK);                    // [E]
  unsigned* tmask = reinterpret_cast<unsigned*>(cnt + E);           // [E]
  int* off = reinterpret_cast<int*>(tmask + E);                     // [E]
  const Route R = carve_route(off + E, TK, T);

  // logits of this wave's first token and the shared-gate logits, requested before x is staged
  // (the logits region always holds the T gate logits after the T x E router logits)
  float lv[NJ];
  if (wave < T) load_logits<NJ>(p.b.logits + (size_t)wave * E, E, lane, lv);
  const float glog = p.b.logits[(size_t)T * E + (tid < T ? tid : T - 1)];
  stage_x<TC, 64 * kDecBWaves>(xs, p.x, (T * H) >> 3);
  if (T > 1)
    for (int e = tid; e < E; e += 64 * kDecBWaves) {
      cnt[e] = 0;
      tmask[e] = 0u;
    }
  if (tid < T && Fs > 0) R.sgs[tid] = 1.0f / (1.0f + __expf(-glog));
  if (T == 1 && tid < K) {
    // one token: its K experts are distinct, so the entries are the ranks themselves (entry k =
    // the rank-k expert, one row, A row k); no grouping pass is needed. ent_e[k] = -1 until
    // the top-k has chosen rank k.
    R.ent_e[tid] = -1;
    R.ent_m[tid] = 1;
    R.ent_row0[tid] = tid;
    R.ent_mask[tid] = 1u;
    R.row_tok[tid] = 0;
    if (tid == 0) *R.nd = K;
  }
  __syncthreads();
  if (T == 1) {
    // Wave 0 publishes each rank's expert as soon as its round has chosen it; the other waves
    // wait for the rank of their task only (below) and request its rows while the later
    // rounds still run, so most of the weight traffic overlaps the selection.
    if (wave == 0) {
      float my_v, my_w;
      int my_i;
      wave_topk_softmax<NJ>(lv, E, K, lane, my_v, my_i, my_w, [&](int r, int I) {
        if (lane == 0) __hip_atomic_store(R.ent_e + r, I, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      });
      if (lane < K) R.row_w[lane] = my_w;
      if (blockIdx.x == 0) {  // the route record for the down projection (this wave's writes)
        const int n = (int)route_words(TK, T);
        for (int i = lane; i < n; i += 64) p.b.route[i] = R.nd[i];
      }
    }
  } else {
    for (int t = wave; t < T; t += kDecBWaves) {
      if (t != wave) load_logits<NJ>(p.b.logits + (size_t)t * E, E, lane, lv);
      float my_v, my_w;
      int my_i;
      wave_topk_softmax<NJ>(lv, E, K, lane, my_v, my_i, my_w);
      if (lane < K) {
        sel_idx[t * K + lane] = my_i;
        sel_w[t * K + lane] = my_w;
        atomicAdd(&cnt[my_i], 1);
        atomicOr(&tmask[my_i], 1u << t);
      }
    }
    __syncthreads();
    build_route(R, sel_idx, sel_w, cnt, tmask, off, T, E, K);
    if (blockIdx.x == 0) {  // the route record for the down projection
      const int n = (int)route_words(TK, T);
      for (int i = tid; i < n; i += 64 * kDecBWaves) p.b.route[i] = R.nd[i];
    }
  }
  const int D = T == 1 ? K : *R.nd;
  // expert of entry d: for one token, wait until wave 0 has published it (it always publishes
  // all K ranks, so the wait ends); the value is read once per wave (readfirstlane)
  auto expert_of = [&](int d) -> int {
    if (T > 1) return R.ent_e[d];
    int e;
    while ((e = __builtin_amdgcn_readfirstlane(__hip_atomic_load(
                R.ent_e + d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP))) < 0)
      __builtin_amdgcn_s_sleep(1);
    return e;
  };

  // Tasks task = gw + NW*i, in batches of kPB; the next batch's rows are requested before the
  // current batch is used. A batch requests no rows past the last task. Task tk is row f of
  // entry d: for one token d = tk % K, so a workgroup's waves spread over the ranks and the
  // rows that wait for the last rounds of the selection are shared out over all CUs; for
  // several tokens d = tk / F (an entry's rows on neighbouring waves).
  const int nB = D * F;
  auto task_d = [&](int tk) { return T == 1 ? tk % K : tk / F; };
  auto task_f = [&](int tk) { return T == 1 ? tk / K : tk % F; };
  constexpr int kPB = 2;
  const int step = kPB * NW;
  auto issue = [&](PairW (&w)[kPB], int t0) {
#pragma unroll
    for (int b = 0; b < kPB; ++b) {
      const int tk = t0 + b * NW;
      if (b == 0 || tk < nB)  // uniform over the wave; t0 < nB at every call
        load_pair<true>(w[b], p.gate, p.up, (size_t)expert_of(task_d(tk)) * F + task_f(tk), H, lane);
    }
  };
  auto run = [&](const PairW (&w)[kPB], int t0) {
#pragma unroll
    for (int b = 0; b < kPB; ++b) {
      const int tk = t0 + b * NW;
      if (tk < nB) {  // uniform over the wave
        const int d = task_d(tk), f = task_f(tk);
        const int m = __builtin_amdgcn_readfirstlane(R.ent_m[d]);
        const int row0 = R.ent_row0[d];
        auto a_row = [&](int j) { return (size_t)(row0 + j) * F; };
        if (TC > 1 && m == 1) {  // most experts of a small batch serve one token
          float v[2];
          pair_dots<1>(w[b], xs, H, lane, R.row_tok + row0, 1, v);
          pair_finish<1>(v, lane, 1, f, p.b.a, a_row);
        } else {
          float v[2 * TC];
          pair_dots<TC>(w[b], xs, H, lane, R.row_tok + row0, m, v);
          pair_finish<TC>(v, lane, m, f, p.b.a, a_row);
        }
      }
    }
  };
  PairW w0[kPB], w1[kPB];
  int t0 = gw;
  if (t0 < nB) issue(w0, t0);
  __builtin_amdgcn_sched_barrier(0);
  for (; t0 < nB; t0 += 2 * step) {
    if (t0 + step < nB) issue(w1, t0 + step);
    __builtin_amdgcn_sched_barrier(0);  // keep the requests ahead of the use of w0
    run(w0, t0);
    if (t0 + step >= nB) break;
    if (t0 + 2 * step < nB) issue(w0, t0 + 2 * step);
    __builtin_amdgcn_sched_barrier(0);
    run(w1, t0 + step);
  }
}

// ============================================================================ C
struct DownW {
  uint4 q;
  uint16_t s, b;  // raw bf16 bits (16-bit for the same reason as in PairW)
};

// A workgroup of NW waves (blockDim.x = 64*NW, NW <= 16) owns the 4*kRG output rows
// h = 4*(kRG*blockIdx.x + r) + g, r < kRG: 16-lane group g of every wave takes kRG rows
// (one workgroup per CU for the full-size layer, all resident at once). Wave w walks the entries
// d = w, w + NW, ... (ascending expert id, the shared expert last); lane sl of a group
// accumulates, for token sl, the routing-weighted fp32 expert outputs of the wave's
// entries. The waves' sums are then added in LDS in wave order, so the result is deterministic.
// The launcher sizes NW to the number of entries (at most 16): for a single token every wave
// has exactly one entry, and each lane's 32 activations of that entry are requested from
// global memory together with its weights (the four groups of a wave read the same
// addresses). Larger batches stage the activations in LDS when they fit (A_LDS).
template <int TC, bool A_LDS>
__global__ __launch_bounds__(1024) void k_dec_c(DecodeArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint4 smem[];
  constexpr int kRG = dec_c_rows(TC);
  const int T = p.T, H = p.H, F = p.F, Fs = p.Fs, TK = T * p.K;
  const int tid = threadIdx.x, lane = tid & 63;
  const int NW = __builtin_amdgcn_readfirstlane((int)blockDim.x >> 6);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  const int sl = lane & 15, grp = lane >> 4;
  const int h0 = 4 * kRG * (int)blockIdx.x + grp;  // row r of the group: h0 + 4*r
  const size_t a_elems = (size_t)TK * F + (size_t)T * Fs;
  uint16_t* as = reinterpret_cast<uint16_t*>(smem);                       // [a_elems] if A_LDS
  float* part = reinterpret_cast<float*>(A_LDS ? (void*)(as + a_elems) : (void*)smem);  // [NW][kRG][64]
  const Route R = carve_route(part + 64 * kRG * NW, TK, T);

  // inside the stack the residual values this wave adds the layer output to are requested
  // first, so that the final update does not wait for them
  float rold[kRG];
#pragma unroll
  for (int r = 0; r < kRG; ++r)
    rold[r] = p.acc_out && sl < T && r % NW == wave % NW ? p.out[(size_t)sl * H + h0 + 4 * r] : 0.0f;
  const int nw = (int)route_words(TK, T);
  for (int i = tid; i < nw; i += (int)blockDim.x) R.nd[i] = p.b.route[i];
  // D entries (a single token's are its K ranks, known before the route record arrives), the
  // shared expert last; ni of them on this wave
  int D = TC == 1 ? p.K : 0, nD = 0, ni = 0;
  const uint16_t* abase = A_LDS ? as : p.b.a;

  // Entries i0 .. i0+kB-1 of this wave; none past the wave's list is requested. Lanes past a
  // short row re-read its last chunk (never used), so the loads of an entry are unconditional;
  // the weight pointers are selected as values, not as references into the argument block
  // (which would be read with vector loads and waited for).
  constexpr int kB = TC == 1 ? 1 : kNB;  // entries per batch
  const uint32_t* const rq = p.down.q;
  const uint16_t* const rs = p.down.scale;
  const uint16_t* const rb = p.down.bias;
  const uint32_t* const sq = p.sh_down.q;
  const uint16_t* const ss = p.sh_down.scale;
  const uint16_t* const sb = p.sh_down.bias;
  struct Batch {
    DownW w[kB][kRG];
    uint4 a[TC == 1 ? kB : 1][4];  // single token: the lane's 32 activations of the entry
  };
  auto load_down = [&](int i0, Batch& bt) {
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      const int d = wave + NW * (i0 + b);
      if (d >= nD) break;  // uniform over the wave
      const bool sh = d == D;
      const int Kd = sh ? Fs : F;
      const int c = sl < (Kd >> 5) ? sl : (Kd >> 5) - 1;
      const uint32_t* q = sh ? sq : rq;
      const uint16_t* sp = sh ? ss : rs;
      const uint16_t* bp = sh ? sb : rb;
#pragma unroll
      for (int r = 0; r < kRG; ++r) {
        const int h = h0 + 4 * r;
        const size_t row = sh ? (size_t)h : (size_t)R.ent_e[d] * H + h;
        const size_t g = row * (size_t)(Kd >> 6) + (c >> 1);
        // non-temporal for every entry: the shared expert's rows are a small part of the
        // bytes, and one kind of load keeps the entry's loads free of a branch
        bt.w[b][r].q = load_nt(q + row * (size_t)(Kd >> 3) + 4 * c);
        bt.w[b][r].s = __builtin_nontemporal_load(sp + g);
        bt.w[b][r].b = __builtin_nontemporal_load(bp + g);
      }
      if constexpr (TC == 1) {
        const uint16_t* ar = sh ? p.b.a + (size_t)TK * F : p.b.a + (size_t)R.ent_row0[d] * F;
        const uint4* av = reinterpret_cast<const uint4*>(ar + 32 * c);
#pragma unroll
        for (int k = 0; k < 4; ++k) bt.a[b][k] = av[k];
      }
    }
  };
  auto use_down = [&](int i0, const Batch& bt, float (&accr)[kRG]) {
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      if (i0 + b >= ni) break;  // uniform over the wave
      const int d = wave + NW * (i0 + b);
      const bool sh = d == D;
      const int Kd = sh ? Fs : F;
      const int row0 = sh ? 0 : R.ent_row0[d];
#pragma unroll
      for (int r = 0; r < kRG; ++r) {
        float& acc = accr[r];
        uint32_t wd[16];
        const float ds = bf16_to_f32(bt.w[b][r].s), db = bf16_to_f32(bt.w[b][r].b);
        dequant8(bt.w[b][r].q.x, ds, db, wd + 0);
        dequant8(bt.w[b][r].q.y, ds, db, wd + 4);
        dequant8(bt.w[b][r].q.z, ds, db, wd + 8);
        dequant8(bt.w[b][r].q.w, ds, db, wd + 12);
        if constexpr (TC == 1) {
          float one[1] = {0.0f};
          if (sl < (Kd >> 5)) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              one[0] = dot2_bf16(bt.a[b][k].x, wd[4 * k + 0], one[0]);
              one[0] = dot2_bf16(bt.a[b][k].y, wd[4 * k + 1], one[0]);
              one[0] = dot2_bf16(bt.a[b][k].z, wd[4 * k + 2], one[0]);
              one[0] = dot2_bf16(bt.a[b][k].w, wd[4 * k + 3], one[0]);
            }
          }
          group_reduce<1, 16>(one, sl);
          const float wgt = sh ? R.sgs[0] : R.row_w[row0];
          if (sl == 0) acc = __builtin_fmaf(wgt, one[0], acc);
          continue;
        } else {
          const int m = __builtin_amdgcn_readfirstlane(sh ? T : R.ent_m[d]);
          const unsigned tmask = sh ? 0xFFFFFFFFu : R.ent_mask[d];
          if (m == 1) {
            // one token (bit t of the mask): every lane of the group ends with the row's sum
            float one[1] = {0.0f};
            if (sl < (Kd >> 5)) {
              const uint4* av = reinterpret_cast<const uint4*>(abase + (size_t)row0 * F + 32 * sl);
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const uint4 a4 = av[q];
                one[0] = dot2_bf16(a4.x, wd[4 * q + 0], one[0]);
                one[0] = dot2_bf16(a4.y, wd[4 * q + 1], one[0]);
                one[0] = dot2_bf16(a4.z, wd[4 * q + 2], one[0]);
                one[0] = dot2_bf16(a4.w, wd[4 * q + 3], one[0]);
              }
            }
            group_reduce<1, 16>(one, sl);
            if (sl < T && ((tmask >> sl) & 1u))
              acc = __builtin_fmaf(R.row_w[row0], one[0], acc);
            continue;
          }
          // tokens in pairs: one branch per pair, both rows' activation reads issued
          // together (the second row of a pair past m reads the first and is never taken)
          float dots[TC];
          const bool lane_in = sl < (Kd >> 5);
          const int sc = lane_in ? sl : 0;
#pragma unroll
          for (int j = 0; j < TC; ++j) dots[j] = 0.0f;
#pragma unroll
          for (int j = 0; j < TC; j += 2) {
            if (j < m && lane_in) {
#pragma unroll
              for (int h = 0; h < 2 && j + h < TC; ++h) {
                const int jr = j + h < m ? j + h : j;
                const uint16_t* ar = sh ? abase + (size_t)TK * F + (size_t)jr * Fs
                                        : abase + (size_t)(row0 + jr) * F;
                const uint4* av = reinterpret_cast<const uint4*>(ar + 32 * sc);
                float s = 0.0f;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                  const uint4 a4 = av[q];
                  s = dot2_bf16(a4.x, wd[4 * q + 0], s);
                  s = dot2_bf16(a4.y, wd[4 * q + 1], s);
                  s = dot2_bf16(a4.z, wd[4 * q + 2], s);
                  s = dot2_bf16(a4.w, wd[4 * q + 3], s);
                }
                dots[j + h] = s;
              }
            }
          }
          group_reduce<TC, 16>(dots, sl);
          // lane sl (= token) takes its entry: the token's rank inside this expert
          int j = 0;
          bool mine = false;
          float wgt = 0.0f;
          if (sl < T && ((tmask >> sl) & 1u)) {
            j = __popc(tmask & ((1u << sl) - 1u));
            mine = true;
            wgt = sh ? R.sgs[sl] : R.row_w[row0 + j];
          }
          const float val = __shfl(dots[0], (lane & ~15) + (j * 16) / TC, 64);
          if (mine) acc = __builtin_fmaf(wgt, val, acc);
        }
      }
    }
  };

  // The first batch is requested as soon as the route record is in LDS; the activations are
  // staged (A_LDS) while those loads are in flight. For a single token the shared expert's
  // entry (the first of wave K when there are more than K waves) depends on no routing: that
  // wave requests it before the route record has arrived and has it multiplied while the other
  // waves still wait for their rows.
  float acc[kRG];
#pragma unroll
  for (int r = 0; r < kRG; ++r) acc[r] = 0.0f;
  Batch b0, b1;
  const bool early = TC == 1 && Fs > 0 && wave == D;
  if (early) {
    nD = D + 1;
    ni = 1;
    load_down(0, b0);
  }
  __syncthreads();  // the route record is in LDS
  if (TC != 1) D = *R.nd;
  nD = D + (Fs > 0 ? 1 : 0);
  ni = wave < nD ? (nD - wave + NW - 1) / NW : 0;
  if (ni > 0 && !early) load_down(0, b0);
  __builtin_amdgcn_sched_barrier(0);
  if (A_LDS) {
    stage_pieces<8>(reinterpret_cast<uint4*>(as), reinterpret_cast<const uint4*>(p.b.a),
                    (int)(a_elems / 8), (int)blockDim.x);
    __syncthreads();
  }
  // batches of kB entries, the next batch requested before the current one is used
  for (int i0 = 0; i0 < ni; i0 += 2 * kB) {
    if (i0 + kB < ni) load_down(i0 + kB, b1);
    __builtin_amdgcn_sched_barrier(0);
    use_down(i0, b0, acc);
    if (i0 + kB >= ni) break;
    if (i0 + 2 * kB < ni) load_down(i0 + 2 * kB, b0);
    __builtin_amdgcn_sched_barrier(0);
    use_down(i0 + kB, b1, acc);
  }
#pragma unroll
  for (int r = 0; r < kRG; ++r) part[(wave * kRG + r) * 64 + lane] = acc[r];
  __syncthreads();
  // waves r, r + NW, ... add row r's partial sums over the waves in wave order
  for (int r = wave; r < kRG; r += NW) {
    if (sl < T) {
      float v = part[r * 64 + lane];
      for (int w = 1; w < NW; ++w) v += part[(w * kRG + r) * 64 + lane];
      // inside the stack: the residual update r + y
      p.out[(size_t)sl * H + h0 + 4 * r] = p.acc_out ? rold[r] + v : v;
    }
  }
}

// ------------------------------------------------------------------------ launcher
namespace {
int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}
constexpr size_t kDecLdsMax = 80 * 1024;  // two workgroups per CU (160 KiB of LDS)
// k_dec_c's workgroups of up to 16 waves are alone on their CU (registers), so C may stage its
// activations in up to this much LDS
constexpr size_t kDecCLdsMax = 144 * 1024;
}  // namespace

size_t decode_route_bytes(const Dims& d) { return route_words(d.TK(), d.T) * 4; }

// B's LDS after x: sel_idx, sel_w [TK], cnt, tmask, off [E], the route record, row_tok [TK].
size_t decode_b_lds_words(const Dims& d) {
  return 3 * (size_t)d.TK() + 3 * (size_t)d.E + route_words(d.TK(), d.T);
}

bool decode_fast_ok(const Dims& d) {
  const size_t lds_b = (size_t)d.T * d.H * 2 + decode_b_lds_words(d) * 4;
  return d.T >= 1 && d.T <= kDecodeMaxT && d.H <= 2048 && d.F <= 512 && d.Fs <= 512 &&
         d.E <= 1024 && d.K <= 32 && lds_b <= kDecLdsMax;
}

hipError_t launch_decode_layer(const Dims& d, const moe_layer_desc_t& desc, const uint16_t* x,
                               const DecodeBufs& b, float* out, hipStream_t s, int phase,
                               const StackFuse* sf) {
  DecodeArgs p;
  p.x = sf ? sf->x : x;
  p.rin = sf ? sf->resid : nullptr;
  p.xw = sf ? sf->x : nullptr;
  p.eps = sf ? sf->eps : 0.0f;
  p.acc_out = sf ? 1 : 0;
  if (sf) out = sf->resid;
  p.router_w = desc.router_w;
  p.router_bias = desc.router_bias;
  p.wg = d.Fs > 0 ? desc.shared_gate_w : nullptr;
  p.gate = desc.gate;
  p.up = desc.up;
  p.down = desc.down;
  p.sh_gate = desc.sh_gate;
  p.sh_up = desc.sh_up;
  p.sh_down = desc.sh_down;
  p.T = d.T;
  p.H = d.H;
  p.E = d.E;
  p.K = d.K;
  p.F = d.F;
  p.Fs = d.Fs;
  p.b = b;
  p.out = out;
  const size_t lds_x = (size_t)d.T * d.H * 2;
  const size_t lds_b = lds_x + decode_b_lds_words(d) * 4;
  const size_t a_bytes = ((size_t)d.TK() * d.F + (size_t)d.T * d.Fs) * 2;
  // C: one wave per entry (the selected experts and the shared one), at most 16 waves
  const int ent_max = d.TK() + (d.Fs > 0 ? 1 : 0);
  const int nwc = ent_max < 16 ? ent_max : 16;
  const int rgc = dec_c_rows(d.T <= 1 ? 1 : 2);
  const size_t lds_c_route = (route_words(d.TK(), d.T) + d.TK()) * 4 + (size_t)nwc * rgc * 64 * 4;
  const bool a_lds = d.T > 1 && a_bytes + lds_c_route <= kDecCLdsMax;
  const size_t lds_c = (a_lds ? a_bytes : 0) + lds_c_route;
  const int nA = d.E + (d.Fs > 0 ? 1 + d.Fs : 0);
  const dim3 gA((nA + 3) / 4), gB(device_cus() * 4 / (kDecBWaves / 4)), gC(d.H / (4 * rgc)), blk(256);
  const dim3 blkB(64 * kDecBWaves), blkC(64 * nwc);
#define MOE_DEC(TCV, NJV)                                                        \
  do {                                                                           \
    if (phase < 0 || phase == 0)                                                 \
      hipLaunchKernelGGL((k_dec_a<TCV>), gA, blk, lds_x + 16, s, p);             \
    if (phase < 0 || phase == 1)                                                 \
      hipLaunchKernelGGL((k_dec_b<TCV, NJV>), gB, blkB, lds_b, s, p);            \
    if (phase < 0 || phase == 2) {                                               \
      if (a_lds)                                                                 \
        hipLaunchKernelGGL((k_dec_c<TCV, true>), gC, blkC, lds_c, s, p);         \
      else                                                                       \
        hipLaunchKernelGGL((k_dec_c<TCV, false>), gC, blkC, lds_c, s, p);        \
    }                                                                            \
  } while (0)
#define MOE_DEC_T(NJV) \
  if (d.T <= 1)        \
    MOE_DEC(1, NJV);   \
  else if (d.T <= 2)   \
    MOE_DEC(2, NJV);   \
  else if (d.T <= 4)   \
    MOE_DEC(4, NJV);   \
  else if (d.T <= 8)   \
    MOE_DEC(8, NJV);   \
  else                 \
    MOE_DEC(16, NJV);
  if (d.E <= 64) {
    MOE_DEC_T(1)
  } else if (d.E <= 256) {
    MOE_DEC_T(4)
  } else if (d.E <= 512) {
    MOE_DEC_T(8)
  } else {
    MOE_DEC_T(16)
  }
#undef MOE_DEC_T
#undef MOE_DEC
  return hipGetLastError();
}

}  // namespace moe
