// Token permutation into per-expert groups: histogram, exclusive scan, stable scatter and the
// block map, all on the device with no host synchronisation.
//
// "Perplexity's Lily: A Breakthrough Local Inference Engine Tailored Exclusively for Apple
// Silicon", section "How It Works: Prefill and Decode Strategies": the histogram and the
// routing logic (prefix scan, scatter, block maps) stay inside one GPU submission, with no
// CPU synchronisation between expert layers.
//
// Slots s = t*K + k are split into chunks of kChunkSlots. Pass 1 writes one histogram row per
// chunk (plus a bin for invalid expert ids). Pass 2 (one workgroup) turns the rows into
// per-chunk starting positions, the expert offsets and the block map. Pass 3 scatters each
// chunk in slot order, so the result is stable: inside an expert, slots stay ascending.
#include "moe_internal.h"

namespace moe {

// hist row c: [E] counts of chunk c, then hist[c][E] = invalid ids in chunk c.
__global__ __launch_bounds__(256) void k_hist(const int32_t* __restrict__ idx, int TK, int E,
                                              int32_t* __restrict__ hist) {
  __shared__ int h[1025];
  for (int e = threadIdx.x; e <= E; e += 256) h[e] = 0;
  __syncthreads();
  const int s0 = blockIdx.x * kChunkSlots, s1 = min(TK, s0 + kChunkSlots);
  for (int s = s0 + threadIdx.x; s < s1; s += 256) {
    const int e = idx[s];
    atomicAdd(&h[(e >= 0 && e < E) ? e : E], 1);
  }
  __syncthreads();
  int32_t* row = hist + (size_t)blockIdx.x * (E + 1);
  for (int e = threadIdx.x; e <= E; e += 256) row[e] = h[e];
}

// Exclusive scan over a 1024-thread workgroup (wave scans, then a scan of wave totals).
__device__ int block_exclusive_scan_1024(int v, int* wave_tot, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(inc, off, 64);
    if (lane >= off) inc += o;
  }
  if (lane == 63) wave_tot[wave] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < 16; ++w) {
      const int t = wave_tot[w];
      wave_tot[w] = run;
      run += t;
    }
    *total = run;
  }
  __syncthreads();
  const int r = wave_tot[wave] + inc - v;
  __syncthreads();  // wave_tot may be reused by the caller
  return r;
}

// One workgroup of 1024 threads (E <= 1024). Converts hist rows to chunk starting positions in
// place, and writes counts, offsets, the block map and num_blocks (-1 if any id was invalid).
__global__ __launch_bounds__(1024) void k_scan(int32_t* __restrict__ hist, int nchunks, int E,
                                               int T, int K, int has_shared,
                                               int32_t* __restrict__ counts,
                                               int32_t* __restrict__ offsets,
                                               int4* __restrict__ blocks,
                                               int32_t* __restrict__ num_blocks) {
  __shared__ int wave_tot[16];
  __shared__ int total_slots, total_blocks, bad;
  const int e = threadIdx.x;
  // the rows are read eight at a time, so the latency of a row read is paid once per eight rows
  int cnt = 0;
  if (e < E)
    for (int c0 = 0; c0 < nchunks; c0 += 8) {
      int v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = c0 + i < nchunks ? hist[(size_t)(c0 + i) * (E + 1) + e] : 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) cnt += v[i];
    }
  if (threadIdx.x == 0) {
    int b = 0;
    for (int c0 = 0; c0 < nchunks; c0 += 8) {
      int v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = c0 + i < nchunks ? hist[(size_t)(c0 + i) * (E + 1) + E] : 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) b += v[i];
    }
    bad = b;
  }
  const int off = block_exclusive_scan_1024(e < E ? cnt : 0, wave_tot, &total_slots);
  if (e < E) {
    counts[e] = cnt;
    offsets[e] = off;
    int run = off;
    for (int c0 = 0; c0 < nchunks; c0 += 8) {
      int v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = c0 + i < nchunks ? hist[(size_t)(c0 + i) * (E + 1) + e] : 0;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (c0 + i < nchunks) {
          hist[(size_t)(c0 + i) * (E + 1) + e] = run;
          run += v[i];
        }
    }
  }
  const int nb = (e < E) ? (cnt + kBlockM - 1) / kBlockM : 0;
  const int boff = block_exclusive_scan_1024(nb, wave_tot, &total_blocks);
  if (e == 0) offsets[E] = total_slots;
  for (int j = 0; j < nb; ++j) {
    const int m0 = j * kBlockM;
    blocks[boff + j] = make_int4(e, m0, min(kBlockM, cnt - m0), off + m0);
  }
  const int TK = T * K;
  const int nbs = has_shared ? (T + kBlockM - 1) / kBlockM : 0;
  for (int j = threadIdx.x; j < nbs; j += 1024) {
    const int m0 = j * kBlockM;
    blocks[total_blocks + j] = make_int4(E, m0, min(kBlockM, T - m0), TK + m0);
  }
  __syncthreads();
  if (threadIdx.x == 0) *num_blocks = bad ? -1 : total_blocks + nbs;
}

// One workgroup of 4 waves per chunk; wave w takes the w-th quarter of the chunk's slots.
// Each wave first counts its quarter per expert; the counts of the lower quarters, added to
// the chunk's starting positions, give each wave its own running positions, so the quarters
// are scattered concurrently and the result is still stable. For 64 slots at a time, the
// lanes that hold the same expert are found with one ballot per bit of the expert id; a
// lane's rank among its peers is the number of lower peer lanes, and the lowest peer advances
// the expert's running position afterwards.
__global__ __launch_bounds__(256) void k_scatter(const int32_t* __restrict__ idx, int TK, int E,
                                                 int nbits, const int32_t* __restrict__ base,
                                                 int32_t* __restrict__ sorted_slots,
                                                 int32_t* __restrict__ slot_pos) {
  __shared__ int cur[4][1024];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  for (int e = tid; e < 4 * 1024; e += 256) (&cur[0][0])[e] = 0;
  __syncthreads();
  const int s0 = blockIdx.x * kChunkSlots, s1 = min(TK, s0 + kChunkSlots);
  constexpr int kQ = kChunkSlots / 4;
  const int q0 = s0 + wave * kQ, q1 = min(s1, q0 + kQ);
  // per-quarter counts (the quarter itself is the wave's own)
  for (int s = q0 + lane; s < q1; s += 64) {
    const int e = idx[s];
    if (e >= 0 && e < E) atomicAdd(&cur[wave][e], 1);
  }
  __syncthreads();
  // cur[w][e] <- chunk start of e + counts of e in quarters < w
  const int32_t* row = base + (size_t)blockIdx.x * (E + 1);
  for (int e = tid; e < E; e += 256) {
    int run = row[e];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int c = cur[w][e];
      cur[w][e] = run;
      run += c;
    }
  }
  __syncthreads();
  int* my = cur[wave];
  for (int sb = q0; sb < q1; sb += 64) {
    const int s = sb + lane;
    const int e = (s < q1) ? idx[s] : -1;
    const bool ok = e >= 0 && e < E;
    uint64_t peers = __ballot(ok);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = ok && ((e >> b) & 1);
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    const uint64_t lower = peers & ((1ull << lane) - 1ull);
    int p = 0;
    if (ok) p = my[e] + __popcll(lower);
    // the wave's own LDS accesses complete in order: every lane's read of my[e] above comes
    // before the lowest peer's update below
    if (ok && lower == 0) my[e] += __popcll(peers);
    if (ok) {
      sorted_slots[p] = s;
      slot_pos[s] = p;
    }
  }
}

// Up to kPermuteOneMax slots in one workgroup of 16 waves, with the results of the three passes
// above and no launches between them: wave w takes the w-th sixteenth of the slots (a multiple
// of 64 slots, held in registers from the first pass to the last) and counts it per expert in
// LDS; thread e then forms expert e's count, offset,
// blocks and the running position of each sixteenth (the offset plus the counts of the lower
// sixteenths); finally every wave scatters its sixteenth in slot order with the peer ranks of
// k_scatter. Inside an expert the slots therefore stay ascending, as in the three-pass path.
__global__ __launch_bounds__(1024) void k_permute_one(
    const int32_t* __restrict__ idx, int TK, int E, int T, int K, int has_shared, int nbits,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int4* __restrict__ blocks,
    int32_t* __restrict__ num_blocks, int32_t* __restrict__ sorted_slots,
    int32_t* __restrict__ slot_pos) {
  extern __shared__ int cur[];  // [16][E]
  __shared__ int wave_tot[16];
  __shared__ int total_slots, total_blocks, bad;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  for (int i = tid; i < 16 * E; i += 1024) cur[i] = 0;
  if (tid == 0) bad = 0;
  __syncthreads();
  const int per = (TK + 16 * 64 - 1) / (16 * 64) * 64;  // slots per wave
  const int q0 = wave * per, q1 = min(TK, q0 + per);
  int* my = cur + wave * E;
  // this wave's ids, all requested at once and kept in registers for the scatter (step i holds
  // slots q0 + 64i .. q0 + 64i + 63; -1 past the end), then counted per expert
  constexpr int kSteps = kPermuteOneMax / (16 * 64);
  int ev[kSteps];
#pragma unroll
  for (int i = 0; i < kSteps; ++i) {
    const int s = q0 + 64 * i + lane;
    ev[i] = (64 * i < per && s < q1) ? idx[s] : -1;
  }
  int nbad = 0;
#pragma unroll
  for (int i = 0; i < kSteps; ++i) {
    const int s = q0 + 64 * i + lane;
    if (64 * i < per && s < q1) {
      if (ev[i] >= 0 && ev[i] < E)
        atomicAdd(&my[ev[i]], 1);
      else
        ++nbad;
    }
  }
  if (nbad) atomicAdd(&bad, nbad);
  __syncthreads();
  const int ex = tid;
  int cnt = 0;
  if (ex < E)
    for (int w = 0; w < 16; ++w) cnt += cur[w * E + ex];
  const int off = block_exclusive_scan_1024(ex < E ? cnt : 0, wave_tot, &total_slots);
  if (ex < E) {
    counts[ex] = cnt;
    offsets[ex] = off;
    int run = off;
    for (int w = 0; w < 16; ++w) {
      const int c = cur[w * E + ex];
      cur[w * E + ex] = run;
      run += c;
    }
  }
  const int nb = (ex < E) ? (cnt + kBlockM - 1) / kBlockM : 0;
  const int boff = block_exclusive_scan_1024(nb, wave_tot, &total_blocks);
  if (ex == 0) offsets[E] = total_slots;
  for (int j = 0; j < nb; ++j) {
    const int m0 = j * kBlockM;
    blocks[boff + j] = make_int4(ex, m0, min(kBlockM, cnt - m0), off + m0);
  }
  const int nbs = has_shared ? (T + kBlockM - 1) / kBlockM : 0;
  for (int j = tid; j < nbs; j += 1024) {
    const int m0 = j * kBlockM;
    blocks[total_blocks + j] = make_int4(E, m0, min(kBlockM, T - m0), T * K + m0);
  }
  __syncthreads();  // the running positions are complete
  if (tid == 0) *num_blocks = bad ? -1 : total_blocks + nbs;
  // scatter in slot order
#pragma unroll
  for (int i = 0; i < kSteps; ++i) {
    if (64 * i >= per) break;  // uniform
    const int s = q0 + 64 * i + lane;
    const int e = ev[i];
    const bool ok = s < q1 && e >= 0 && e < E;
    uint64_t peers = __ballot(ok);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = ok && ((e >> b) & 1);
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    const uint64_t lower = peers & ((1ull << lane) - 1ull);
    int p = 0;
    if (ok) p = my[e] + __popcll(lower);
    // the wave's own LDS accesses complete in order: every lane's read of my[e] above comes
    // before the lowest peer's update below
    if (ok && lower == 0) my[e] += __popcll(peers);
    if (ok) {
      sorted_slots[p] = s;
      slot_pos[s] = p;
    }
  }
}

// Decode routing in one workgroup (T <= 16 tokens, E <= 1024): wave t selects token t's top-k
// (softmax-renormalised) and its shared gate, then the workgroup builds counts, offsets,
// the block map (one block per active expert: an expert holds at most T < 128 rows) and the
// stable permutation. Inside an expert, slot (t, k) has rank #{t' < t routed to it}, read off
// a per-expert token bitmask.
template <int NJ>
__global__ __launch_bounds__(1024) void k_route_small(
    const float* __restrict__ logits, const uint16_t* __restrict__ x, const float* __restrict__ wg,
    int T, int E, int K, int H, int32_t* __restrict__ idx, float* __restrict__ wout,
    float* __restrict__ sgate, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_slots, int32_t* __restrict__ slot_pos, int4* __restrict__ blocks,
    int32_t* __restrict__ num_blocks) {
  __shared__ int cnt[1024];
  __shared__ unsigned mask[1024];
  __shared__ int off_s[1024];
  __shared__ int wave_tot[16];
  __shared__ int total_slots, total_blocks;
  const int tid = threadIdx.x, lane = tid & 63, t = tid >> 6;
  cnt[tid] = 0;
  mask[tid] = 0u;
  __syncthreads();
  float my_v = -INFINITY;
  int my_i = 0;
  if (t < T) {
    float my_w;
    wave_topk<NJ>(logits + (size_t)t * E, E, K, lane, my_v, my_i, my_w);
    if (lane < K) {
      idx[t * K + lane] = my_i;
      wout[t * K + lane] = my_w;
      atomicAdd(&cnt[my_i], 1);
      atomicOr(&mask[my_i], 1u << t);
    }
    if (wg != nullptr) {
      const float g = shared_gate_logit(x + (size_t)t * H, wg, H, lane);
      if (lane == 0) sgate[t] = 1.0f / (1.0f + __expf(-g));
    }
  }
  __syncthreads();
  const int c = tid < E ? cnt[tid] : 0;
  const int off = block_exclusive_scan_1024(c, wave_tot, &total_slots);
  const int bo = block_exclusive_scan_1024(c > 0 ? 1 : 0, wave_tot, &total_blocks);
  if (tid < E) {
    counts[tid] = c;
    offsets[tid] = off;
    off_s[tid] = off;
    if (c > 0) blocks[bo] = make_int4(tid, 0, c, off);
  }
  if (tid == 0) {
    offsets[E] = total_slots;
    int nb = total_blocks;
    if (wg != nullptr) blocks[nb++] = make_int4(E, 0, T, T * K);
    *num_blocks = nb;
  }
  __syncthreads();
  if (t < T && lane < K) {
    const int pos = off_s[my_i] + __popc(mask[my_i] & ((1u << t) - 1u));
    sorted_slots[pos] = t * K + lane;
    slot_pos[t * K + lane] = pos;
  }
}

hipError_t launch_route_small(const float* logits, const uint16_t* x, const float* wg,
                              const Dims& d, int32_t* idx, float* w, float* sgate,
                              const moe_plan_t& plan, hipStream_t s) {
#define MOE_RS(NJ)                                                                           \
  hipLaunchKernelGGL(k_route_small<NJ>, dim3(1), dim3(1024), 0, s, logits, x, wg, d.T, d.E, d.K, \
                     d.H, idx, w, sgate, plan.counts, plan.offsets, plan.sorted_slots,            \
                     plan.slot_pos, reinterpret_cast<int4*>(plan.blocks), plan.num_blocks)
  if (d.E <= 64)
    MOE_RS(1);
  else if (d.E <= 256)
    MOE_RS(4);
  else if (d.E <= 512)
    MOE_RS(8);
  else
    MOE_RS(16);
#undef MOE_RS
  return hipGetLastError();
}

hipError_t launch_permute(const int32_t* idx, const Dims& d, bool shared, int32_t* hist,
                          const moe_plan_t& plan, hipStream_t s) {
  const int TK = d.TK();
  const int nchunks = (TK + kChunkSlots - 1) / kChunkSlots;
  int nbits = 0;
  while ((1 << nbits) < d.E) ++nbits;
  if (TK <= kPermuteOneMax) {
    hipLaunchKernelGGL(k_permute_one, dim3(1), dim3(1024), (size_t)16 * d.E * sizeof(int), s, idx,
                       TK, d.E, d.T, d.K, shared ? 1 : 0, nbits, plan.counts, plan.offsets,
                       reinterpret_cast<int4*>(plan.blocks), plan.num_blocks, plan.sorted_slots,
                       plan.slot_pos);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_hist, dim3(nchunks), dim3(256), 0, s, idx, TK, d.E, hist);
  hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, s, hist, nchunks, d.E, d.T, d.K,
                     shared ? 1 : 0, plan.counts, plan.offsets,
                     reinterpret_cast<int4*>(plan.blocks), plan.num_blocks);
  hipLaunchKernelGGL(k_scatter, dim3(nchunks), dim3(256), 0, s, idx, TK, d.E, nbits, hist,
                     plan.sorted_slots, plan.slot_pos);
  return hipGetLastError();
}

}  // namespace moe
