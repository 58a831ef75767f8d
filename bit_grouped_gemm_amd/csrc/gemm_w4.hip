// Prefill grouped GEMM with 4-bit group-64 affine weights dequantised inside the kernel.
//
// "Perplexity's Lily: A Breakthrough Local Inference Engine Tailored Exclusively for Apple
// Silicon": section "The Model: Qwen3.6-35B-A3B in Focus" (weights w = scale*q + bias per
// group of 64, rebuilt one tile at a time into bf16 for the tensor operations, fp32
// accumulation, never expanded in memory) and section "How It Works: Prefill and Decode
// Strategies" (the 4-bit reconstruction happens inside the grouped GEMM).
//
// Layout of the work (gfx950, wave64, v_mfma_f32_32x32x16_bf16):
//  * One workgroup = one block-map tile (up to 256 rows of one expert) x one column slice,
//    one workgroup per CU and one wave per SIMD. The 4 waves split the COLUMNS; every wave
//    runs over all (up to 8) row tiles of the block, so each dequantised weight fragment is
//    built once and feeds up to 16 MFMAs: dequantisation costs under two VALU instructions
//    per MFMA, and the accumulators (up to 256 registers) live in the AGPR half of the
//    register file. The K loop and the epilogue are compiled for 1..8 active row tiles.
//  * The K loop runs over chunks of 64 inputs (one quantisation group). Activation rows
//    (gathered through the permutation for gate/up) are copied per chunk straight from global
//    memory into LDS with global_load_lds_dwordx4 (no staging registers). Two LDS buffers
//    keep the next chunk in flight while one is multiplied: measured on the full-size layer,
//    deeper rings (up to seven chunks in flight) made the loop slower, not faster, because the
//    extra copies in flight delayed the chunk being waited for. A chunk row is 128 B; its 16-byte
//    segment g is stored at g ^ ((row >> 1) & 7), so the A-fragment reads of the MFMAs
//    (32 rows, one segment each) are free of bank conflicts.
//  * Packed weights go straight from HBM to registers: lane l owns column (l & 31) of a
//    32-column tile and half (l >> 5) of the chunk's 64 inputs, i.e. four words (one 16-byte
//    load) with the group's scale and bias, kept as raw bf16 bits until the chunk is
//    multiplied. MFMA step s (16 inputs) takes word s of both halves: the lane dequantises it
//    into the 8 bf16 of the B operand; the A operand takes the same 8 inputs from LDS.
//    Inside a chunk the A reads and the dequantisation of step s+1 are issued among the MFMAs
//    of step s (the compiler's schedule inside each step).
//  * Gate/up mode: each wave owns 32 gate columns and the same 32 up columns, so SwiGLU
//    is applied in registers and only the bf16 activation A = silu(G) * U is stored.
//  * The down projection has a kernel of its own (below): its K is short, so it trades the
//    deep pipeline for two workgroups per CU.
#include "moe_internal.h"

namespace moe {

namespace {
constexpr int kKC = 64;                          // inputs per K-chunk (one quantisation group)
constexpr int kRowBytes = kKC * 2;               // one activation row of a chunk in LDS
constexpr int kMT = kBlockM / 32;                // row tiles per block
constexpr int kArrRows = 128;                    // rows of a chunk per LDS array
constexpr int kArrBytes = kArrRows * kRowBytes;  // 16 KiB
constexpr int kNArr = 4;                         // LDS arrays (64 KiB)
static_assert(kMT == 8 && kBlockM == 2 * kArrRows, "a chunk of a full block spans two arrays");
}  // namespace

// The LDS arrays of the kernel (indexed with compile-time constants only, or through pick()).
struct LdsArrays {
  char* a[kNArr];
  __device__ __forceinline__ char* pick(int i) const {  // i uniform, not a compile-time constant
    return i == 0 ? a[0] : i == 1 ? a[1] : i == 2 ? a[2] : a[3];
  }
};

// The packed words of one chunk for this lane's NC column tiles, and the raw bf16 bits of the
// chunk's scale and bias per tile.
template <int NC>
struct BChunk {
  uint4 q[NC];
};
template <int NC>
struct SChunk {
  uint32_t s[NC], b[NC];  // bf16 bits in the low half
};

// One K-chunk (4 MFMA steps of 16 inputs) for NT active row tiles and NC column tiles.
// a_lo / a_hi: this lane's row in the chunk's first / second array (row tiles 0-3 / 4-7);
// seg0: its swizzled segment for step 0 (step s uses seg0 ^ s).
template <int NT, int NC>
__device__ __forceinline__ void mma_chunk(const char* a_lo, const char* a_hi, int seg0,
                                          const BChunk<NC>& b, const SChunk<NC>& sb,
                                          f32x16_t (&acc)[NT][NC]) {
  float sc[NC], bi[NC];
  uint32_t w[NC][4];
#pragma unroll
  for (int t = 0; t < NC; ++t) {
    sc[t] = bf16_to_f32(sb.s[t] & 0xFFFFu);
    bi[t] = bf16_to_f32(sb.b[t] & 0xFFFFu);
    w[t][0] = b.q[t].x;
    w[t][1] = b.q[t].y;
    w[t][2] = b.q[t].z;
    w[t][3] = b.q[t].w;
  }
  bf16x8_t av[2][NT], bv[2][NC];
  auto fetch = [&](int s, int slot) {
#pragma unroll
    for (int mt = 0; mt < NT; ++mt)
      av[slot][mt] = *reinterpret_cast<const bf16x8_t*>((mt < 4 ? a_lo : a_hi) +
                                                        (mt & 3) * 32 * kRowBytes + ((seg0 ^ s) << 4));
#pragma unroll
    for (int t = 0; t < NC; ++t) {
      uint32_t d[4];
      dequant8(w[t][s], sc[t], bi[t], d);
      bv[slot][t] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<uint4*>(d));
    }
  };
  fetch(0, 0);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int cur = s & 1;
    if (s < 3) fetch(s + 1, cur ^ 1);
#pragma unroll
    for (int mt = 0; mt < NT; ++mt)
#pragma unroll
      for (int t = 0; t < NC; ++t)
        acc[mt][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[cur][mt], bv[cur][t], acc[mt][t], 0, 0, 0);
    // the compiler interleaves the next step's LDS reads and dequantisation with these MFMAs
    // (measured slightly faster than a prescribed one-MFMA, four-VALU, one-read pattern)
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One block-map tile with NT active row tiles (1..kMT) and NC column tiles per wave.
// Gate/up: column tile 2t is gate column-tile t of the wave and 2t+1 the same up columns.
template <int MODE, int NT, int NC, int SW, int NARR>
__device__ __forceinline__ void gemm_block(const GemmParams& p, const LdsArrays& lds, int e,
                                           int m0, int m_len, int row0, bool shared, int kdim,
                                           int ncols, int slice0) {
  static_assert(MODE != kGateUp || NC % 2 == 0, "gate/up tiles come in pairs");
  constexpr int kColsPerWave = (MODE == kGateUp ? NC / 2 : NC) * 32;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, half = lane >> 5;
  const int wcol0 = slice0 + wave * kColsPerWave;  // first output column of the wave
  const int wpr = kdim >> 3;   // words per weight row
  const int gpr = kdim >> 6;   // groups per weight row (= chunks)
  const size_t mat_rows = shared ? 0 : (size_t)e * ncols;

  // ---- the wave's column tiles: output column of tile t for this lane, whether the tile is
  // inside the matrix (columns come in multiples of 32), and the weight rows it reads (rows of
  // tiles past the matrix read row 0 of the expert: valid memory, never stored)
  int col[NC];
  bool tval[NC];
  const uint4* qp[NC];
  const uint16_t* sp[NC];
  const uint16_t* bp[NC];
#pragma unroll
  for (int t = 0; t < NC; ++t) {
    const bool up = MODE == kGateUp && (t & 1);
    const int ct = MODE == kGateUp ? (t >> 1) : t;  // tile of output columns
    col[t] = wcol0 + ct * 32 + n;
    tval[t] = wcol0 + ct * 32 < ncols;
    // pointers selected as values (a reference picked at run time into the argument block
    // would be read with vector loads)
    const uint32_t* wq = up ? (shared ? p.sw1.q : p.w1.q) : (shared ? p.sw0.q : p.w0.q);
    const uint16_t* ws = up ? (shared ? p.sw1.scale : p.w1.scale) : (shared ? p.sw0.scale : p.w0.scale);
    const uint16_t* wb = up ? (shared ? p.sw1.bias : p.w1.bias) : (shared ? p.sw0.bias : p.w0.bias);
    const size_t r = mat_rows + (tval[t] ? col[t] : 0);
    // this lane's 16-byte word quad of chunk c is uint4 number 2c + half of its row
    qp[t] = reinterpret_cast<const uint4*>(wq + r * wpr) + half;
    sp[t] = ws + r * gpr;
    bp[t] = wb + r * gpr;
  }
  const bool wave_active = tval[0];

  // ---- chunk slots. Blocks of up to 4 row tiles use one 16 KiB array per chunk, larger
  // blocks two (rows 0-127, 128-255). Separate arrays let the compiler see that reads of one
  // slot never depend on copies into another. Blocks of one or two row tiles have little work
  // per chunk, so a chunk's HBM round trip would dominate: they keep three chunks in flight
  // (four slots); taller blocks keep one (two slots), which measured faster for them.
  static_assert(NARR == kNArr, "up to four chunk slots of one array or two of two arrays");
  constexpr int kNB = NT <= 2 ? 4 : 2;
  auto slot_lo = [&](int k) -> char* { return NT <= 4 ? lds.a[k] : lds.a[2 * k]; };
  auto slot_hi = [&](int k) -> char* { return NT <= 4 ? lds.a[k] : lds.a[2 * k + 1]; };

  // ---- activation copies: the block's 32*NT rows in 4*NT copies of 1 KiB = 8 rows of 128 B;
  // wave w issues copies J = w + 4j, j < NT (copies 16.. go to the slot's second array).
  // Lane i fills LDS segment (i & 7) of row 8J + (i >> 3) with global segment
  // (i & 7) ^ ((row >> 1) & 7). Rows past the block copy the block's first row (never
  // stored), so every address is in bounds and every copied value is a finite activation.
  const uint16_t* abase = shared ? p.a_shared : p.a_routed;
  auto arow_of = [&](int r) -> int {
    if (MODE == kGateUp) return shared ? (m0 + r) : (p.sorted_slots[row0 + r] / p.K);
    return shared ? (m0 + r) : (row0 + r);
  };
  const int arow0 = arow_of(0);
  const uint16_t* asrc[NT];  // this lane's source (row and swizzled segment) for copy j
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int r = 8 * (wave + 4 * j) + (lane >> 3);
    const int ar = r < m_len ? arow_of(r) : arow0;
    asrc[j] = abase + (size_t)ar * kdim + 8 * ((lane & 7) ^ ((r >> 1) & 7));
  }
  // Chunk c's activations into slot k and weights into bq. Past the last chunk the last one is
  // requested again (into a slot nobody reads any more), so the number of requests in flight
  // is the same at every step and no load is conditional.
  auto issue = [&](int c, int k, BChunk<NC>& bq) {
    c = c < gpr ? c : gpr - 1;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int J = wave + 4 * j;
      char* dst = J < 16 ? slot_lo(k) + J * 1024 : slot_hi(k) + (J - 16) * 1024;
      __builtin_amdgcn_global_load_lds(asrc[j] + c * kKC, dst, 16, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < NC; ++t) bq.q[t] = qp[t][2 * c];
  };
  // Scales and biases. SW > 0: a row has exactly 2*SW groups (SW a multiple of 4, so rows are
  // 16-byte aligned); they are loaded once, 16 bytes at a time, as SW words per tile; word i
  // holds groups 2i, 2i+1, and the words are shifted down as the K loop advances, so that
  // chunk c + k of an unrolled step reads word k / 2. SW = 0: each chunk's pair is loaded with
  // the chunk.
  constexpr bool SU = SW > 0;
  static_assert(SW % 4 == 0, "16-byte scale rows");
  uint32_t sw[NC][SU ? SW : 1], bw[NC][SU ? SW : 1];
  if constexpr (SU) {
#pragma unroll
    for (int t = 0; t < NC; ++t)
#pragma unroll
      for (int i = 0; i < SW / 4; ++i) {
        const uint4 vs = reinterpret_cast<const uint4*>(sp[t])[i];
        const uint4 vb = reinterpret_cast<const uint4*>(bp[t])[i];
        sw[t][4 * i + 0] = vs.x; sw[t][4 * i + 1] = vs.y; sw[t][4 * i + 2] = vs.z; sw[t][4 * i + 3] = vs.w;
        bw[t][4 * i + 0] = vb.x; bw[t][4 * i + 1] = vb.y; bw[t][4 * i + 2] = vb.z; bw[t][4 * i + 3] = vb.w;
      }
  }
  SChunk<NC> sq[SU ? 1 : 8];  // per-chunk scales (not SU), slot-indexed like bq
  auto issue_s = [&](int c, int k) {
    if constexpr (!SU) {
      c = c < gpr ? c : gpr - 1;
#pragma unroll
      for (int t = 0; t < NC; ++t) {
        sq[k].s[t] = sp[t][c];
        sq[k].b[t] = bp[t][c];
      }
    }
  };
  // scale/bias of chunk c0 + k, c0 the loop body's first chunk (SU: words already shifted;
  // not SU: k < kNB is the chunk's slot)
  auto scales_of = [&](int k) -> SChunk<NC> {
    SChunk<NC> r;
    if constexpr (SU) {
#pragma unroll
      for (int t = 0; t < NC; ++t) {
        r.s[t] = (k & 1) ? (sw[t][k >> 1] >> 16) : sw[t][k >> 1];
        r.b[t] = (k & 1) ? (bw[t][k >> 1] >> 16) : bw[t][k >> 1];
      }
    } else {
      r = sq[k];
    }
    return r;
  };

  f32x16_t acc[NT][NC];
#pragma unroll
  for (int mt = 0; mt < NT; ++mt)
#pragma unroll
    for (int t = 0; t < NC; ++t) acc[mt][t] = f32x16_t{};

  // this lane's A-fragment row (tile 0) and the swizzled segment of its step-0 inputs
  const int a_row_off = n * kRowBytes;
  const int seg0 = (half * 4) ^ ((n >> 1) & 7);
  auto multiply = [&](int k, const BChunk<NC>& bq, const SChunk<NC>& sb) {
    if (wave_active)
      mma_chunk<NT, NC>(slot_lo(k) + a_row_off, slot_hi(k) + a_row_off, seg0, bq, sb, acc);
  };
  // Chunk c is complete for this wave once only the kNB - 2 later chunks' requests are
  // pending; after the barrier every wave's copies of chunk c are in LDS, and every wave is
  // done reading the slot the next copies go to (its reads fed MFMAs issued before the
  // barrier). A plain s_barrier: __syncthreads() would add a fence that waits for every
  // request in flight, which would drain the prefetch at every chunk. The empty asm
  // statements keep the compiler from moving memory accesses across the barrier.
  auto wait_chunk = [&]() {
    // vmcnt = the later chunks' requests (NT copies, NC word loads and, not SU, 2*NC scale
    // loads each), in bits 3:0 and 15:14; expcnt and lgkmcnt are not waited for
    constexpr int v = (kNB - 2) * (NT + (SU ? 1 : 3) * NC);
    static_assert(v <= 63, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((v & 15) | ((v >> 4) << 14) | (7 << 4) | (15 << 8));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  const int nchunks = gpr;
  BChunk<NC> bq[kNB];
  static_assert(SU || kNB <= 8, "per-chunk scale slots");
#pragma unroll
  for (int k = 0; k < kNB - 1; ++k) {
    issue(k, k, bq[k]);
    issue_s(k, k);
  }
  // With preloaded scales the loop body covers kU = 8 chunks, so the scale words move to the
  // front once per 8 chunks (4 words) instead of once per kNB chunks.
  constexpr int kU = SU ? 8 : kNB;
  static_assert(kU % kNB == 0 && (!SU || SW % (kU / 2) == 0), "whole slot rounds per body");
  for (int c = 0; c < nchunks; c += kU) {
#pragma unroll
    for (int kk = 0; kk < kU; ++kk) {
      const int k = kk % kNB;  // slot of chunk c + kk (c is a multiple of kNB)
      if (c + kk >= nchunks) break;
      wait_chunk();
      issue(c + kk + kNB - 1, (k + kNB - 1) % kNB, bq[(k + kNB - 1) % kNB]);
      issue_s(c + kk + kNB - 1, (k + kNB - 1) % kNB);
      multiply(k, bq[k], scales_of(kk));
    }
    if constexpr (SU) {  // the next kU chunks' scale words move to the front
#pragma unroll
      for (int t = 0; t < NC; ++t)
#pragma unroll
        for (int i = 0; i + kU / 2 < SW; ++i) {
          sw[t][i] = sw[t][i + kU / 2];
          bw[t][i] = bw[t][i + kU / 2];
        }
    }
  }
  // every request issued above has landed, and every wave is done with the chunk buffers
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (!wave_active) return;

  // ---- epilogue. D layout (32x32): register i of lane l is row 8*(i/4) + 4*(l/32) + i%4,
  // column l%32 of the tile. The wave's output tile is staged in its own chunk buffer (row r's
  // 16-byte segments permuted by (r >> 2), so that rows r and r + 4, written by the two halves
  // of the wave, fall in different banks) and written back in 16-byte pieces.
  char* tile = lds.pick(wave);
  static_assert(MODE == kGateUp, "the down projection has its own kernel");
  {
    constexpr int kPairs = NC / 2;
    constexpr int kRB = kPairs * 64;      // bytes per staged row (bf16)
    constexpr int kSegs = kRB / 16;
    static_assert(NT * 32 * kRB <= kArrBytes, "staged tile fits an array");
#pragma unroll
    for (int mt = 0; mt < NT; ++mt)
#pragma unroll
      for (int pt = 0; pt < kPairs; ++pt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = mt * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
          const int c = pt * 32 + n;
          const int seg = (c >> 3) ^ ((r >> 2) & (kSegs - 1));
          *reinterpret_cast<uint16_t*>(tile + r * kRB + seg * 16 + 2 * (c & 7)) =
              f32_to_bf16(silu_mul(acc[mt][2 * pt][i], acc[mt][2 * pt + 1][i]));
        }
    uint16_t* out = static_cast<uint16_t*>(p.out);
    uint16_t* orow = shared ? out + (size_t)p.TK * p.n_routed + (size_t)m0 * ncols
                            : out + (size_t)row0 * ncols;
    constexpr int kRowsPerPass = 64 / kSegs;
    const int q = lane % kSegs;  // this lane's 16-byte piece of a row
    const bool qval = wcol0 + 8 * q < ncols;
    orow += wcol0 + 8 * q;
#pragma unroll
    for (int pass = 0; pass < NT * 32 / kRowsPerPass; ++pass) {
      const int r = pass * kRowsPerPass + lane / kSegs;
      const int seg = q ^ ((r >> 2) & (kSegs - 1));
      const uint4 v = *reinterpret_cast<const uint4*>(tile + r * kRB + seg * 16);
      if (r < m_len && qval) *reinterpret_cast<uint4*>(orow + (size_t)r * ncols) = v;
    }
  }
}

// Workgroups are dispatched round-robin over the XCDs (workgroup id mod kXcds), each with its
// own L2. The linear workgroup id is mapped so that all column slices of one block run on the
// same XCD, one after the other: the block's activation rows then come from that XCD's L2
// after the first slice has fetched them.
constexpr int kXcds = 8;

// Gate/up: one full block-map tile (up to 256 rows) per workgroup, one workgroup per CU.
__global__ __launch_bounds__(256, 1) void k_gemm_w4_gate_up(GemmParams p, int nslices) {
  constexpr int MODE = kGateUp;
  // separate arrays, so that reads of one slot never wait for copies into another
  __shared__ __attribute__((aligned(1024))) char lds0[kArrBytes];
  __shared__ __attribute__((aligned(1024))) char lds1[kArrBytes];
  __shared__ __attribute__((aligned(1024))) char lds2[kArrBytes];
  __shared__ __attribute__((aligned(1024))) char lds3[kArrBytes];
  const LdsArrays lds{{lds0, lds1, lds2, lds3}};

  const int xcd = blockIdx.x % kXcds, local = blockIdx.x / kXcds;
  const int jd = kXcds * (local / nslices) + xcd;  // dispatch position
  const int slice = local % nslices;
  const int nb = *p.num_blocks;
  if (jd >= nb) return;
  // The shared expert's blocks (the last nsh entries, each a full block of every token) are
  // dispatched first and the routed blocks after them, so that the longest workgroups do not
  // start last and leave a tail with most CUs idle.
  const int nsh = p.n_shared > 0 ? (p.TK / p.K + kBlockM - 1) / kBlockM : 0;
  const int j = jd < nsh ? nb - nsh + jd : jd - nsh;  // block-map entry
  const int4 blk = p.blocks[j];
  const int e = blk.x, m0 = blk.y, m_len = blk.z, row0 = blk.w;
  const bool shared = e >= p.E;
  const int kdim = shared ? p.kdim_shared : p.kdim_routed;
  const int ncols = shared ? p.n_shared : p.n_routed;
  const int slice0 = slice * 128;
  if (slice0 >= ncols) return;  // uniform over the workgroup, before any barrier
  // scales loaded up front for the 2048-input rows of the full-size layer (32 groups)
  const bool su = kdim == 2048;
#define MOE_GEMM_BLOCK(NTV)                                                                      \
  do {                                                                                           \
    if (su)                                                                                      \
      gemm_block<MODE, NTV, 2, 16, kNArr>(p, lds, e, m0, m_len, row0, shared, kdim, ncols,        \
                                          slice0);                                               \
    else                                                                                         \
      gemm_block<MODE, NTV, 2, 0, kNArr>(p, lds, e, m0, m_len, row0, shared, kdim, ncols,         \
                                         slice0);                                                \
  } while (0)
  switch ((m_len + 31) >> 5) {  // uniform over the workgroup
    case 1: MOE_GEMM_BLOCK(1); break;
    case 2: MOE_GEMM_BLOCK(2); break;
    case 3: MOE_GEMM_BLOCK(3); break;
    case 4: MOE_GEMM_BLOCK(4); break;
    case 5: MOE_GEMM_BLOCK(5); break;
    case 6: MOE_GEMM_BLOCK(6); break;
    case 7: MOE_GEMM_BLOCK(7); break;
    default: MOE_GEMM_BLOCK(8); break;
  }
#undef MOE_GEMM_BLOCK
}

// Work unit u of the small-batch kernels (units are dispatched in order of u, round-robin over
// the XCDs) -> block-map entry j and piece hb: first every piece of the shared expert's tiles
// (tall: T rows), then the first piece of every routed tile, then the second pieces, and so
// on. The tall tiles' pieces then start in the first round, spread over all XCDs, instead of
// trailing the grid on the XCDs of their tiles; units past the last piece return at once.
__device__ __forceinline__ bool small_unit(int u, int nb, int nsh, int pieces, int& j, int& hb) {
  const int ns = nsh * pieces;
  if (u < ns) {
    j = nb - nsh + u / pieces;
    hb = u % pieces;
    return true;
  }
  const int nr = nb - nsh, r = u - ns;
  if (nr <= 0) return false;
  hb = r / nr;
  j = r % nr;
  return hb < pieces;
}

// Gate/up for small batches (few rows per expert): block-map tiles are cut into pieces of at
// most 64 rows (two row tiles), one per workgroup, and two workgroups share a CU, so that one
// wave's dequantisation (most of the work when a chunk feeds only one or two row tiles) runs
// while the other wave waits for memory or issues MFMAs. Units are ordered by small_unit.
constexpr int kGUSRows = 64;
__global__ __launch_bounds__(256, 2) void k_gemm_w4_gate_up_small(GemmParams p, int nslices) {
  constexpr int MODE = kGateUp;
  __shared__ __attribute__((aligned(1024))) char lds0[kArrBytes];
  __shared__ __attribute__((aligned(1024))) char lds1[kArrBytes];
  __shared__ __attribute__((aligned(1024))) char lds2[kArrBytes];
  __shared__ __attribute__((aligned(1024))) char lds3[kArrBytes];
  const LdsArrays lds{{lds0, lds1, lds2, lds3}};

  const int nb = *p.num_blocks;
  const int xcd = blockIdx.x % kXcds, local = blockIdx.x / kXcds;
  const int slice = local % nslices;
  constexpr int kPieces = kBlockM / kGUSRows;
  const int nsh = p.n_shared > 0 ? (p.TK / p.K + kBlockM - 1) / kBlockM : 0;
  int j, hb;  // the unit's block-map entry and piece (all slices of a unit on one XCD)
  if (!small_unit(kXcds * (local / nslices) + xcd, nb, nsh, kPieces, j, hb)) return;
  const int4 blk = p.blocks[j];
  const int e = blk.x;
  const int m_len = blk.z - kGUSRows * hb;
  if (m_len <= 0) return;
  const int m0 = blk.y + kGUSRows * hb, row0 = blk.w + kGUSRows * hb;
  const bool shared = e >= p.E;
  const int kdim = shared ? p.kdim_shared : p.kdim_routed;
  const int ncols = shared ? p.n_shared : p.n_routed;
  const int slice0 = slice * 128;
  if (slice0 >= ncols) return;  // uniform over the workgroup, before any barrier
  const int ml = m_len < kGUSRows ? m_len : kGUSRows;
  const bool su = kdim == 2048;
  if (ml > 32) {
    if (su) gemm_block<MODE, 2, 2, 16, kNArr>(p, lds, e, m0, ml, row0, shared, kdim, ncols, slice0);
    else gemm_block<MODE, 2, 2, 0, kNArr>(p, lds, e, m0, ml, row0, shared, kdim, ncols, slice0);
  } else {
    if (su) gemm_block<MODE, 1, 2, 16, kNArr>(p, lds, e, m0, ml, row0, shared, kdim, ncols, slice0);
    else gemm_block<MODE, 1, 2, 0, kNArr>(p, lds, e, m0, ml, row0, shared, kdim, ncols, slice0);
  }
}

// ============================================================================ down
// Down projection (K = the FFN width: a few chunks, so the time to the first chunk matters
// more than the depth of the pipeline). Block-map tiles are split into pieces of at most 128
// rows, one per workgroup; two workgroups share a CU (two waves per SIMD), so one
// workgroup's first loads and epilogue overlap the other's MFMAs. K-chunks of 128 inputs
// (two quantisation groups): lane half h owns group 2c + h of its columns (8 words, two
// 16-byte loads), and MFMA step s takes word s of that group on both halves; the A operand
// takes the same inputs from LDS (row segment 8h + s, XOR-swizzled by the row). Chunk c + 1 is
// in flight while chunk c is multiplied. Each wave owns 64 output columns (two tiles).
namespace {
constexpr int kDKC = 128;                         // inputs per K-chunk
constexpr int kDRowBytes = kDKC * 2;              // one activation row of a chunk in LDS
constexpr int kDRows = kBlockM / 2;               // rows per workgroup (half a block)
constexpr int kDBufBytes = kDRows * kDRowBytes;   // 32 KiB
}  // namespace

// One K-chunk (8 MFMA steps of 16 inputs) for NT row tiles and the wave's two column tiles.
// Software-pipelined so that the dequantisation can run between MFMAs of the same wave (on
// gfx950 a wave's VALU work overlaps its MFMAs only when the two are interleaved): tile 0's
// MFMAs of step s are grouped with tile 1's dequantisation of step s, and tile 1's MFMAs with
// tile 0's dequantisation and the A-fragment reads of step s + 1; the compiler orders each group.
// Every accumulator takes the same MFMAs in the same order as a step-by-step loop.
template <int NT>
__device__ __forceinline__ void down_mma_chunk(const char* a_lane, int seg0, const uint4 (&q)[4],
                                               float s0, float b0, float s1, float b1,
                                               f32x16_t (&acc)[NT][2]) {
  auto deq = [&](int t, int s) -> bf16x8_t {
    const uint4& v = q[2 * t + (s >> 2)];
    const uint32_t w = (s & 3) == 0 ? v.x : (s & 3) == 1 ? v.y : (s & 3) == 2 ? v.z : v.w;
    uint32_t d[4];
    dequant8(w, t ? s1 : s0, t ? b1 : b0, d);
    return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<uint4*>(d));
  };
  auto read_a = [&](int s, bf16x8_t (&av)[NT]) {
#pragma unroll
    for (int mt = 0; mt < NT; ++mt)
      av[mt] = *reinterpret_cast<const bf16x8_t*>(a_lane + mt * 32 * kDRowBytes + ((seg0 ^ s) << 4));
  };
  bf16x8_t av[NT];
  read_a(0, av);
  bf16x8_t bv0 = deq(0, 0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const bf16x8_t bv1 = deq(1, s);
#pragma unroll
    for (int mt = 0; mt < NT; ++mt)
      acc[mt][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[mt], bv0, acc[mt][0], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    bf16x8_t avn[NT], bvn;
    if (s < 7) {
      bvn = deq(0, s + 1);
      read_a(s + 1, avn);
    }
#pragma unroll
    for (int mt = 0; mt < NT; ++mt)
      acc[mt][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[mt], bv1, acc[mt][1], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    if (s < 7) {
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) av[mt] = avn[mt];
      bv0 = bvn;
    }
  }
}
// PR: rows of the piece a workgroup owns (128, or 32 for the small-batch kernel); the two
// chunk buffers are PR rows of 256 B each.
template <int MODE, int NT, int PR = kDRows>
__device__ __forceinline__ void down_block(const GemmParams& p, char* buf0, char* buf1, int e,
                                           int m0, int m_len, int row0, bool shared, int kdim,
                                           int ncols, int slice0) {
  static_assert(NT * 32 <= PR, "the row tiles fit the piece");
  constexpr int kBuf = PR * kDRowBytes;     // bytes per chunk buffer
  constexpr int kCP = kBuf / 1024 / 4;      // 1 KiB LDS copies per wave and chunk
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, half = lane >> 5;
  const int col0 = slice0 + wave * 64 + n, col1 = col0 + 32;
  const uint32_t* qb = shared ? p.sw0.q : p.w0.q;
  const uint16_t* sb = shared ? p.sw0.scale : p.w0.scale;
  const uint16_t* bb = shared ? p.sw0.bias : p.w0.bias;
  const bool wave_active = slice0 + wave * 64 < ncols;
  const bool tile1 = slice0 + wave * 64 + 32 < ncols;  // columns come in multiples of 32
  const int wpr = kdim >> 3;  // words per weight row
  const int gpr = kdim >> 6;  // groups per weight row
  const size_t mat_rows = shared ? 0 : (size_t)e * ncols;
  const size_t r0 = mat_rows + (wave_active ? col0 : 0);
  const size_t r1 = mat_rows + (tile1 ? col1 : 0);
  const uint4* q0 = reinterpret_cast<const uint4*>(qb + r0 * wpr);
  const uint4* q1 = reinterpret_cast<const uint4*>(qb + r1 * wpr);
  const uint16_t* s0p = sb + r0 * gpr;
  const uint16_t* b0p = bb + r0 * gpr;
  const uint16_t* s1p = sb + r1 * gpr;
  const uint16_t* b1p = bb + r1 * gpr;

  // ---- activation copies: wave w issues copies J = w*kCP + j, each 1 KiB = 4 rows of
  // 256 B. Lane i fills LDS segment (i & 15) of row 4J + (i >> 4) with global segment
  // (i & 15) ^ (row & 15). Rows past the tile copy its first row (never stored) and segments
  // past kdim copy the row's first segment (their weights are zero), so every address is in
  // bounds and every copied value is a finite activation.
  const uint16_t* abase = shared ? p.a_shared : p.a_routed;
  auto arow_of = [&](int r) -> int { return shared ? (m0 + r) : (row0 + r); };
  const int arow0 = arow_of(0);
  uint32_t aoff[kCP];  // element offset of this lane's row for copy j
  const int lseg = lane & 15;
#pragma unroll
  for (int j = 0; j < kCP; ++j) {
    const int r = 4 * (wave * kCP + j) + (lane >> 4);
    aoff[j] = (uint32_t)(r < m_len ? arow_of(r) : arow0) * (uint32_t)kdim;
  }
  auto copy_a = [&](int c, char* buf) {
#pragma unroll
    for (int j = 0; j < kCP; ++j) {
      const int J = wave * kCP + j;
      const int r = 4 * J + (lane >> 4);
      int k = c * kDKC + 8 * (lseg ^ (r & 15));
      if (k >= kdim) k = 0;
      __builtin_amdgcn_global_load_lds(abase + aoff[j] + k, buf + J * 1024, 16, 0, 0);
    }
  };

  // Words of this lane's group for the two column tiles, and the raw bf16 scale/bias bits.
  uint4 qc[4], qn[4];       // [tile0 lo, tile0 hi, tile1 lo, tile1 hi]
  uint32_t sbc[4], sbn[4];  // {scale0, bias0, scale1, bias1}
  auto load_b = [&](int c, uint4* q, uint32_t* sbv) {
    const int g = c * 2 + half;  // this lane's group
    if (wave_active && g < gpr) {
      const int w4 = g * 2;  // uint4 index of the group's first word (8 words = 2 x uint4)
      q[0] = q0[w4];
      q[1] = q0[w4 + 1];
      q[2] = q1[w4];
      q[3] = q1[w4 + 1];
      sbv[0] = s0p[g];
      sbv[1] = b0p[g];
      sbv[2] = s1p[g];
      sbv[3] = b1p[g];
    } else {  // beyond Kin (last half chunk) or idle wave: weights are exactly zero
      q[0] = q[1] = q[2] = q[3] = make_uint4(0, 0, 0, 0);
      sbv[0] = sbv[1] = sbv[2] = sbv[3] = 0u;
    }
  };

  f32x16_t acc[NT][2];
#pragma unroll
  for (int mt = 0; mt < NT; ++mt) {
    acc[mt][0] = f32x16_t{};
    acc[mt][1] = f32x16_t{};
  }
  const int a_row_off = n * kDRowBytes;
  const int seg0 = (half * 8) ^ (n & 15);
  auto multiply = [&](const char* buf, const uint4 (&q)[4], const uint32_t (&sbv)[4]) {
    if (wave_active)
      down_mma_chunk<NT>(buf + a_row_off, seg0, q, bf16_to_f32(sbv[0]), bf16_to_f32(sbv[1]),
                         bf16_to_f32(sbv[2]), bf16_to_f32(sbv[3]), acc);
  };

  const int nchunks = (kdim + kDKC - 1) / kDKC;
  copy_a(0, buf0);
  load_b(0, qc, sbc);
  for (int c = 0; c < nchunks; c += 2) {
    // chunk c: buffer 0, registers qc
    __builtin_amdgcn_s_waitcnt(0);  // this wave's copies and loads for chunk c are complete
    __syncthreads();                // ... and every wave's; buffer 1 is no longer being read
    if (c + 1 < nchunks) {
      copy_a(c + 1, buf1);
      load_b(c + 1, qn, sbn);
    }
    multiply(buf0, qc, sbc);
    if (c + 1 >= nchunks) break;
    // chunk c + 1: buffer 1, registers qn
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // buffer 0 is no longer being read
    if (c + 2 < nchunks) {
      copy_a(c + 2, buf0);
      load_b(c + 2, qc, sbc);
    }
    multiply(buf1, qn, sbn);
  }
  __syncthreads();  // every wave is done reading the activation buffers
  if (!wave_active) return;

  // ---- epilogue. D layout (32x32): register i of lane l is row 8*(i/4) + 4*(l/32) + i%4,
  // column l%32 of the tile. The expert outputs stay fp32 (the fp32 accumulators themselves).
  // Store: register i of the 64 lanes covers 32 consecutive columns of two rows, i.e. two
  // full 128-byte lines of Y, so the stores go straight from the accumulators.
  // Atomic: out[t] += weight * Y row, the weighted combine fused into the epilogue.
  float* const outf = static_cast<float*>(p.out);
#pragma unroll
  for (int mt = 0; mt < NT; ++mt) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = mt * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
      if (r >= m_len) continue;
      if constexpr (MODE == kDownStore) {
        float* orow = outf + (size_t)(row0 + r) * p.out_ld;
        orow[col0] = acc[mt][0][i];
        if (tile1) orow[col1] = acc[mt][1][i];
      } else {
        int tok;
        float wgt;
        if (shared) {
          tok = m0 + r;
          wgt = p.shared_gate[tok];
        } else {
          const int slot = p.sorted_slots[row0 + r];
          tok = slot / p.K;
          wgt = p.topk_w[slot];
        }
        float* out = outf + (size_t)tok * p.out_ld;
        atomicAdd(out + col0, wgt * acc[mt][0][i]);
        if (tile1) atomicAdd(out + col1, wgt * acc[mt][1][i]);
      }
    }
  }
}

template <int MODE>
__global__ __launch_bounds__(256, 2) void k_gemm_w4_down(GemmParams p, int nslices) {
  // two separate arrays, so that reads of one buffer never wait for copies into the other
  __shared__ __attribute__((aligned(1024))) char lds0[kDBufBytes];
  __shared__ __attribute__((aligned(1024))) char lds1[kDBufBytes];

  // Work units are the first 128-row pieces of all tiles (in block-map order), then the second
  // pieces: a tile of more than 128 rows adds a unit in the second half of the grid, and the
  // units without rows (the second pieces of short tiles) come last.
  const int nb = *p.num_blocks;
  const int xcd = blockIdx.x % kXcds, local = blockIdx.x / kXcds;
  const int hd = kXcds * (local / nslices) + xcd;  // work unit
  const int slice = local % nslices;
  const int rounds = (gridDim.x / kXcds) / nslices;  // units per half of the grid / kXcds
  const int half_units = kXcds * (rounds / 2);
  const int hb = hd >= half_units ? 1 : 0;
  const int j = hd - hb * half_units;
  if (j >= nb) return;
  const int4 blk = p.blocks[j];
  const int e = blk.x;
  const int m_len = blk.z - kDRows * hb;
  if (m_len <= 0) return;
  const int m0 = blk.y + kDRows * hb, row0 = blk.w + kDRows * hb;
  const bool shared = e >= p.E;
  const int kdim = shared ? p.kdim_shared : p.kdim_routed;
  const int ncols = shared ? p.n_shared : p.n_routed;
  const int slice0 = slice * 256;
  if (slice0 >= ncols) return;  // uniform over the workgroup, before any barrier
  const int ml = m_len < kDRows ? m_len : kDRows;
  switch ((ml + 31) >> 5) {  // uniform over the workgroup
    case 1: down_block<MODE, 1>(p, lds0, lds1, e, m0, ml, row0, shared, kdim, ncols, slice0); break;
    case 2: down_block<MODE, 2>(p, lds0, lds1, e, m0, ml, row0, shared, kdim, ncols, slice0); break;
    case 3: down_block<MODE, 3>(p, lds0, lds1, e, m0, ml, row0, shared, kdim, ncols, slice0); break;
    default: down_block<MODE, 4>(p, lds0, lds1, e, m0, ml, row0, shared, kdim, ncols, slice0); break;
  }
}

// Down projection for small batches (the same condition as k_gemm_w4_gate_up_small): pieces of
// at most 32 rows (one row tile) with 8 KiB chunk buffers, so that four workgroups share a CU
// and one workgroup's dequantisation overlaps the others' loads. Units are ordered by
// small_unit; units without rows return at once.
template <int MODE>
__global__ __launch_bounds__(256, 4) void k_gemm_w4_down_small(GemmParams p, int nslices) {
  constexpr int kRowsS = 32;
  constexpr int kPieces = kBlockM / kRowsS;
  __shared__ __attribute__((aligned(1024))) char lds0[kRowsS * kDRowBytes];
  __shared__ __attribute__((aligned(1024))) char lds1[kRowsS * kDRowBytes];
  const int nb = *p.num_blocks;
  const int xcd = blockIdx.x % kXcds, local = blockIdx.x / kXcds;
  const int slice = local % nslices;
  const int nsh = p.n_shared > 0 ? (p.TK / p.K + kBlockM - 1) / kBlockM : 0;
  int j, hb;  // the unit's block-map entry and piece (all slices of a unit on one XCD)
  if (!small_unit(kXcds * (local / nslices) + xcd, nb, nsh, kPieces, j, hb)) return;
  const int4 blk = p.blocks[j];
  const int e = blk.x;
  const int m_len = blk.z - kRowsS * hb;
  if (m_len <= 0) return;
  const int m0 = blk.y + kRowsS * hb, row0 = blk.w + kRowsS * hb;
  const bool shared = e >= p.E;
  const int kdim = shared ? p.kdim_shared : p.kdim_routed;
  const int ncols = shared ? p.n_shared : p.n_routed;
  const int slice0 = slice * 256;
  if (slice0 >= ncols) return;  // uniform over the workgroup, before any barrier
  const int ml = m_len < kRowsS ? m_len : kRowsS;
  down_block<MODE, 1, kRowsS>(p, lds0, lds1, e, m0, ml, row0, shared, kdim, ncols, slice0);
}

hipError_t launch_gemm_w4(int mode, const GemmParams& p, int max_blocks, hipStream_t s) {
  const int ncols = p.n_routed > p.n_shared ? p.n_routed : p.n_shared;
  const int slice = (mode == kGateUp) ? 128 : 256;
  const int nslices = (ncols + slice - 1) / slice;
  if (max_blocks <= 0) return hipSuccess;
  // every (block, slice[, half]) of the remapping in the kernels appears once in the grid
  const int rounds = (max_blocks + kXcds - 1) / kXcds;
  if (mode == kGateUp) {
    if ((size_t)p.TK <= (size_t)32 * p.E) {
      // small batches (at most 32 rows per expert on average): 64-row pieces, two per CU
      hipLaunchKernelGGL(k_gemm_w4_gate_up_small, dim3(kXcds * (kBlockM / kGUSRows) * rounds * nslices),
                         dim3(256), 0, s, p, nslices);
    } else {
      hipLaunchKernelGGL(k_gemm_w4_gate_up, dim3(kXcds * rounds * nslices), dim3(256), 0, s, p,
                         nslices);
    }
  } else {
    if ((size_t)p.TK <= (size_t)32 * p.E) {
      // small batches: 32-row pieces, four workgroups per CU
      const dim3 grid(kXcds * (kBlockM / 32) * rounds * nslices);
      if (mode == kDownStore)
        hipLaunchKernelGGL(k_gemm_w4_down_small<kDownStore>, grid, dim3(256), 0, s, p, nslices);
      else
        hipLaunchKernelGGL(k_gemm_w4_down_small<kDownAtomic>, grid, dim3(256), 0, s, p, nslices);
      return hipGetLastError();
    }
    // two halves: the first pieces of all tiles, then the second pieces
    const dim3 grid(kXcds * 2 * rounds * nslices);
    if (mode == kDownStore)
      hipLaunchKernelGGL(k_gemm_w4_down<kDownStore>, grid, dim3(256), 0, s, p, nslices);
    else
      hipLaunchKernelGGL(k_gemm_w4_down<kDownAtomic>, grid, dim3(256), 0, s, p, nslices);
  }
  return hipGetLastError();
}

__global__ void k_fill_zero(float4* __restrict__ p, size_t n4) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n4) p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

hipError_t launch_fill_zero(float* p, size_t n, hipStream_t s) {
  const size_t n4 = n / 4;  // callers pass multiples of 4 (H is a multiple of 64)
  if (n4 == 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s,
                     reinterpret_cast<float4*>(p), n4);
  return hipGetLastError();
}

}  // namespace moe
