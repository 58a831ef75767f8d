// Prefill grouped GEMM with 4-bit group-64 affine weights dequantised inside the kernel.
//
// "Perplexity's Lily: A Breakthrough Local Inference Engine Tailored Exclusively for Apple
// Silicon": section "The Model: Qwen3.6-35B-A3B in Focus" (weights w = scale*q + bias per
// group of 64, rebuilt one tile at a time into bf16 for the tensor operations, fp32
// accumulation, never expanded in memory) and section "How It Works: Prefill and Decode
// Strategies" (the 4-bit reconstruction happens inside the grouped GEMM).
//
// Layout of the work (gfx950, wave64, v_mfma_f32_32x32x16_bf16):
//  * One workgroup = one block-map tile (up to 128 rows of one expert) x one column slice,
//    two workgroups per CU (two waves per SIMD, so one wave's dequantisation overlaps the
//    other's MFMAs). 4 waves split the COLUMNS; every wave runs over all row tiles of the
//    block, so each dequantised weight fragment is built once and used by up to 4 MFMAs.
//    The K loop and the epilogue are compiled for 1..4 active row tiles.
//  * Activation rows (gathered through the permutation for gate/up) are copied per K-chunk
//    of 128 inputs straight from global memory into LDS with global_load_lds_dwordx4 (no
//    staging registers), into two buffers that alternate between chunks. A row is 256 B;
//    its 16-byte segments are XOR-swizzled by the row index, so the A-fragment reads of the
//    MFMAs (32 rows, one segment each) are free of bank conflicts.
//  * Packed weights go straight from HBM to registers: lane l owns column (l & 31) of a
//    32-column tile and half (l >> 5) of the chunk's 128 inputs, i.e. one group of 64 =
//    8 words (two 16-byte loads), with one scale and one bias, kept as raw bf16 bits until
//    the chunk is multiplied. For MFMA step s (16 inputs) the lane dequantises its word s
//    into the 8 bf16 of the B operand; the A operand takes the same 8 inputs from LDS.
//    Chunk c+1's weights and activations are in flight while chunk c is multiplied.
//  * Gate/up mode: each wave owns 32 gate columns and the same 32 up columns, so SwiGLU
//    is applied in registers and only the bf16 activation A = silu(G) * U is stored.
//  * Down mode: each wave owns 64 output columns (two tiles); the epilogue stores fp32 rows
//    or adds topk_w * row into the token's output with fp32 atomics.
#include "moe_internal.h"

namespace moe {

namespace {
constexpr int kKC = 128;                  // inputs per K-chunk (two quantisation groups)
constexpr int kRowBytes = kKC * 2;        // one activation row of a chunk in LDS
constexpr int kBufBytes = kBlockM * kRowBytes;
constexpr int kMT = kBlockM / 32;         // row tiles per block
constexpr int kCopies = kBufBytes / 1024 / 4;  // 1 KiB LDS copies per wave and chunk
}  // namespace

// One K-chunk (8 MFMA steps of 16 inputs) for NT active row tiles: per step the lane's words
// of both column tiles are dequantised once and used by the 2*NT MFMAs of that step.
// a_lane: this lane's row (tile 0) in the chunk buffer; seg0: the swizzled segment of its
// step-0 inputs (step s uses segment seg0 ^ s).
template <int NT>
__device__ __forceinline__ void mma_chunk(const char* a_lane, int seg0, const uint4 (&q)[4],
                                          float s0, float b0, float s1, float b1,
                                          f32x16_t (&acc)[NT][2]) {
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const uint32_t w0 = (s < 4) ? ((const uint32_t*)&q[0])[s] : ((const uint32_t*)&q[1])[s - 4];
    const uint32_t w1 = (s < 4) ? ((const uint32_t*)&q[2])[s] : ((const uint32_t*)&q[3])[s - 4];
    uint32_t d0[4], d1[4];
    dequant8(w0, s0, b0, d0);
    dequant8(w1, s1, b1, d1);
    const bf16x8_t bv0 = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<uint4*>(d0));
    const bf16x8_t bv1 = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<uint4*>(d1));
    const int off = (seg0 ^ s) << 4;
    bf16x8_t av[NT];
#pragma unroll
    for (int mt = 0; mt < NT; ++mt)
      av[mt] = *reinterpret_cast<const bf16x8_t*>(a_lane + mt * 32 * kRowBytes + off);
#pragma unroll
    for (int mt = 0; mt < NT; ++mt) {
      acc[mt][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[mt], bv0, acc[mt][0], 0, 0, 0);
      acc[mt][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[mt], bv1, acc[mt][1], 0, 0, 0);
    }
    // keep each step's fragments within the step (bounds register pressure at two waves
    // per SIMD: the accumulators alone take 32*NT VGPRs)
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One block-map tile with NT active row tiles (1..kMT): the whole K loop and the epilogue are
// compiled per NT, so that each version keeps only the accumulators it uses.
template <int MODE, int NT>
__device__ __forceinline__ void gemm_block(const GemmParams& p, char* buf0, char* buf1, int e,
                                           int m0, int m_len, int row0, bool shared, int kdim,
                                           int ncols, int slice0) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, half = lane >> 5;
  // ---- columns owned by this wave (two 32-column tiles) and their weight rows
  int col0, col1;
  const uint32_t *qb0, *qb1;
  const uint16_t *sb0, *sb1, *bb0, *bb1;
  if (MODE == kGateUp) {
    col0 = col1 = slice0 + wave * 32 + n;
    qb0 = shared ? p.sw0.q : p.w0.q;
    sb0 = shared ? p.sw0.scale : p.w0.scale;
    bb0 = shared ? p.sw0.bias : p.w0.bias;
    qb1 = shared ? p.sw1.q : p.w1.q;
    sb1 = shared ? p.sw1.scale : p.w1.scale;
    bb1 = shared ? p.sw1.bias : p.w1.bias;
  } else {
    col0 = slice0 + wave * 64 + n;
    col1 = col0 + 32;
    qb0 = qb1 = shared ? p.sw0.q : p.w0.q;
    sb0 = sb1 = shared ? p.sw0.scale : p.w0.scale;
    bb0 = bb1 = shared ? p.sw0.bias : p.w0.bias;
  }
  const bool wave_active = (MODE == kGateUp ? slice0 + wave * 32 : slice0 + wave * 64) < ncols;
  const int wpr = kdim >> 3;   // words per weight row
  const int gpr = kdim >> 6;   // groups per weight row
  const size_t mat_rows = shared ? 0 : (size_t)e * ncols;
  const size_t r0 = mat_rows + (wave_active ? col0 : 0);
  const size_t r1 = mat_rows + (wave_active ? col1 : 0);
  const uint4* q0 = reinterpret_cast<const uint4*>(qb0 + r0 * wpr);
  const uint4* q1 = reinterpret_cast<const uint4*>(qb1 + r1 * wpr);
  const uint16_t* s0p = sb0 + r0 * gpr;
  const uint16_t* b0p = bb0 + r0 * gpr;
  const uint16_t* s1p = sb1 + r1 * gpr;
  const uint16_t* b1p = bb1 + r1 * gpr;

  // ---- activation copies: wave w issues copies J = w*kCopies + j, each 1 KiB = 4 rows of
  // 256 B. Lane i fills LDS segment (i & 15) of row 4J + (i >> 4) with global segment
  // (i & 15) ^ (row & 15). Rows past the block copy the block's first row (never stored) and
  // segments past kdim copy the row's first segment (their weights are zero), so every
  // address is in bounds and every copied value is a finite activation.
  const uint16_t* abase = shared ? p.a_shared : p.a_routed;
  auto arow_of = [&](int r) -> int {
    if (MODE == kGateUp) return shared ? (m0 + r) : (p.sorted_slots[row0 + r] / p.K);
    return shared ? (m0 + r) : (row0 + r);
  };
  const int arow0 = arow_of(0);
  uint32_t aoff[kCopies];  // element offset of this lane's row for copy j
  const int lseg = lane & 15;
#pragma unroll
  for (int j = 0; j < kCopies; ++j) {
    const int r = 4 * (wave * kCopies + j) + (lane >> 4);
    aoff[j] = (uint32_t)(r < m_len ? arow_of(r) : arow0) * (uint32_t)kdim;
  }
  auto copy_a = [&](int c, char* buf) {
#pragma unroll
    for (int j = 0; j < kCopies; ++j) {
      const int J = wave * kCopies + j;
      const int r = 4 * J + (lane >> 4);
      int k = c * kKC + 8 * (lseg ^ (r & 15));
      if (k >= kdim) k = 0;
      __builtin_amdgcn_global_load_lds(abase + aoff[j] + k, buf + J * 1024, 16, 0, 0);
    }
  };

  // Words of this lane's group for the two column tiles, and the raw bf16 scale/bias bits
  // (converted only when the chunk is multiplied, so that prefetching them does not wait).
  uint4 qc[4], qn[4];  // [tile0 lo, tile0 hi, tile1 lo, tile1 hi]
  uint32_t sbc[4], sbn[4];  // {scale0, bias0, scale1, bias1}
  auto load_b = [&](int c, uint4* q, uint32_t* sb) {
    const int g = c * 2 + half;  // this lane's group
    if (wave_active && g < gpr) {
      const int w4 = g * 2;  // uint4 index of the group's first word (8 words = 2 x uint4)
      q[0] = q0[w4];
      q[1] = q0[w4 + 1];
      q[2] = q1[w4];
      q[3] = q1[w4 + 1];
      sb[0] = s0p[g];
      sb[1] = b0p[g];
      sb[2] = s1p[g];
      sb[3] = b1p[g];
    } else {  // beyond Kin (last half chunk) or idle wave: weights are exactly zero
      q[0] = q[1] = q[2] = q[3] = make_uint4(0, 0, 0, 0);
      sb[0] = sb[1] = sb[2] = sb[3] = 0u;
    }
  };

  f32x16_t acc[NT][2];
#pragma unroll
  for (int mt = 0; mt < NT; ++mt) {
    acc[mt][0] = f32x16_t{};
    acc[mt][1] = f32x16_t{};
  }

  // this lane's A-fragment row (tile 0) and the swizzled segment of its step-0 inputs
  const int a_row_off = n * kRowBytes;
  const int seg0 = (half * 8) ^ (n & 15);
  auto multiply = [&](const char* buf, const uint4 (&q)[4], const uint32_t (&sb)[4]) {
    if (wave_active)
      mma_chunk<NT>(buf + a_row_off, seg0, q, bf16_to_f32(sb[0]), bf16_to_f32(sb[1]),
                    bf16_to_f32(sb[2]), bf16_to_f32(sb[3]), acc);
  };

  const int nchunks = (kdim + kKC - 1) / kKC;
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
    __syncthreads();                // buffer 0 is no longer being read
    if (c + 2 < nchunks) {
      copy_a(c + 2, buf0);
      load_b(c + 2, qc, sbc);
    }
    multiply(buf1, qn, sbn);
  }
  if (!wave_active) return;

  // ---- epilogue. D layout (32x32): register i of lane l is row 8*(i/4) + 4*(l/32) + i%4,
  // column l%32 of the tile.
#pragma unroll
  for (int mt = 0; mt < NT; ++mt) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = mt * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
      if (r >= m_len) continue;
      if (MODE == kGateUp) {
        const float a = silu_mul(acc[mt][0][i], acc[mt][1][i]);
        uint16_t* out = static_cast<uint16_t*>(p.out);
        const size_t o = shared ? (size_t)p.TK * p.n_routed + (size_t)(m0 + r) * ncols
                                : (size_t)(row0 + r) * ncols;
        out[o + col0] = f32_to_bf16(a);
      } else if (MODE == kDownStore) {
        float* out = static_cast<float*>(p.out) + (size_t)(row0 + r) * p.out_ld;
        out[col0] = acc[mt][0][i];
        out[col1] = acc[mt][1][i];
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
        float* out = static_cast<float*>(p.out) + (size_t)tok * p.out_ld;
        atomicAdd(out + col0, wgt * acc[mt][0][i]);
        atomicAdd(out + col1, wgt * acc[mt][1][i]);
      }
    }
  }
}

// Workgroups are dispatched round-robin over the XCDs (workgroup id mod kXcds), each with its
// own L2. The linear workgroup id is mapped so that all column slices of one block run on the
// same XCD, one after the other: the block's activation rows then come from that XCD's L2
// after the first slice has fetched them.
constexpr int kXcds = 8;

template <int MODE>
__global__ __launch_bounds__(256, 2) void k_gemm_w4(GemmParams p, int nslices) {
  // two separate arrays, so that reads of one buffer never wait for copies into the other
  __shared__ __attribute__((aligned(1024))) char lds0[kBufBytes];
  __shared__ __attribute__((aligned(1024))) char lds1[kBufBytes];

  const int xcd = blockIdx.x % kXcds, local = blockIdx.x / kXcds;
  const int j = kXcds * (local / nslices) + xcd;  // block-map entry
  const int slice = local % nslices;
  if (j >= *p.num_blocks) return;
  const int4 blk = p.blocks[j];
  const int e = blk.x, m0 = blk.y, m_len = blk.z, row0 = blk.w;
  const bool shared = e >= p.E;
  const int kdim = shared ? p.kdim_shared : p.kdim_routed;
  const int ncols = shared ? p.n_shared : p.n_routed;
  constexpr int kSliceCols = (MODE == kGateUp) ? 128 : 256;
  const int slice0 = slice * kSliceCols;
  if (slice0 >= ncols) return;  // uniform over the workgroup, before any barrier
  static_assert(kMT == 4, "the dispatch below covers 1..4 row tiles");
  switch ((m_len + 31) >> 5) {  // uniform over the workgroup
    case 1: gemm_block<MODE, 1>(p, lds0, lds1, e, m0, m_len, row0, shared, kdim, ncols, slice0); break;
    case 2: gemm_block<MODE, 2>(p, lds0, lds1, e, m0, m_len, row0, shared, kdim, ncols, slice0); break;
    case 3: gemm_block<MODE, 3>(p, lds0, lds1, e, m0, m_len, row0, shared, kdim, ncols, slice0); break;
    default: gemm_block<MODE, 4>(p, lds0, lds1, e, m0, m_len, row0, shared, kdim, ncols, slice0); break;
  }
}

hipError_t launch_gemm_w4(int mode, const GemmParams& p, int max_blocks, hipStream_t s) {
  const int ncols = p.n_routed > p.n_shared ? p.n_routed : p.n_shared;
  const int slice = (mode == kGateUp) ? 128 : 256;
  const int nslices = (ncols + slice - 1) / slice;
  if (max_blocks <= 0) return hipSuccess;
  // every (block, slice) pair of the remapping in k_gemm_w4 appears once in this grid
  const int rounds = (max_blocks + kXcds - 1) / kXcds;
  const dim3 grid(kXcds * rounds * nslices);
  if (mode == kGateUp)
    hipLaunchKernelGGL(k_gemm_w4<kGateUp>, grid, dim3(256), 0, s, p, nslices);
  else if (mode == kDownStore)
    hipLaunchKernelGGL(k_gemm_w4<kDownStore>, grid, dim3(256), 0, s, p, nslices);
  else
    hipLaunchKernelGGL(k_gemm_w4<kDownAtomic>, grid, dim3(256), 0, s, p, nslices);
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
