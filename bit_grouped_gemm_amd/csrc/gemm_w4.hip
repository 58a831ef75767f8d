// Prefill grouped GEMM with 4-bit group-64 affine weights dequantised inside the kernel.
//
// "Perplexity's Lily: A Breakthrough Local Inference Engine Tailored Exclusively for Apple
// Silicon": section "The Model: Qwen3.6-35B-A3B in Focus" (weights w = scale*q + bias per
// group of 64, rebuilt one tile at a time into bf16 for the tensor operations, fp32
// accumulation, never expanded in memory) and section "How It Works: Prefill and Decode
// Strategies" (the 4-bit reconstruction happens inside the grouped GEMM).
//
// Layout of the work (gfx950, wave64, v_mfma_f32_32x32x16_bf16):
//  * One workgroup = one block-map tile (up to 128 rows of one expert) x one column slice.
//    4 waves split the COLUMNS; every wave runs over all row tiles of the block, so each
//    dequantised weight fragment is built once and reused for up to 4 MFMAs (128 rows).
//  * Activation rows (gathered through the permutation for gate/up) are staged per K-chunk
//    of 128 inputs into LDS (double buffered, rows padded to 272 B against bank conflicts)
//    and shared by the 4 waves.
//  * Packed weights go straight from HBM to registers: lane l owns column (l & 31) of a
//    32-column tile and half (l >> 5) of the chunk's 128 inputs, i.e. one group of 64 =
//    8 words (two 16-byte loads), with one scale and one bias. For MFMA step s (16 inputs)
//    the lane dequantises its word s into the 8 bf16 of the B operand; the A operand
//    takes the same 8 inputs from LDS. Chunk c+1's weights and activations are in flight
//    while chunk c is multiplied.
//  * Gate/up mode: each wave owns 32 gate columns and the same 32 up columns, so SwiGLU
//    is applied in registers and only the bf16 activation A = silu(G) * U is stored.
//  * Down mode: each wave owns 64 output columns (two tiles); the epilogue stores fp32 rows
//    or adds topk_w * row into the token's output with fp32 atomics.
#include "moe_internal.h"

namespace moe {

namespace {
constexpr int kKC = 128;               // inputs per K-chunk (two quantisation groups)
constexpr int kLdsRow = kKC + 8;       // bf16 elements per LDS row (16 B pad)
constexpr int kLdsBuf = kBlockM * kLdsRow;
constexpr int kMT = kBlockM / 32;      // row tiles per block
}  // namespace

template <int MODE>
__global__ __launch_bounds__(256, 2) void k_gemm_w4(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * kLdsBuf];

  const int j = blockIdx.y;
  if (j >= *p.num_blocks) return;
  const int4 blk = p.blocks[j];
  const int e = blk.x, m0 = blk.y, m_len = blk.z, row0 = blk.w;
  const bool shared = e >= p.E;
  const int kdim = shared ? p.kdim_shared : p.kdim_routed;
  const int ncols = shared ? p.n_shared : p.n_routed;
  constexpr int kSliceCols = (MODE == kGateUp) ? 128 : 256;
  const int slice0 = blockIdx.x * kSliceCols;
  if (slice0 >= ncols) return;  // uniform over the workgroup, before any barrier

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

  // ---- activation rows staged by this thread: rows (tid>>4) + 16*i, 16-byte segment tid&15
  const int seg = tid & 15;
  const uint16_t* abase = shared ? p.a_shared : p.a_routed;
  uint32_t aoff[8];  // element offset of the row in abase, or ~0u past the block's rows
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = (tid >> 4) + 16 * i;
    aoff[i] = ~0u;
    if (r < m_len) {
      int arow;
      if (MODE == kGateUp)
        arow = shared ? (m0 + r) : (p.sorted_slots[row0 + r] / p.K);
      else
        arow = shared ? (m0 + r) : (row0 + r);
      aoff[i] = (uint32_t)arow * (uint32_t)kdim;
    }
  }

  const int nchunks = (kdim + kKC - 1) / kKC;
  uint4 areg[8];
  auto load_a = [&](int c) {
    const int k = c * kKC + seg * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      areg[i] = make_uint4(0, 0, 0, 0);
      if (aoff[i] != ~0u && k < kdim)
        areg[i] = *reinterpret_cast<const uint4*>(abase + aoff[i] + k);
    }
  };
  auto store_a = [&](int buf) {
    uint16_t* base = lds + buf * kLdsBuf + seg * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = (tid >> 4) + 16 * i;
      *reinterpret_cast<uint4*>(base + r * kLdsRow) = areg[i];
    }
  };

  uint4 qc[4], qn[4];  // [tile0 lo, tile0 hi, tile1 lo, tile1 hi] words of this lane's group
  float sc[2], bc[2], sn[2], bn[2];
  auto load_b = [&](int c, uint4* q, float* s, float* b) {
    const int g = c * 2 + half;  // this lane's group
    if (wave_active && g < gpr) {
      const int w4 = g * 2;  // uint4 index of the group's first word (8 words = 2 x uint4)
      q[0] = q0[w4];
      q[1] = q0[w4 + 1];
      q[2] = q1[w4];
      q[3] = q1[w4 + 1];
      s[0] = bf16_to_f32(s0p[g]);
      b[0] = bf16_to_f32(b0p[g]);
      s[1] = bf16_to_f32(s1p[g]);
      b[1] = bf16_to_f32(b1p[g]);
    } else {  // beyond Kin (last half chunk) or idle wave: weights are exactly zero
      q[0] = q[1] = q[2] = q[3] = make_uint4(0, 0, 0, 0);
      s[0] = s[1] = b[0] = b[1] = 0.0f;
    }
  };

  f32x16_t acc[kMT][2];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt) {
    acc[mt][0] = f32x16_t{};
    acc[mt][1] = f32x16_t{};
  }

  load_a(0);
  load_b(0, qc, sc, bc);
  store_a(0);
  __syncthreads();

  for (int c = 0; c < nchunks; ++c) {
    const bool more = c + 1 < nchunks;
    if (more) {
      load_a(c + 1);
      load_b(c + 1, qn, sn, bn);
    }
    if (wave_active) {
      const uint16_t* abuf = lds + (c & 1) * kLdsBuf + n * kLdsRow + half * 64;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const uint32_t w0 = (s < 4) ? ((const uint32_t*)&qc[0])[s] : ((const uint32_t*)&qc[1])[s - 4];
        const uint32_t w1 = (s < 4) ? ((const uint32_t*)&qc[2])[s] : ((const uint32_t*)&qc[3])[s - 4];
        uint32_t b0[4], b1[4];
        dequant8(w0, sc[0], bc[0], b0);
        dequant8(w1, sc[1], bc[1], b1);
        const bf16x8_t bv0 = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<uint4*>(b0));
        const bf16x8_t bv1 = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<uint4*>(b1));
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
          if (mt * 32 < m_len) {
            const bf16x8_t av =
                *reinterpret_cast<const bf16x8_t*>(abuf + mt * 32 * kLdsRow + s * 8);
            acc[mt][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv0, acc[mt][0], 0, 0, 0);
            acc[mt][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv1, acc[mt][1], 0, 0, 0);
          }
        }
      }
    }
    if (more) store_a((c + 1) & 1);
    __syncthreads();
    if (more) {
#pragma unroll
      for (int i = 0; i < 4; ++i) qc[i] = qn[i];
      sc[0] = sn[0];
      sc[1] = sn[1];
      bc[0] = bn[0];
      bc[1] = bn[1];
    }
  }
  if (!wave_active) return;

  // ---- epilogue. D layout (32x32): register i of lane l is row 8*(i/4) + 4*(l/32) + i%4,
  // column l%32 of the tile.
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt) {
    if (mt * 32 >= m_len) continue;
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

hipError_t launch_gemm_w4(int mode, const GemmParams& p, int max_blocks, hipStream_t s) {
  const int ncols = p.n_routed > p.n_shared ? p.n_routed : p.n_shared;
  const int slice = (mode == kGateUp) ? 128 : 256;
  dim3 grid((ncols + slice - 1) / slice, max_blocks);
  if (max_blocks <= 0) return hipSuccess;
  if (mode == kGateUp)
    hipLaunchKernelGGL(k_gemm_w4<kGateUp>, grid, dim3(256), 0, s, p);
  else if (mode == kDownStore)
    hipLaunchKernelGGL(k_gemm_w4<kDownStore>, grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(k_gemm_w4<kDownAtomic>, grid, dim3(256), 0, s, p);
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
