// Decode path (T <= 16): bandwidth-bound GEMV kernels that stream only the selected experts'
// packed weights with coalesced 16-byte loads and dequantise them in registers.
//
// "Perplexity's Lily: A Breakthrough Local Inference Engine Tailored Exclusively for Apple
// Silicon", section "How It Works: Prefill and Decode Strategies" (batch-1 decode barely reuses
// weights, so it is bound by bandwidth) and the FAQ entry on the decode bottleneck (moving
// weights per token). Each selected weight is read from HBM exactly once per layer call.
//
// The weights are rounded to bf16 after the exact fp32 FMA s*q+b, as in the prefill kernels,
// so both paths compute the same products; products with the bf16 activations are exact and
// summed in fp32 (v_dot2_f32_bf16).
#include "moe_internal.h"

namespace moe {

// ---------------------------------------------------------------- gate/up + SwiGLU
// Grid: x = 16-row slices of the expert's intermediate dimension, y = block-map entries (one
// per active expert plus the shared expert). Each wave owns 4 intermediate rows f and reads
// the gate row f and the up row f (1 KiB each at H = 2048, one 16-byte load per lane).
template <int TC>
__global__ __launch_bounds__(256) void k_dec_gateup(
    const int4* __restrict__ blocks, const int* __restrict__ num_blocks,
    const int32_t* __restrict__ sorted_slots, const uint16_t* __restrict__ x, int H, int E, int K,
    int F, int Fs, int TK, moe_w4_t gate, moe_w4_t up, moe_w4_t sh_gate, moe_w4_t sh_up,
    uint16_t* __restrict__ a_out) {
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];  // [m_len][H]
  const int j = blockIdx.y;
  if (j >= *num_blocks) return;
  const int4 blk = blocks[j];
  const int e = blk.x, m0 = blk.y, m_len = blk.z, row0 = blk.w;
  const bool shared = e >= E;
  const int Ne = shared ? Fs : F;
  const int f_base = blockIdx.x * 16;
  if (f_base >= Ne) return;  // uniform, before the barrier

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t* gq = shared ? sh_gate.q : gate.q + (size_t)e * F * (H >> 3);
  const uint32_t* uq = shared ? sh_up.q : up.q + (size_t)e * F * (H >> 3);
  const uint16_t* gs = shared ? sh_gate.scale : gate.scale + (size_t)e * F * (H >> 6);
  const uint16_t* gb = shared ? sh_gate.bias : gate.bias + (size_t)e * F * (H >> 6);
  const uint16_t* us = shared ? sh_up.scale : up.scale + (size_t)e * F * (H >> 6);
  const uint16_t* ub = shared ? sh_up.bias : up.bias + (size_t)e * F * (H >> 6);

  const int U = H >> 5;  // 32-input units per row (one 16-byte load)
  uint4 wgq[4], wuq[4];
  float sg[4], bg[4], su[4], bu[4];
  auto load_w = [&](int u) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int f = min(f_base + wave * 4 + r, Ne - 1);
      wgq[r] = reinterpret_cast<const uint4*>(gq + (size_t)f * (H >> 3))[u];
      wuq[r] = reinterpret_cast<const uint4*>(uq + (size_t)f * (H >> 3))[u];
      const size_t g = (size_t)f * (H >> 6) + (u >> 1);
      sg[r] = bf16_to_f32(gs[g]);
      bg[r] = bf16_to_f32(gb[g]);
      su[r] = bf16_to_f32(us[g]);
      bu[r] = bf16_to_f32(ub[g]);
    }
  };
  if (lane < U) load_w(lane);  // in flight while the token rows are staged

  // stage the block's token rows
  const int h8 = H >> 3;
  for (int v = threadIdx.x; v < m_len * h8; v += 256) {
    const int i = v / h8, c = v - i * h8;
    const int tok = shared ? (m0 + i) : (sorted_slots[row0 + i] / K);
    reinterpret_cast<uint4*>(xs)[v] = reinterpret_cast<const uint4*>(x + (size_t)tok * H)[c];
  }
  __syncthreads();

  float pg[4][TC], pu[4][TC];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int i = 0; i < TC; ++i) pg[r][i] = pu[r][i] = 0.0f;

  for (int u = lane; u < U; u += 64) {
    if (u != lane) load_w(u);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      uint32_t wg[16], wu[16];
      dequant8(wgq[r].x, sg[r], bg[r], wg + 0);
      dequant8(wgq[r].y, sg[r], bg[r], wg + 4);
      dequant8(wgq[r].z, sg[r], bg[r], wg + 8);
      dequant8(wgq[r].w, sg[r], bg[r], wg + 12);
      dequant8(wuq[r].x, su[r], bu[r], wu + 0);
      dequant8(wuq[r].y, su[r], bu[r], wu + 4);
      dequant8(wuq[r].z, su[r], bu[r], wu + 8);
      dequant8(wuq[r].w, su[r], bu[r], wu + 12);
#pragma unroll
      for (int i = 0; i < TC; ++i) {
        if (i < m_len) {
          const uint4* xr = reinterpret_cast<const uint4*>(xs + (size_t)i * H + u * 32);
          float ag = pg[r][i], au = pu[r][i];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const uint4 xv = xr[v];
            ag = dot2_bf16(xv.x, wg[4 * v + 0], ag);
            ag = dot2_bf16(xv.y, wg[4 * v + 1], ag);
            ag = dot2_bf16(xv.z, wg[4 * v + 2], ag);
            ag = dot2_bf16(xv.w, wg[4 * v + 3], ag);
            au = dot2_bf16(xv.x, wu[4 * v + 0], au);
            au = dot2_bf16(xv.y, wu[4 * v + 1], au);
            au = dot2_bf16(xv.z, wu[4 * v + 2], au);
            au = dot2_bf16(xv.w, wu[4 * v + 3], au);
          }
          pg[r][i] = ag;
          pu[r][i] = au;
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int f = f_base + wave * 4 + r;
#pragma unroll
    for (int i = 0; i < TC; ++i) {
      if (i < m_len) {
        const float g = wave_sum(pg[r][i]);
        const float uu = wave_sum(pu[r][i]);
        if (lane == 0 && f < Ne) {
          const size_t o = shared ? (size_t)TK * F + (size_t)(m0 + i) * Fs
                                  : (size_t)(row0 + i) * F;
          a_out[o + f] = f32_to_bf16(silu_mul(g, uu));
        }
      }
    }
  }
}

hipError_t launch_dec_gateup(const Dims& d, const moe_layer_desc_t& desc, const uint16_t* x,
                             const moe_plan_t& plan, int max_blocks, uint16_t* a_out,
                             hipStream_t s) {
  const int nmax = d.F > d.Fs ? d.F : d.Fs;
  dim3 grid((nmax + 15) / 16, max_blocks);
  const size_t lds = (size_t)d.T * d.H * sizeof(uint16_t);
  const int4* blocks = reinterpret_cast<const int4*>(plan.blocks);
#define MOE_DEC_GU(TCV)                                                                      \
  hipLaunchKernelGGL(k_dec_gateup<TCV>, grid, dim3(256), lds, s, blocks, plan.num_blocks,     \
                     plan.sorted_slots, x, d.H, d.E, d.K, d.F, d.Fs, d.TK(), desc.gate, desc.up, \
                     desc.sh_gate, desc.sh_up, a_out)
  if (d.T <= 1)
    MOE_DEC_GU(1);
  else if (d.T <= 2)
    MOE_DEC_GU(2);
  else if (d.T <= 4)
    MOE_DEC_GU(4);
  else if (d.T <= 8)
    MOE_DEC_GU(8);
  else
    MOE_DEC_GU(16);
#undef MOE_DEC_GU
  return hipGetLastError();
}

// ------------------------------------------------------------ down + fused combine
// Grid: 16 output rows h per workgroup; a wave owns 4 rows, one per 16-lane group. Every
// group walks the block map in order (active experts ascending, then the shared expert) and
// for each block reads the expert's down row h (256 B at F = 512) once, forms the dot product
// with each of the block's activation rows and adds it, times the token's routing weight (or
// the shared gate), into that token's accumulator. Lane (l & 15) = t holds token t's sum, so
// the order of additions is fixed: the result is deterministic.
// The weights of up to kNB blocks (4 for T > 4) are requested before any arithmetic; when the activations
// of the whole call are small (T <= 4 at F = 512) they are staged once into LDS alongside.
constexpr int kNB = 16;
constexpr int kDownLdsBytes = 40 * 1024;

template <int TC, bool kLds>
__global__ __launch_bounds__(256) void k_dec_down(
    const int4* __restrict__ blocks, const int* __restrict__ num_blocks,
    const int32_t* __restrict__ sorted_slots, const uint16_t* __restrict__ a, int H, int E, int K,
    int F, int Fs, int TK, moe_w4_t down, moe_w4_t sh_down, const float* __restrict__ topk_w,
    const float* __restrict__ sgate, int T, float* __restrict__ out) {
  extern __shared__ __attribute__((aligned(16))) uint16_t as[];  // A rows (kLds only)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = lane >> 4, sl = lane & 15;
  const int h = blockIdx.x * 16 + wave * 4 + grp;
  const int hh = h < H ? h : H - 1;
  const int nblk = *num_blocks;
  float acc = 0.0f;  // token sl's running sum for row h

  constexpr int NB = TC <= 4 ? kNB : 4;
  for (int jb = 0; jb < nblk; jb += NB) {
    int4 blk[NB];
    uint4 wq[NB];
    float ws[NB], wb[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      blk[b] = (jb + b < nblk) ? blocks[jb + b] : make_int4(-1, 0, 0, 0);
      const int e = blk[b].x;
      const bool sh = e >= E;
      const int Kd = sh ? Fs : F;
      wq[b] = make_uint4(0, 0, 0, 0);
      ws[b] = wb[b] = 0.0f;
      if (e >= 0 && sl < (Kd >> 5)) {
        const uint32_t* q = sh ? sh_down.q : down.q + (size_t)e * H * (F >> 3);
        const uint16_t* sp = sh ? sh_down.scale : down.scale + (size_t)e * H * (F >> 6);
        const uint16_t* bp = sh ? sh_down.bias : down.bias + (size_t)e * H * (F >> 6);
        wq[b] = reinterpret_cast<const uint4*>(q + (size_t)hh * (Kd >> 3))[sl];
        ws[b] = bf16_to_f32(sp[(size_t)hh * (Kd >> 6) + (sl >> 1)]);
        wb[b] = bf16_to_f32(bp[(size_t)hh * (Kd >> 6) + (sl >> 1)]);
      }
    }
    if (kLds && jb == 0) {  // all activation rows of the call: [TK][F] then [T][Fs]
      const int n16 = (TK * F + T * Fs) >> 3;
      for (int v = threadIdx.x; v < n16; v += 256)
        reinterpret_cast<uint4*>(as)[v] = reinterpret_cast<const uint4*>(a)[v];
      __syncthreads();
    }
    const uint16_t* abase = kLds ? as : a;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int e = blk[b].x;
      if (e < 0) continue;  // uniform: trailing entries of the last batch
      const bool sh = e >= E;
      const int Kd = sh ? Fs : F;
      const int m0 = blk[b].y, m_len = blk[b].z, row0 = blk[b].w;
      uint32_t w[16];
      dequant8(wq[b].x, ws[b], wb[b], w + 0);
      dequant8(wq[b].y, ws[b], wb[b], w + 4);
      dequant8(wq[b].z, ws[b], wb[b], w + 8);
      dequant8(wq[b].w, ws[b], wb[b], w + 12);
      const bool lane_has = sl < (Kd >> 5);
#pragma unroll
      for (int i = 0; i < TC; ++i) {
        if (i < m_len) {
          float part = 0.0f;
          if (lane_has) {
            const uint16_t* ar = sh ? abase + (size_t)TK * F + (size_t)(m0 + i) * Fs
                                    : abase + (size_t)(row0 + i) * F;
            const uint4* av = reinterpret_cast<const uint4*>(ar + sl * 32);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const uint4 x4 = av[v];
              part = dot2_bf16(x4.x, w[4 * v + 0], part);
              part = dot2_bf16(x4.y, w[4 * v + 1], part);
              part = dot2_bf16(x4.z, w[4 * v + 2], part);
              part = dot2_bf16(x4.w, w[4 * v + 3], part);
            }
          }
#pragma unroll
          for (int off = 8; off > 0; off >>= 1) part += __shfl_xor(part, off, 64);
          int tok;
          float wgt;
          if (sh) {
            tok = m0 + i;
            wgt = sgate[tok];
          } else {
            const int slot = sorted_slots[row0 + i];
            tok = slot / K;
            wgt = topk_w[slot];
          }
          if (sl == tok) acc = __builtin_fmaf(wgt, part, acc);
        }
      }
    }
  }
  if (h < H && sl < T) out[(size_t)sl * H + h] = acc;
}

hipError_t launch_dec_down(const Dims& d, const moe_layer_desc_t& desc, const uint16_t* a,
                           const moe_plan_t& plan, const float* topk_w, const float* sgate,
                           float* out, hipStream_t s) {
  dim3 grid((d.H + 15) / 16);
  const int4* blocks = reinterpret_cast<const int4*>(plan.blocks);
  const size_t abytes = ((size_t)d.TK() * d.F + (size_t)d.T * d.Fs) * sizeof(uint16_t);
  const bool lds = abytes <= (size_t)kDownLdsBytes;
#define MOE_DEC_DN(TCV, L)                                                                    \
  hipLaunchKernelGGL((k_dec_down<TCV, L>), grid, dim3(256), L ? abytes : 0, s, blocks,         \
                     plan.num_blocks, plan.sorted_slots, a, d.H, d.E, d.K, d.F, d.Fs, d.TK(),   \
                     desc.down, desc.sh_down, topk_w, sgate, d.T, out)
  if (d.T <= 1) {
    if (lds) MOE_DEC_DN(1, true); else MOE_DEC_DN(1, false);
  } else if (d.T <= 2) {
    if (lds) MOE_DEC_DN(2, true); else MOE_DEC_DN(2, false);
  } else if (d.T <= 4) {
    if (lds) MOE_DEC_DN(4, true); else MOE_DEC_DN(4, false);
  } else if (d.T <= 8) {
    MOE_DEC_DN(8, false);
  } else {
    MOE_DEC_DN(16, false);
  }
#undef MOE_DEC_DN
  return hipGetLastError();
}

}  // namespace moe
