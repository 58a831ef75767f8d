// C ABI of the MoE library: argument validation, workspace carving and kernel dispatch.
// The operations and their sources are documented in moe_w4.h.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>

#include "moe_internal.h"
#include "moe_w4.h"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool w4_ok(const moe_w4_t& w) {
  return w.q && w.scale && w.bias && aligned(w.q, 16) && aligned(w.scale, 2) && aligned(w.bias, 2);
}

// Descriptor checks shared by every entry point.
int check_desc(const moe_layer_desc_t* d) {
  if (!d) return MOE_INVALID_ARG;
  if (d->bits != 4 || d->group_size != 64 || d->renormalize != 1) return MOE_UNSUPPORTED;
  if (d->hidden <= 0 || d->num_experts <= 0 || d->top_k <= 0 || d->ffn <= 0 || d->shared_ffn < 0)
    return MOE_INVALID_ARG;
  if (d->hidden % 64 || d->ffn % 64 || d->shared_ffn % 64) return MOE_UNSUPPORTED;
  if (d->num_experts > 1024 || d->top_k > 32 || d->top_k > d->num_experts) return MOE_UNSUPPORTED;
  if (d->hidden > 16384 || d->ffn > 16384 || d->shared_ffn > 16384) return MOE_UNSUPPORTED;
  if (!d->router_w || !aligned(d->router_w, 16)) return MOE_INVALID_ARG;
  if (d->router_bias && !aligned(d->router_bias, 4)) return MOE_INVALID_ARG;
  if (!w4_ok(d->gate) || !w4_ok(d->up) || !w4_ok(d->down)) return MOE_INVALID_ARG;
  if (d->shared_ffn > 0) {
    if (!w4_ok(d->sh_gate) || !w4_ok(d->sh_up) || !w4_ok(d->sh_down)) return MOE_INVALID_ARG;
    if (!d->shared_gate_w || !aligned(d->shared_gate_w, 4)) return MOE_INVALID_ARG;
  }
  return MOE_OK;
}

Dims dims_of(const moe_layer_desc_t* d, int T) {
  return Dims{d->hidden, d->num_experts, d->top_k, d->ffn, d->shared_ffn, T};
}

int max_blocks(const Dims& d) {
  const int TK = d.TK();
  const int routed = (TK + kBlockM - 1) / kBlockM + (d.E < TK ? d.E : TK);
  const int shared = d.Fs > 0 ? (d.T + kBlockM - 1) / kBlockM : 0;
  return routed + shared;
}

// Every index into the grouped activations stays inside 32 bits.
bool sizes_ok(const Dims& d) {
  const int64_t rows = (int64_t)d.T * d.K + d.T;
  int64_t w = d.H;
  if (d.F > w) w = d.F;
  if (d.Fs > w) w = d.Fs;
  return rows * w < (int64_t(1) << 31) && (int64_t)d.T * d.K < (int64_t(1) << 30);
}

// Workspace regions for T tokens, in order of use.
struct Layout {
  size_t logits, hist, topk_idx, topk_w, sgate, droute;
  size_t counts, offsets, sorted, slotpos, blocks, nblk;
  size_t a, y;
  size_t end_route, end_permute, end_no_y, total;
};

Layout layout_of(const Dims& d, int flags) {
  Layout L{};
  size_t o = 0;
  const size_t TK = (size_t)d.T * d.K;
  const int nchunks = (int)((TK + kChunkSlots - 1) / kChunkSlots);
  // up to kRouterMaxSplits partial slices of [T, E+1] (prefill router, split-K)
  L.logits = o;  o = align_up(o + (size_t)kRouterMaxSplits * d.T * (d.E + 1) * 4);
  L.end_route = o;
  L.hist = o;    o = align_up(o + (size_t)nchunks * (d.E + 1) * 4);
  L.end_permute = o;
  L.topk_idx = o; o = align_up(o + TK * 4);
  L.topk_w = o;  o = align_up(o + TK * 4);
  L.sgate = o;   o = align_up(o + (size_t)d.T * 4);
  L.droute = o;  o = align_up(o + decode_route_bytes(d));
  L.counts = o;  o = align_up(o + (size_t)d.E * 4);
  L.offsets = o; o = align_up(o + (size_t)(d.E + 1) * 4);
  L.sorted = o;  o = align_up(o + TK * 4);
  L.slotpos = o; o = align_up(o + TK * 4);
  L.blocks = o;  o = align_up(o + (size_t)max_blocks(d) * 16);
  L.nblk = o;    o = align_up(o + 4);
  L.a = o;       o = align_up(o + (TK * d.F + (size_t)d.T * d.Fs) * 2);
  L.end_no_y = o;
  L.y = o;
  // fp32 expert outputs for the deterministic (store + gather) combine; the fused atomic
  // combine needs none
  if (!(flags & MOE_FLAG_ATOMIC_COMBINE)) o = align_up(o + (TK + d.T) * d.H * 4);
  L.total = o;
  return L;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_HIP_ERROR; }

// Known bits only.
bool flags_ok(int flags) {
  return !(flags & ~(MOE_FLAG_ATOMIC_COMBINE | MOE_FLAG_FORCE_PREFILL));
}

bool use_decode(const Dims& d, int flags) {
  return d.T <= kDecodeMaxT && !(flags & MOE_FLAG_FORCE_PREFILL) && d.F <= 512 && d.Fs <= 512 &&
         (size_t)d.T * d.H * 2 <= 65536;
}

int run_route(const moe_layer_desc_t* desc, const Dims& d, const uint16_t* x, int32_t* idx,
              float* w, float* sgate, void* ws, const Layout& L, bool decode, hipStream_t s) {
  float* logits = at<float>(ws, L.logits);
  const float* wg = d.Fs > 0 ? desc->shared_gate_w : nullptr;
  hipError_t e;
  if (decode) {
    e = launch_router_logits_gemv(x, desc->router_w, desc->router_bias, d.T, d.E, d.H, logits, s);
    if (e != hipSuccess) return MOE_HIP_ERROR;
    return hip_status(launch_topk(logits, 1, d.E, false, x, wg, d.T, d.E, d.K, d.H, idx, w,
                                  sgate, s));
  }
  // the MFMA router leaves partial slices, with the shared-gate logit in column E
  e = launch_router_logits_mfma(x, desc->router_w, desc->router_bias, wg, d.T, d.E, d.H, logits,
                                s);
  if (e != hipSuccess) return MOE_HIP_ERROR;
  return hip_status(launch_topk(logits, router_splits(d.T, d.E, d.H), d.E + 1, wg != nullptr, x,
                                nullptr, d.T, d.E, d.K, d.H, idx, w, sgate, s));
}

GemmParams gemm_params(const moe_layer_desc_t* desc, const Dims& d, int which, const void* in,
                       const moe_plan_t* plan, const float* topk_w, const float* sgate,
                       void* out) {
  GemmParams p{};
  p.blocks = reinterpret_cast<const int4*>(plan->blocks);
  p.num_blocks = plan->num_blocks;
  p.sorted_slots = plan->sorted_slots;
  p.K = d.K;
  p.E = d.E;
  p.TK = d.TK();
  p.topk_w = topk_w;
  p.shared_gate = sgate;
  p.out = out;
  p.out_ld = d.H;
  const uint16_t* a = static_cast<const uint16_t*>(in);
  if (which == MOE_GEMM_GATE_UP) {
    p.a_routed = p.a_shared = a;
    p.kdim_routed = p.kdim_shared = d.H;
    p.n_routed = d.F;
    p.n_shared = d.Fs;
    p.w0 = desc->gate;
    p.w1 = desc->up;
    p.sw0 = desc->sh_gate;
    p.sw1 = desc->sh_up;
  } else {
    p.a_routed = a;
    p.a_shared = a + (size_t)d.TK() * d.F;
    p.kdim_routed = d.F;
    p.kdim_shared = d.Fs > 0 ? d.Fs : 64;
    p.n_routed = d.H;
    p.n_shared = d.Fs > 0 ? d.H : 0;
    p.w0 = p.w1 = desc->down;
    p.sw0 = p.sw1 = desc->sh_down;
  }
  return p;
}

bool plan_ok(const moe_plan_t* p) {
  return p && p->counts && p->offsets && p->sorted_slots && p->slot_pos && p->blocks &&
         p->num_blocks && aligned(p->blocks, 16);
}


// The launch sequence of moe_layer_forward. phase == -1 enqueues all of it, phase >= 0 only
// launch `phase`, phase == -2 enqueues nothing; *nphases (if given) receives the count.
//   decode, one-pass kernels: 0 router + shared expert, 1 top-k + routed gate/up,
//                             2 down + combine
//   decode, other shapes:     0 router, 1 top-k + permutation, 2 gate/up, 3 down + combine
//   prefill:                  0 router, 1 top-k, 2 permutation, 3 gate/up GEMM,
//                             4 down GEMM storing fp32 Y, 5 combine
//                             (MOE_FLAG_ATOMIC_COMBINE: 4 zero fill, 5 down GEMM + combine)
int layer_sequence(const moe_layer_desc_t* desc, const Dims& d, const uint16_t* x, float* out,
                   void* ws, const Layout& L, int flags, hipStream_t s, int phase,
                   int* nphases) {
  int k = 0;
  hipError_t err = hipSuccess;
  auto step = [&](auto&& launch) {
    if (err == hipSuccess && (phase == -1 || phase == k)) err = launch();
    ++k;
  };
  const bool decode = use_decode(d, flags);
  int32_t* idx = at<int32_t>(ws, L.topk_idx);
  float* w = at<float>(ws, L.topk_w);
  float* sgate = at<float>(ws, L.sgate);
  float* logits = at<float>(ws, L.logits);
  moe_plan_t plan{at<int32_t>(ws, L.counts), at<int32_t>(ws, L.offsets),
                  at<int32_t>(ws, L.sorted),  at<int32_t>(ws, L.slotpos),
                  at<int32_t>(ws, L.blocks),  at<int32_t>(ws, L.nblk)};
  uint16_t* a = at<uint16_t>(ws, L.a);
  const int mb = max_blocks(d);
  const float* wg = d.Fs > 0 ? desc->shared_gate_w : nullptr;

  if (decode && decode_fast_ok(d)) {
    const DecodeBufs b{logits, at<int32_t>(ws, L.droute), a};
    for (int ph = 0; ph < 3; ++ph)
      step([&] { return launch_decode_layer(d, *desc, x, b, out, s, ph); });
  } else if (decode) {
    step([&] { return launch_router_logits_gemv(x, desc->router_w, desc->router_bias, d.T, d.E,
                                                d.H, logits, s); });
    step([&] { return launch_route_small(logits, x, wg, d, idx, w, sgate, plan, s); });
    step([&] { return launch_dec_gateup(d, *desc, x, plan, mb, a, s); });
    step([&] { return launch_dec_down(d, *desc, a, plan, w, sgate, out, s); });
  } else {
    step([&] { return launch_router_logits_mfma(x, desc->router_w, desc->router_bias, wg, d.T,
                                                d.E, d.H, logits, s); });
    step([&] {
      return launch_topk(logits, router_splits(d.T, d.E, d.H), d.E + 1, wg != nullptr, x, nullptr,
                         d.T, d.E, d.K, d.H, idx, w, sgate, s);
    });
    step([&] { return launch_permute(idx, d, d.Fs > 0, at<int32_t>(ws, L.hist), plan, s); });
    step([&] {
      const GemmParams pg = gemm_params(desc, d, MOE_GEMM_GATE_UP, x, &plan, nullptr, nullptr, a);
      return launch_gemm_w4(kGateUp, pg, mb, s);
    });
    if (flags & MOE_FLAG_ATOMIC_COMBINE) {
      step([&] { return launch_fill_zero(out, (size_t)d.T * d.H, s); });
      step([&] {
        const GemmParams pd =
            gemm_params(desc, d, MOE_GEMM_DOWN_COMBINE_ATOMIC, a, &plan, w, sgate, out);
        return launch_gemm_w4(kDownAtomic, pd, mb, s);
      });
    } else {
      float* y = at<float>(ws, L.y);
      step([&] {
        const GemmParams pd = gemm_params(desc, d, MOE_GEMM_DOWN, a, &plan, nullptr, nullptr, y);
        return launch_gemm_w4(kDownStore, pd, mb, s);
      });
      step([&] {
        return launch_combine(y, plan.slot_pos, w, d.Fs > 0 ? y + (size_t)d.TK() * d.H : nullptr,
                              sgate, d, out, s);
      });
    }
  }
  if (nphases) *nphases = k;
  return hip_status(err);
}

}  // namespace

extern "C" {

const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_INVALID_ARG: return "invalid argument";
    case MOE_UNSUPPORTED: return "unsupported layer layout";
    case MOE_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MOE_HIP_ERROR: return "HIP launch error";
    default: return "unknown status";
  }
}

const char* moe_version(void) { return "moe_w4 1.0 gfx950"; }

size_t moe_workspace_bytes(const moe_layer_desc_t* desc, int32_t T_max, int32_t flags) {
  if (check_desc(desc) != MOE_OK || T_max < 0 || !flags_ok(flags)) return 0;
  const Dims d = dims_of(desc, T_max);
  if (!sizes_ok(d)) return 0;
  return layout_of(d, flags).total;
}

int32_t moe_plan_max_blocks(const moe_layer_desc_t* desc, int32_t T) {
  if (check_desc(desc) != MOE_OK || T < 0) return 0;
  return max_blocks(dims_of(desc, T));
}

int moe_route(const moe_layer_desc_t* desc, const uint16_t* x, int32_t T, int32_t* topk_idx,
              float* topk_w, float* shared_gate, int32_t* counts, void* workspace,
              size_t ws_bytes, void* stream) {
  int st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (T < 0) return MOE_INVALID_ARG;
  if (T == 0) return MOE_OK;
  const Dims d = dims_of(desc, T);
  if (!sizes_ok(d)) return MOE_UNSUPPORTED;
  if (!x || !aligned(x, 16) || !topk_idx || !topk_w || !counts || !workspace)
    return MOE_INVALID_ARG;
  if (d.Fs > 0 && !shared_gate) return MOE_INVALID_ARG;
  const Layout L = layout_of(d, 0);
  if (ws_bytes < L.end_route) return MOE_WORKSPACE_TOO_SMALL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = run_route(desc, d, x, topk_idx, topk_w, shared_gate, workspace, L, use_decode(d, 0), s);
  if (st != MOE_OK) return st;
  return hip_status(launch_count(topk_idx, d.TK(), d.E, counts, s));
}

int moe_permute(const moe_layer_desc_t* desc, const int32_t* topk_idx, int32_t T,
                const moe_plan_t* plan, void* workspace, size_t ws_bytes, void* stream) {
  int st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (T < 0) return MOE_INVALID_ARG;
  if (T == 0) return MOE_OK;
  const Dims d = dims_of(desc, T);
  if (!sizes_ok(d)) return MOE_UNSUPPORTED;
  if (!topk_idx || !plan_ok(plan) || !workspace) return MOE_INVALID_ARG;
  const Layout L = layout_of(d, 0);
  if (ws_bytes < L.end_permute) return MOE_WORKSPACE_TOO_SMALL;
  return hip_status(launch_permute(topk_idx, d, d.Fs > 0, at<int32_t>(workspace, L.hist), *plan,
                                   static_cast<hipStream_t>(stream)));
}

int moe_grouped_gemm_w4(const moe_layer_desc_t* desc, int32_t which, const void* in, int32_t T,
                        const moe_plan_t* plan, const float* topk_w, const float* shared_gate,
                        void* out, void* workspace, size_t ws_bytes, void* stream) {
  int st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (which < MOE_GEMM_GATE_UP || which > MOE_GEMM_DOWN_COMBINE_ATOMIC || T < 0)
    return MOE_INVALID_ARG;
  if (T == 0) return MOE_OK;
  const Dims d = dims_of(desc, T);
  if (!sizes_ok(d)) return MOE_UNSUPPORTED;
  if (!in || !aligned(in, 16) || !out || !aligned(out, 16) || !plan_ok(plan))
    return MOE_INVALID_ARG;
  const bool combine = which == MOE_GEMM_DOWN_COMBINE || which == MOE_GEMM_DOWN_COMBINE_ATOMIC;
  if (combine && (!topk_w || (d.Fs > 0 && !shared_gate))) return MOE_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int mb = max_blocks(d);
  // Few tokens: the same bandwidth-bound GEMV kernels as moe_layer_forward's decode path.
  if (use_decode(d, 0) && which == MOE_GEMM_GATE_UP)
    return hip_status(launch_dec_gateup(d, *desc, static_cast<const uint16_t*>(in), *plan, mb,
                                        static_cast<uint16_t*>(out), s));
  if (use_decode(d, 0) && which == MOE_GEMM_DOWN_COMBINE)
    return hip_status(launch_dec_down(d, *desc, static_cast<const uint16_t*>(in), *plan, topk_w,
                                      shared_gate, static_cast<float*>(out), s));
  if (which == MOE_GEMM_GATE_UP || which == MOE_GEMM_DOWN) {
    const GemmParams p = gemm_params(desc, d, which, in, plan, nullptr, nullptr, out);
    return hip_status(launch_gemm_w4(which == MOE_GEMM_GATE_UP ? kGateUp : kDownStore, p, mb, s));
  }
  if (which == MOE_GEMM_DOWN_COMBINE_ATOMIC) {
    if (launch_fill_zero(static_cast<float*>(out), (size_t)d.T * d.H, s) != hipSuccess)
      return MOE_HIP_ERROR;
    const GemmParams p = gemm_params(desc, d, which, in, plan, topk_w, shared_gate, out);
    return hip_status(launch_gemm_w4(kDownAtomic, p, mb, s));
  }
  const Layout L = layout_of(d, 0);
  if (!workspace) return MOE_INVALID_ARG;
  if (ws_bytes < L.total) return MOE_WORKSPACE_TOO_SMALL;
  float* y = at<float>(workspace, L.y);
  const GemmParams p = gemm_params(desc, d, MOE_GEMM_DOWN, in, plan, nullptr, nullptr, y);
  if (launch_gemm_w4(kDownStore, p, mb, s) != hipSuccess) return MOE_HIP_ERROR;
  return hip_status(launch_combine(y, plan->slot_pos, topk_w,
                                   d.Fs > 0 ? y + (size_t)d.TK() * d.H : nullptr, shared_gate, d,
                                   static_cast<float*>(out), s));
}

int moe_combine(const moe_layer_desc_t* desc, const float* y_perm, const int32_t* slot_pos,
                const float* topk_w, const float* shared_y, const float* shared_gate,
                int32_t T, float* out, void* stream) {
  int st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (T < 0) return MOE_INVALID_ARG;
  if (T == 0) return MOE_OK;
  const Dims d = dims_of(desc, T);
  if (!sizes_ok(d)) return MOE_UNSUPPORTED;
  if (!y_perm || !aligned(y_perm, 16) || !slot_pos || !topk_w || !out || !aligned(out, 16))
    return MOE_INVALID_ARG;
  if (d.Fs > 0 && (!shared_y || !aligned(shared_y, 16) || !shared_gate)) return MOE_INVALID_ARG;
  return hip_status(launch_combine(y_perm, slot_pos, topk_w, d.Fs > 0 ? shared_y : nullptr,
                                   shared_gate, d, out, static_cast<hipStream_t>(stream)));
}

int moe_layer_forward(const moe_layer_desc_t* desc, const uint16_t* x, int32_t T, float* out,
                      void* workspace, size_t ws_bytes, int32_t flags, void* stream) {
  return moe_layer_forward_phase(desc, x, T, out, workspace, ws_bytes, flags, -1, stream);
}

int32_t moe_layer_num_phases(const moe_layer_desc_t* desc, int32_t T, int32_t flags) {
  if (check_desc(desc) != MOE_OK || T <= 0) return 0;
  const Dims d = dims_of(desc, T);
  if (!sizes_ok(d)) return 0;
  int n = 0;
  layer_sequence(desc, d, nullptr, nullptr, nullptr, layout_of(d, flags), flags, nullptr, -2, &n);
  return n;
}

int moe_layer_forward_phase(const moe_layer_desc_t* desc, const uint16_t* x, int32_t T,
                            float* out, void* workspace, size_t ws_bytes, int32_t flags,
                            int32_t phase, void* stream) {
  int st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (T < 0 || !flags_ok(flags)) return MOE_INVALID_ARG;
  if (T == 0) return MOE_OK;
  const Dims d = dims_of(desc, T);
  if (!sizes_ok(d)) return MOE_UNSUPPORTED;
  if (!x || !aligned(x, 16) || !out || !aligned(out, 16) || !workspace || !aligned(workspace, 256))
    return MOE_INVALID_ARG;
  const Layout L = layout_of(d, flags);
  if (ws_bytes < L.total) return MOE_WORKSPACE_TOO_SMALL;
  if (phase >= 0 && phase >= moe_layer_num_phases(desc, T, flags)) return MOE_INVALID_ARG;
  if (phase < -1) return MOE_INVALID_ARG;
  return layer_sequence(desc, d, x, out, workspace, L, flags, static_cast<hipStream_t>(stream),
                        phase, nullptr);
}

int moe_residual_rmsnorm(const float* y, float* resid, uint16_t* x_out, int32_t T, int32_t H,
                         float eps, int32_t init, void* stream) {
  if (T < 0 || H <= 0 || H % 64 || H > 16384 || !(eps >= 0.0f) || (init != 0 && init != 1))
    return MOE_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!resid || !aligned(resid, 16) || !x_out || !aligned(x_out, 16)) return MOE_INVALID_ARG;
  if (!init && (!y || !aligned(y, 16))) return MOE_INVALID_ARG;
  return hip_status(launch_residual_rmsnorm(y, resid, x_out, T, H, eps, init,
                                            static_cast<hipStream_t>(stream)));
}

size_t moe_stack_workspace_bytes(const moe_layer_desc_t* const* layers, int32_t n_layers,
                                 int32_t T_max, int32_t flags) {
  if (!layers || n_layers <= 0 || T_max < 0) return 0;
  size_t need = 0;
  for (int l = 0; l < n_layers; ++l) {
    const size_t w = moe_workspace_bytes(layers[l], T_max, flags);
    if (w == 0) return 0;
    if (layers[l]->hidden != layers[0]->hidden) return 0;
    if (w > need) need = w;
  }
  // the layer workspace, then the layer output y [T_max, H] fp32
  return align_up(need) + align_up((size_t)T_max * layers[0]->hidden * 4);
}

int moe_stack_forward(const moe_layer_desc_t* const* layers, int32_t n_layers, float* resid,
                      uint16_t* x, int32_t T, float eps, void* workspace, size_t ws_bytes,
                      int32_t flags, void* stream) {
  if (!layers || n_layers <= 0 || T < 0 || !(eps >= 0.0f)) return MOE_INVALID_ARG;
  for (int l = 0; l < n_layers; ++l) {
    const int st = check_desc(layers[l]);
    if (st != MOE_OK) return st;
    if (layers[l]->hidden != layers[0]->hidden) return MOE_INVALID_ARG;
  }
  if (T == 0) return MOE_OK;
  const int H = layers[0]->hidden;
  if (!resid || !aligned(resid, 16) || !x || !aligned(x, 16) || !workspace ||
      !aligned(workspace, 256))
    return MOE_INVALID_ARG;
  const size_t need = moe_stack_workspace_bytes(layers, n_layers, T, flags);
  if (need == 0) return MOE_UNSUPPORTED;
  if (ws_bytes < need) return MOE_WORKSPACE_TOO_SMALL;
  const size_t lws = need - align_up((size_t)T * H * 4);
  float* y = at<float>(workspace, lws);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (launch_residual_rmsnorm(nullptr, resid, x, T, H, eps, 1, s) != hipSuccess)
    return MOE_HIP_ERROR;
  // Decode-sized batches: three launches per layer, the residual update and the RMSNorm folded
  // into the layer's first and last kernels (same arithmetic, same bits), then one final
  // normalisation of the last residual.
  bool fused = true;
  for (int l = 0; l < n_layers && fused; ++l) {
    const Dims d = dims_of(layers[l], T);
    fused = use_decode(d, flags) && decode_fast_ok(d);
  }
  if (fused) {
    const StackFuse sf{resid, x, eps};
    for (int l = 0; l < n_layers; ++l) {
      const Dims d = dims_of(layers[l], T);
      const Layout L = layout_of(d, flags);
      const DecodeBufs b{at<float>(workspace, L.logits), at<int32_t>(workspace, L.droute),
                         at<uint16_t>(workspace, L.a)};
      if (launch_decode_layer(d, *layers[l], nullptr, b, nullptr, s, -1, &sf) != hipSuccess)
        return MOE_HIP_ERROR;
    }
    return hip_status(launch_residual_rmsnorm(nullptr, resid, x, T, H, eps, 2, s));
  }
  for (int l = 0; l < n_layers; ++l) {
    int st = moe_layer_forward(layers[l], x, T, y, workspace, lws, flags, stream);
    if (st != MOE_OK) return st;
    if (launch_residual_rmsnorm(y, resid, x, T, H, eps, 0, s) != hipSuccess) return MOE_HIP_ERROR;
  }
  return MOE_OK;
}

int moe_debug_dequant_w4(const moe_w4_t* w, int32_t n_rows, int32_t Kin, int32_t mat,
                         int32_t row, float* out_f32, uint16_t* out_bf16, void* stream) {
  if (!w || !w4_ok(*w) || n_rows <= 0 || Kin <= 0 || mat < 0 || row < 0 || row >= n_rows)
    return MOE_INVALID_ARG;
  if (Kin % 64) return MOE_UNSUPPORTED;
  if (!out_f32 && !out_bf16) return MOE_INVALID_ARG;
  return hip_status(launch_debug_dequant(*w, n_rows, Kin, mat, row, out_f32, out_bf16,
                                         static_cast<hipStream_t>(stream)));
}

int moe_debug_workspace_layout(const moe_layer_desc_t* desc, int32_t T, int32_t flags,
                               size_t* offsets, int32_t n) {
  int st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (T < 0 || !flags_ok(flags) || !offsets || n < 0) return MOE_INVALID_ARG;
  const Dims d = dims_of(desc, T);
  if (!sizes_ok(d)) return MOE_UNSUPPORTED;
  const Layout L = layout_of(d, flags);
  const size_t v[14] = {L.logits, L.topk_idx, L.topk_w,  L.sgate, L.droute, L.counts, L.offsets,
                        L.sorted, L.slotpos,  L.blocks, L.nblk,  L.a,      L.y,      L.total};
  for (int i = 0; i < n && i < 14; ++i) offsets[i] = v[i];
  return MOE_OK;
}

int moe_bench_mfma_loop(int32_t workgroups, int32_t iters, float* sink, double* flops,
                        void* stream) {
  if (workgroups <= 0 || iters <= 0 || !sink || !flops) return MOE_INVALID_ARG;
  *flops = mfma_loop_flops(workgroups, iters);
  return hip_status(launch_mfma_loop(workgroups, iters, sink, static_cast<hipStream_t>(stream)));
}

int moe_bench_stream_read(const void* p, size_t bytes, int32_t workgroups, uint32_t* sink,
                          void* stream) {
  if (!p || !aligned(p, 16) || bytes % 16 || workgroups <= 0 || !sink) return MOE_INVALID_ARG;
  return hip_status(launch_stream_read(p, bytes, workgroups, sink, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
