// Host-only stand-ins for the kernel launchers, so that api.cpp's validation, workspace carving
// and launch sequencing can run under AddressSanitizer and UndefinedBehaviorSanitizer on a
// machine without a GPU. Each launcher checks the pointers and sizes it is handed the way the
// kernels would use them (non-null where a kernel would read or write) and enqueues nothing.
#include <cstdio>
#include <cstdlib>

#include "moe_internal.h"

namespace moe {

static void need(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "stub launcher: %s\n", what);
    std::abort();
  }
}

int router_splits(int, int, int) { return 1; }
hipError_t launch_router_logits_mfma(const uint16_t* x, const float* w, const float*, const float*,
                                     int T, int E, int H, float* logits, hipStream_t) {
  need(x && w && logits && T > 0 && E > 0 && H > 0, "router mfma");
  return hipSuccess;
}
hipError_t launch_router_logits_gemv(const uint16_t* x, const float* w, const float*, int T, int E,
                                     int H, float* logits, hipStream_t) {
  need(x && w && logits && T > 0 && E > 0 && H > 0, "router gemv");
  return hipSuccess;
}
hipError_t launch_topk(const float* logits, int S, int, bool, const uint16_t*, const float*, int T,
                       int E, int K, int, int32_t* idx, float* w, float*, hipStream_t) {
  need(logits && idx && w && S >= 1 && T > 0 && K <= E, "topk");
  return hipSuccess;
}
hipError_t launch_count(const int32_t* idx, int TK, int E, int32_t* counts, hipStream_t) {
  need(idx && counts && TK > 0 && E > 0, "count");
  return hipSuccess;
}
hipError_t launch_route_small(const float* logits, const uint16_t*, const float*, const Dims& d,
                              int32_t* idx, float* w, float*, const moe_plan_t& plan, hipStream_t) {
  need(logits && idx && w && plan.blocks && d.T > 0, "route small");
  return hipSuccess;
}
hipError_t launch_permute(const int32_t* idx, const Dims& d, bool, int32_t* hist,
                          const moe_plan_t& plan, hipStream_t) {
  need(idx && hist && plan.counts && plan.offsets && plan.sorted_slots && plan.slot_pos &&
       plan.blocks && plan.num_blocks && d.T > 0, "permute");
  return hipSuccess;
}
hipError_t launch_gemm_w4(int mode, const GemmParams& p, int max_blocks, hipStream_t) {
  need(p.out && p.a_routed && p.blocks && max_blocks > 0 && mode >= 0 && mode <= 2, "gemm");
  return hipSuccess;
}
hipError_t launch_fill_zero(float* p, size_t n, hipStream_t) {
  need(p && n % 4 == 0, "fill");
  return hipSuccess;
}
hipError_t launch_combine(const float* y, const int32_t* pos, const float* w, const float*,
                          const float*, const Dims& d, float* out, hipStream_t) {
  need(y && pos && w && out && d.T > 0, "combine");
  return hipSuccess;
}
hipError_t launch_dec_gateup(const Dims& d, const moe_layer_desc_t&, const uint16_t* x,
                             const moe_plan_t&, int, uint16_t* a, hipStream_t) {
  need(x && a && d.T > 0, "dec gateup");
  return hipSuccess;
}
hipError_t launch_dec_down(const Dims& d, const moe_layer_desc_t&, const uint16_t* a,
                           const moe_plan_t&, const float*, const float*, float* out, hipStream_t) {
  need(a && out && d.T > 0, "dec down");
  return hipSuccess;
}
bool decode_fast_ok(const Dims& d) { return d.T >= 1 && d.T <= 16 && d.H <= 2048; }
size_t decode_route_bytes(const Dims& d) { return (1 + 5 * (size_t)d.TK() + d.T) * 4; }
hipError_t launch_decode_layer(const Dims& d, const moe_layer_desc_t&, const uint16_t*,
                               const DecodeBufs& b, float*, hipStream_t, int phase, const StackFuse*) {
  need(b.logits && b.route && b.a && d.T > 0 && phase >= -1 && phase <= 2, "decode layer");
  return hipSuccess;
}
hipError_t launch_residual_rmsnorm(const float*, float* r, uint16_t* x, int T, int H, float, int,
                                   hipStream_t) {
  need(r && x && T > 0 && H > 0, "rmsnorm");
  return hipSuccess;
}
hipError_t launch_debug_dequant(const moe_w4_t& w, int, int, int, int, float*, uint16_t*, hipStream_t) {
  need(w.q != nullptr, "dequant");
  return hipSuccess;
}
hipError_t launch_mfma_loop(int, int, float* sink, hipStream_t) {
  need(sink != nullptr, "mfma loop");
  return hipSuccess;
}
double mfma_loop_flops(int wg, int it) { return (double)wg * it; }
hipError_t launch_stream_read(const void* p, size_t, int, uint32_t* sink, hipStream_t) {
  need(p && sink, "stream read");
  return hipSuccess;
}

}  // namespace moe
