// Drives the C ABI's host-side paths (validation, workspace sizing and carving, launch
// sequencing) with valid and invalid arguments; built with the stub launchers under ASan/UBSan.
// Device pointers are never dereferenced on the host, so aligned fake addresses stand in.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "moe_w4.h"

static int failures = 0;
#define EXPECT(cond)                                                       \
  do {                                                                     \
    if (!(cond)) {                                                         \
      std::fprintf(stderr, "line %d: expectation failed: %s\n", __LINE__, #cond); \
      ++failures;                                                          \
    }                                                                      \
  } while (0)

template <typename T>
static T* fake(uintptr_t a) { return reinterpret_cast<T*>(a); }

static moe_layer_desc_t desc(int H, int E, int K, int F, int Fs) {
  moe_layer_desc_t d{};
  d.hidden = H; d.num_experts = E; d.top_k = K; d.ffn = F; d.shared_ffn = Fs;
  d.bits = 4; d.group_size = 64; d.renormalize = 1;
  d.router_w = fake<float>(0x100000);
  moe_w4_t w{fake<uint32_t>(0x200000), fake<uint16_t>(0x300000), fake<uint16_t>(0x400000)};
  d.gate = d.up = d.down = d.sh_gate = d.sh_up = d.sh_down = w;
  d.shared_gate_w = fake<float>(0x500000);
  return d;
}

int main() {
  const uint16_t* x = fake<uint16_t>(0x600000);
  float* out = fake<float>(0x700000);
  void* ws = fake<void>(0x800000);
  // shapes: decode and prefill sizes, odd sizes, the largest accepted expert count and top-k
  const int shapes[][5] = {{2048, 256, 8, 512, 512}, {256, 16, 2, 128, 128}, {320, 7, 3, 192, 64},
                           {256, 1024, 32, 64, 64}, {2560, 16, 2, 128, 0}, {16384, 8, 1, 64, 0}};
  for (auto& s : shapes) {
    moe_layer_desc_t d = desc(s[0], s[1], s[2], s[3], s[4]);
    for (int T : {0, 1, 3, 8, 16, 17, 300, 4096}) {
      for (int flags : {0, 1, 2, 3}) {
        const size_t need = moe_workspace_bytes(&d, T, flags);
        EXPECT(need > 0);
        EXPECT(moe_layer_forward(&d, x, T, out, ws, need, flags, nullptr) == MOE_OK);
        if (T > 0) {
          EXPECT(moe_layer_forward(&d, x, T, out, ws, need - 1, flags, nullptr) ==
                 MOE_WORKSPACE_TOO_SMALL);
          const int n = moe_layer_num_phases(&d, T, flags);
          EXPECT(n >= 3 && n <= 6);
          for (int ph = 0; ph < n; ++ph)
            EXPECT(moe_layer_forward_phase(&d, x, T, out, ws, need, flags, ph, nullptr) == MOE_OK);
          EXPECT(moe_layer_forward_phase(&d, x, T, out, ws, need, flags, n, nullptr) == MOE_INVALID_ARG);
        }
      }
      size_t off[14];
      EXPECT(moe_debug_workspace_layout(&d, T, 0, off, 14) == MOE_OK);
      for (int i = 1; i < 14; ++i) EXPECT(off[i] >= off[i - 1]);
    }
    // the stack over three layers, decode and prefill sizes
    const moe_layer_desc_t* layers[3] = {&d, &d, &d};
    for (int T : {1, 8, 512}) {
      const size_t need = moe_stack_workspace_bytes(layers, 3, T, 0);
      EXPECT(need > 0);
      EXPECT(moe_stack_forward(layers, 3, out, fake<uint16_t>(0x900000), T, 1e-6f, ws, need, 0,
                               nullptr) == MOE_OK);
    }
  }
  // rejections
  moe_layer_desc_t d = desc(2048, 256, 8, 512, 512);
  const size_t need = moe_workspace_bytes(&d, 16, 0);
  EXPECT(moe_layer_forward(nullptr, x, 16, out, ws, need, 0, nullptr) == MOE_INVALID_ARG);
  EXPECT(moe_layer_forward(&d, x, -1, out, ws, need, 0, nullptr) == MOE_INVALID_ARG);
  EXPECT(moe_layer_forward(&d, x, 16, out, ws, need, 8, nullptr) == MOE_INVALID_ARG);
  EXPECT(moe_layer_forward(&d, fake<uint16_t>(0x600002), 16, out, ws, need, 0, nullptr) == MOE_INVALID_ARG);
  EXPECT(moe_layer_forward(&d, x, 16, out, fake<void>(0x800010), need, 0, nullptr) == MOE_INVALID_ARG);
  EXPECT(moe_layer_forward(&d, x, 1 << 30, out, ws, ~(size_t)0, 0, nullptr) == MOE_UNSUPPORTED);
  moe_layer_desc_t bad = d;
  bad.bits = 3;
  EXPECT(moe_workspace_bytes(&bad, 16, 0) == 0);
  EXPECT(moe_layer_forward(&bad, x, 16, out, ws, need, 0, nullptr) == MOE_UNSUPPORTED);
  bad = d;
  bad.top_k = 300;
  EXPECT(moe_layer_forward(&bad, x, 16, out, ws, need, 0, nullptr) == MOE_UNSUPPORTED);
  bad = d;
  bad.gate.q = fake<uint32_t>(0x200004);  // misaligned packed words
  EXPECT(moe_layer_forward(&bad, x, 16, out, ws, need, 0, nullptr) == MOE_INVALID_ARG);
  // the single stages
  int32_t* i32 = fake<int32_t>(0xA00000);
  float* f32 = fake<float>(0xB00000);
  moe_plan_t plan{i32, i32, i32, i32, i32, i32};
  for (int T : {1, 16, 300}) {
    const size_t ws_need = moe_workspace_bytes(&d, T, 0);
    EXPECT(moe_route(&d, x, T, i32, f32, f32, i32, ws, ws_need, nullptr) == MOE_OK);
    EXPECT(moe_permute(&d, i32, T, &plan, ws, ws_need, nullptr) == MOE_OK);
    for (int which = 0; which < 4; ++which)
      EXPECT(moe_grouped_gemm_w4(&d, which, x, T, &plan, f32, f32, out, ws, ws_need, nullptr) == MOE_OK);
    EXPECT(moe_grouped_gemm_w4(&d, 4, x, T, &plan, f32, f32, out, ws, ws_need, nullptr) == MOE_INVALID_ARG);
    EXPECT(moe_combine(&d, f32, i32, f32, f32, f32, T, out, nullptr) == MOE_OK);
  }
  EXPECT(moe_residual_rmsnorm(f32, out, fake<uint16_t>(0x900000), 4, 2048, 1e-6f, 0, nullptr) == MOE_OK);
  EXPECT(moe_residual_rmsnorm(f32, out, fake<uint16_t>(0x900000), 4, 2000, 1e-6f, 0, nullptr) == MOE_INVALID_ARG);
  std::printf("%s (%d failures)\n", failures ? "FAILED" : "ok", failures);
  return failures ? 1 : 0;
}
