// moe_layer_forward without a caller workspace: the scratch memory is a file-scope device
// array of MOE_NOALLOC_SCRATCH_BYTES that each GPU holds from the library's load until the
// process ends. For callers that cannot allocate device memory (code under HIP-graph capture,
// tight serving loops, harnesses that forbid hipMalloc).
//
// In host code the array's name is only a host-side stand-in; its device address on the
// current GPU comes from hipGetSymbolAddress, taken once per device and kept, and only that
// address is handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "moe_w4.h"

namespace {

static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices] = {nullptr};
std::mutex g_mutex;

// The device address of this GPU's copy of `scratch` (nullptr on failure).
void* scratch_for_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" int moe_layer_forward_noalloc(const moe_layer_desc_t* desc, const uint16_t* x,
                                         int32_t T, float* out, int32_t flags, void* stream) {
  if (T == 0) return moe_layer_forward(desc, x, T, out, nullptr, 0, flags, stream);
  const size_t need = moe_workspace_bytes(desc, T, flags);
  if (need == 0) {
    // an invalid descriptor, size or flag: the same status moe_layer_forward gives
    return moe_layer_forward(desc, x, T, out, nullptr, 0, flags, stream);
  }
  if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_WORKSPACE_TOO_SMALL;
  void* ws = scratch_for_current_device();
  if (ws == nullptr) return MOE_HIP_ERROR;
  return moe_layer_forward(desc, x, T, out, ws, MOE_NOALLOC_SCRATCH_BYTES, flags, stream);
}
