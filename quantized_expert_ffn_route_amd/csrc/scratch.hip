// Library-owned device scratch for callers that cannot allocate (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
// one file-scope device array per GPU, holding what a decode workspace holds.
//
// In host code the name `scratch` is only a host-side stand-in for the
// symbol, not a device address: every host use goes through the pointer that
// hipGetSymbolAddress returns for the current device, resolved once per
// device on the first call that needs it and kept for the process.
#include <mutex>

#include "internal.hpp"

namespace {

static __device__ __align__(256) unsigned char scratch[moe::kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

namespace moe {

int scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return MOE_EHIP;
  }
  if (dev >= kMaxDevices) return MOE_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return MOE_EHIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace moe
