// File-scope device workspace of the allocation-free verify entry point.
//
// `scratch` holds the split-prefix partial states that cascade_verify_attn
// otherwise takes from a caller-allocated workspace.  Every GPU the library
// runs on holds its own copy until the process ends.  In host code the
// array's name is only a host-side stand-in: the device address of this
// GPU's copy comes from hipGetSymbolAddress, once per device, and only that
// address is ever passed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"

namespace casc {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t scratch_for_current_device(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace casc
