// Instantiations of the attention kernels for head_dim = 128.
#include <hip/hip_ext.h>

#include "attn_kernel.h"
#include "launch.h"

namespace casc {

// Plain launch, or with events recorded around the kernel when timing.
template <typename K>
static void go(K kernel, dim3 g, dim3 b, hipStream_t s, hipEvent_t e0, hipEvent_t e1, const AttnArgs& a) {
  if (e0 || e1) {
    hipExtLaunchKernelGGL(kernel, g, b, 0, s, e0, e1, 0, a);
  } else {
    hipLaunchKernelGGL(kernel, g, b, 0, s, a);
  }
}

template <int RB>
static hipError_t launch_rb(int mode, const AttnArgs& a, int grid, hipStream_t s, hipEvent_t e0,
                            hipEvent_t e1) {
  const dim3 g(grid), b(256);
  switch (mode) {
    case kModePrefix: go(attn_kernel<128, RB, kModePrefix>, g, b, s, e0, e1, a); break;
    case kModeDraft: go(attn_kernel<128, RB, kModeDraft>, g, b, s, e0, e1, a); break;
    case kModeVerify: go(attn_kernel<128, RB, kModeVerify>, g, b, s, e0, e1, a); break;
    case kModeNaive: go(attn_kernel<128, RB, kModeNaive>, g, b, s, e0, e1, a); break;
    case kModePrefixFinish: go(attn_kernel<128, RB, kModePrefixFinish>, g, b, s, e0, e1, a); break;
    case kModeVerifyFinish: go(attn_kernel<128, RB, kModeVerifyFinish>, g, b, s, e0, e1, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn_d128(int mode, int rb, const AttnArgs& a, int grid, hipStream_t s,
                            hipEvent_t e0, hipEvent_t e1) {
  switch (rb) {
    case 1: return launch_rb<1>(mode, a, grid, s, e0, e1);
    case 2: return launch_rb<2>(mode, a, grid, s, e0, e1);
    case 3: return launch_rb<3>(mode, a, grid, s, e0, e1);
    case 4: return launch_rb<4>(mode, a, grid, s, e0, e1);
    case 5: return launch_rb<5>(mode, a, grid, s, e0, e1);
    default: return hipErrorInvalidValue;
  }
}

hipError_t read_error_d128(int* v, int clear) {
  hipError_t e = hipMemcpyFromSymbol(v, HIP_SYMBOL(g_device_error), sizeof(int));
  if (e == hipSuccess && clear) {
    const int zero = 0;
    e = hipMemcpyToSymbol(HIP_SYMBOL(g_device_error), &zero, sizeof(int));
  }
  return e;
}

}  // namespace casc
