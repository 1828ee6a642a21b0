// Instantiations of the attention kernels for head_dim = 128.
#include "attn_kernel.h"
#include "launch.h"

namespace casc {

template <int RB>
static hipError_t launch_rb(int mode, const AttnArgs& a, int grid, hipStream_t s) {
  const dim3 g(grid), b(256);
  switch (mode) {
    case kModePrefix: hipLaunchKernelGGL((attn_kernel<128, RB, kModePrefix>), g, b, 0, s, a); break;
    case kModeDraft: hipLaunchKernelGGL((attn_kernel<128, RB, kModeDraft>), g, b, 0, s, a); break;
    case kModeVerify: hipLaunchKernelGGL((attn_kernel<128, RB, kModeVerify>), g, b, 0, s, a); break;
    case kModeNaive: hipLaunchKernelGGL((attn_kernel<128, RB, kModeNaive>), g, b, 0, s, a); break;
    case kModePrefixFinish: hipLaunchKernelGGL((attn_kernel<128, RB, kModePrefixFinish>), g, b, 0, s, a); break;
    case kModeVerifyFinish: hipLaunchKernelGGL((attn_kernel<128, RB, kModeVerifyFinish>), g, b, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn_d128(int mode, int rb, const AttnArgs& a, int grid, hipStream_t s) {
  switch (rb) {
    case 1: return launch_rb<1>(mode, a, grid, s);
    case 2: return launch_rb<2>(mode, a, grid, s);
    case 3: return launch_rb<3>(mode, a, grid, s);
    case 4: return launch_rb<4>(mode, a, grid, s);
    case 5: return launch_rb<5>(mode, a, grid, s);
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
