// Instantiations of the attention kernels for head_dim = 128, FP8 E4M3 pools.
#include "attn_launch.h"

namespace casc {

hipError_t launch_attn_d128_fp8(int mode, int rb, const AttnArgs& a, int grid, hipStream_t s,
                                hipEvent_t e0, hipEvent_t e1) {
  return launch_any_rb<128, true>(mode, rb, a, grid, s, e0, e1);
}

hipError_t read_error_d128_fp8(int* v, int clear) { return read_error_word(v, clear); }

hipError_t launch_rows_d128_fp8(int mode, const AttnArgs& a, int grid, hipStream_t s, hipEvent_t e0,
                                hipEvent_t e1) {
  return launch_rows<true>(mode, false, a, grid, s, e0, e1);
}

}  // namespace casc
