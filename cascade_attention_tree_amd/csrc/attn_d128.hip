// Instantiations of the attention kernels for head_dim = 128, bf16 pools.
#include "attn_launch.h"

namespace casc {

hipError_t launch_attn_d128(int mode, int rb, const AttnArgs& a, int grid, hipStream_t s,
                           hipEvent_t e0, hipEvent_t e1) {
  return launch_any_rb<128, false>(mode, rb, a, grid, s, e0, e1);
}

hipError_t read_error_d128(int* v, int clear) { return read_error_word(v, clear); }

hipError_t launch_rows_d128(int mode, bool three_wave, const AttnArgs& a, int grid, hipStream_t s, hipEvent_t e0,
                            hipEvent_t e1) {
  return launch_rows<false>(mode, three_wave, a, grid, s, e0, e1);
}

}  // namespace casc
