// Instantiations of the pair kernel (pass A and the fused verify pass with
// few query rows per kv head), head_dim = 128, FP8 E4M3 pools.
#include "attn_launch.h"
#include "pair_kernel.h"

namespace casc {

hipError_t launch_pair_d128_fp8(int mode, const AttnArgs& a, int grid, hipStream_t s, hipEvent_t e0,
                                hipEvent_t e1) {
  return launch_pair<true>(mode, a, grid, s, e0, e1);
}

hipError_t read_error_pair_d128_fp8(int* v, int clear) { return read_error_word(v, clear); }

}  // namespace casc
