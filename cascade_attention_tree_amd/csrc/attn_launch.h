// Launch helpers of the attention translation units: each .hip file
// instantiates the kernels of one head dim and one pool element type, and
// owns its own copy of the sticky device error word.
#pragma once

#include <hip/hip_ext.h>

#include "attn_kernel.h"
#include "launch.h"
#include "rows_kernel.h"

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

template <int D, int RB, bool KV8>
static hipError_t launch_rb(int mode, const AttnArgs& a, int grid, hipStream_t s, hipEvent_t e0,
                            hipEvent_t e1) {
  const dim3 g(grid), b(256);
  switch (mode) {
    case kModePrefix: go(attn_kernel<D, RB, kModePrefix, KV8>, g, b, s, e0, e1, a); break;
    case kModeDraft: go(attn_kernel<D, RB, kModeDraft, KV8>, g, b, s, e0, e1, a); break;
    case kModeVerify: go(attn_kernel<D, RB, kModeVerify, KV8>, g, b, s, e0, e1, a); break;
    case kModeNaive: go(attn_kernel<D, RB, kModeNaive, KV8>, g, b, s, e0, e1, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Row-split kernel (head_dim 128: pass A, the fused verify pass, pass B):
// tiles requested this many steps ahead.
constexpr int kRowDepth = 4;
// 16-row blocks per wave: each K and V fragment read out of LDS serves them all.
constexpr int kRowBlocks = 2;

template <bool KV8, int NS>
static inline hipError_t launch_rows_ns(int mode, const AttnArgs& a, int grid, hipStream_t s, hipEvent_t e0,
                                        hipEvent_t e1) {
  const dim3 g(grid), b(64 * kRowWaves);
  switch (mode) {
    case kModePrefix: go(rows_kernel<kModePrefix, kRowDepth, kRowBlocks, KV8, NS>, g, b, s, e0, e1, a); break;
    case kModeVerify: go(rows_kernel<kModeVerify, kRowDepth, kRowBlocks, KV8, NS>, g, b, s, e0, e1, a); break;
    case kModeDraft: go(rows_kernel<kModeDraft, kRowDepth, kRowBlocks, KV8, NS>, g, b, s, e0, e1, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// three_wave: bf16 pools, three workgroups per CU (three copy stages);
// otherwise two (four stages, or the FP8 register ring).
template <bool KV8>
static inline hipError_t launch_rows(int mode, bool three_wave, const AttnArgs& a, int grid, hipStream_t s,
                                     hipEvent_t e0, hipEvent_t e1) {
  if constexpr (!KV8) {
    if (three_wave) return launch_rows_ns<KV8, 3>(mode, a, grid, s, e0, e1);
  }
  return launch_rows_ns<KV8, 4>(mode, a, grid, s, e0, e1);
}

// Pair kernel (head_dim 128): pass A or the fused verify pass over chunks of
// a.chunk_rows query rows; defined where pair_kernel.h is included.
template <bool KV8>
static hipError_t launch_pair(int mode, const AttnArgs& a, int grid, hipStream_t s, hipEvent_t e0,
                              hipEvent_t e1);

template <int D, bool KV8>
static hipError_t launch_any_rb(int mode, int rb, const AttnArgs& a, int grid, hipStream_t s,
                                hipEvent_t e0, hipEvent_t e1) {
  switch (rb) {
    case 1: return launch_rb<D, 1, KV8>(mode, a, grid, s, e0, e1);
    case 2: return launch_rb<D, 2, KV8>(mode, a, grid, s, e0, e1);
    case 3: return launch_rb<D, 3, KV8>(mode, a, grid, s, e0, e1);
    case 4: return launch_rb<D, 4, KV8>(mode, a, grid, s, e0, e1);
    case 5: return launch_rb<D, 5, KV8>(mode, a, grid, s, e0, e1);
    default: return hipErrorInvalidValue;
  }
}

static hipError_t read_error_word(int* v, int clear) {
  hipError_t e = hipMemcpyFromSymbol(v, HIP_SYMBOL(g_device_error), sizeof(int));
  if (e == hipSuccess && clear) {
    const int zero = 0;
    e = hipMemcpyToSymbol(HIP_SYMBOL(g_device_error), &zero, sizeof(int));
  }
  return e;
}

}  // namespace casc
