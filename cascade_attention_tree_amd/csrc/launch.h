// Host-side launch interface between the C API and the kernel translation units.
#pragma once

#include <hip/hip_runtime_api.h>

#include "args.h"

namespace casc {

// Attention kernels: head_dim 64 or 128, rb = 16-row blocks per chunk (1..5).
// ev_start / ev_stop (may be null): HIP events the command processor records
// immediately before the kernel starts / after it ends.
hipError_t launch_attn_d64(int mode, int rb, const AttnArgs& a, int grid, hipStream_t s,
                           hipEvent_t ev_start, hipEvent_t ev_stop);
hipError_t launch_attn_d128(int mode, int rb, const AttnArgs& a, int grid, hipStream_t s,
                            hipEvent_t ev_start, hipEvent_t ev_stop);
// The same over FP8 E4M3 pools (modes that read keys only).
hipError_t launch_attn_d64_fp8(int mode, int rb, const AttnArgs& a, int grid, hipStream_t s,
                               hipEvent_t ev_start, hipEvent_t ev_stop);
hipError_t launch_attn_d128_fp8(int mode, int rb, const AttnArgs& a, int grid, hipStream_t s,
                                hipEvent_t ev_start, hipEvent_t ev_stop);

// Row-split kernel for head_dim 128 (bf16 / FP8 pools), modes kModePrefix,
// kModeVerify and kModeDraft: work items of at most kRowsPerItem query rows
// (a.n_chunks counts chunks of that size).  three_wave (bf16): three
// workgroups per CU instead of two.
hipError_t launch_rows_d128(int mode, bool three_wave, const AttnArgs& a, int grid, hipStream_t s,
                            hipEvent_t ev_start, hipEvent_t ev_stop);
hipError_t launch_rows_d128_fp8(int mode, const AttnArgs& a, int grid, hipStream_t s, hipEvent_t ev_start,
                                hipEvent_t ev_stop);

// Pair kernel, head_dim 128 (bf16 / FP8 pools), modes kModePrefix and
// kModeVerify: a.n_chunks chunks of a.chunk_rows rows per (request, kv head),
// grid = a.grid_splits * (items rounded up to a multiple of 8) * a.n_chunks.
hipError_t launch_pair_d128(int mode, const AttnArgs& a, int grid, hipStream_t s, hipEvent_t ev_start,
                            hipEvent_t ev_stop);
hipError_t launch_pair_d128_fp8(int mode, const AttnArgs& a, int grid, hipStream_t s, hipEvent_t ev_start,
                                hipEvent_t ev_stop);

// Work list of a row-split launch (one workgroup); ev_start (may be null):
// event recorded when it starts.
hipError_t launch_worklist(const WorkListArgs& a, hipStream_t s, hipEvent_t ev_start);
hipError_t launch_merge(const MergeArgs& a, hipStream_t s);
// Merge of key-split partial states; e1 (may be null): event recorded when it ends.
hipError_t launch_split_merge(const SplitMergeArgs& a, hipStream_t s, hipEvent_t e1);
hipError_t launch_append_kv(const AppendArgs& a, hipStream_t s);
hipError_t launch_stream_read(const void* buf, size_t bytes, unsigned int* sink, hipStream_t s);
hipError_t launch_commit(const CommitArgs& a, hipStream_t s);
hipError_t launch_debug_gather(const DebugArgs& a, hipStream_t s);
hipError_t launch_debug_mask(const DebugArgs& a, hipStream_t s);

// The allocation-free verify entry point's workspace: a file-scope device
// array of kScratchBytes per GPU.  scratch_for_current_device returns the
// current device's copy (looked up once per device).
constexpr size_t kScratchBytes = size_t(32) << 20;
hipError_t scratch_for_current_device(void** ptr);

// Sticky device error words of each translation unit (read, optionally clear).
hipError_t read_error_d64(int* v, int clear);
hipError_t read_error_d128(int* v, int clear);
hipError_t read_error_d64_fp8(int* v, int clear);
hipError_t read_error_d128_fp8(int* v, int clear);
hipError_t read_error_small(int* v, int clear);
hipError_t read_error_pair_d128(int* v, int clear);
hipError_t read_error_pair_d128_fp8(int* v, int clear);

}  // namespace casc
