// Argument blocks passed by value from the host launchers to the kernels.
// Plain data only: included by both the HIP kernel sources and the host API.
#pragma once

#include <stdint.h>

namespace casc {

// One layer's paged K and V.  Element offsets: page*page_stride +
// slot*token_stride + kv_head*head_stride + channel.
struct KvView {
  const uint16_t* k;
  const uint16_t* v;
  int64_t page_stride;
  int64_t token_stride;
  int64_t head_stride;
  int32_t num_pages;
  int32_t log2_page;
  int32_t page_bytes;  // bytes spanned by one page of K (or V): the range of
                       // its buffer descriptor, so reads past it return zero
  int32_t elem_bytes;  // 2: bf16 elements; 1: FP8 E4M3 codes (offsets above
                       // count elements, so they are byte offsets for FP8)
  uint32_t page_stride_b;   // page_stride and token_stride in bytes (each below
  uint32_t token_stride_b;  // 2 GiB: the prefix tile address arithmetic is 32x32-bit)
};

// Query rows per chunk of the pair kernel (three 16-row MFMA blocks).
constexpr int kPairRows = 48;

// Row-split kernel (head_dim 128): waves per workgroup, and query rows per
// work item -- kRowWaves waves of at most 32 rows (two 16-row MFMA blocks).
constexpr int kRowWaves = 4;
constexpr int kRowsPerItem = kRowWaves * 32;

enum AttnMode : int {
  kModePrefix = 0,        // pass A: unsplit -> (o_A, LSE_A); split -> partial states
  kModeDraft = 1,         // pass B -> (o_B, LSE_B)
  kModeVerify = 2,        // pass A; unsplit: + pass B + merge -> (o, LSE); split -> partials
  kModeNaive = 3,         // naive expansion, one softmax per branch -> (o, LSE)
};

struct AttnArgs {
  const uint16_t* q;
  int64_t q_row_stride;
  int64_t q_head_stride;
  int32_t num_qo_heads;
  int32_t group;
  int32_t total_rows;
  float scale_log2;  // sm_scale * k_scale * log2(e): scores are kept in base 2
  float v_scale;     // FP8 pools: the V scale, applied to normalised outputs
  // FP8 pools, per-channel scales [Hkv, D] or NULL: K's multiply the query
  // row (rounded to bf16) as it is loaded, V's each normalised output channel.
  const float* k_cs;
  const float* v_cs;
  KvView kv;
  int32_t num_kv_heads;
  int32_t batch_size;
  const int32_t* page_table;
  int32_t page_table_stride;
  const int32_t* cache_seqlens;
  const int32_t* req_branch_indptr;
  const int32_t* branch_qo_indptr;
  const int32_t* draft_page_table;
  int32_t draft_page_table_stride;
  const int32_t* draft_start;
  const uint64_t* draft_mask;  // per row: ancestor set over its branch's nodes (NULL: chains)
  int32_t draft_mask_words;    // 64-bit words per row of draft_mask (>= 1)
  int32_t n_seg_items;  // (segment, kv head) pairs of the launch (key-split and row-split kernels)
  int32_t n_chunks;     // row chunks per segment and kv head
  int32_t chunk_rows;   // pair kernel: query rows per chunk (<= 16 * its row blocks)
  int32_t grid_splits;  // key splits in this launch's grid
  int32_t n_splits;     // key splits of the prefix (partials in the workspace)
  int32_t split_len;    // keys per split (multiple of 32)
  void* o;
  int32_t o_bf16;
  float* lse;
  float* ws_o;    // [n_splits, total_rows, Hq, D] normalised partial outputs
  float* ws_lse;  // [n_splits, total_rows, Hq] partial LSE, base 2
  // Row-split kernel: the launch's work items, longest first (built on the
  // device by worklist_kernel), or NULL for the fixed grid order.  Entry e
  // of *work_count is (request * n_splits + split) * n_chunks + chunk;
  // workgroup u takes entry u / num_kv_heads, kv head u % num_kv_heads.
  const int32_t* work_list;
  const int32_t* work_count;
};

// Work list of a row-split launch: every (request, key split, row chunk)
// that has work, sorted by its 32-key tiles, longest first.
struct WorkListArgs {
  int32_t batch_size;
  const int32_t* cache_seqlens;
  const int32_t* req_branch_indptr;
  const int32_t* branch_qo_indptr;
  int32_t num_branches;
  int32_t group;       // query heads per kv head
  int32_t n_chunks;    // row chunks per request (kRowsPerItem rows each)
  int32_t n_splits;    // key splits of the prefix
  int32_t split_len;   // keys per split
  int32_t drafts;      // 1: split 0 also takes the request's draft tiles
  int32_t bucket_shift;  // work buckets hold 2^bucket_shift tiles each
  int32_t* list;       // [batch_size * n_splits * n_chunks] entries (first *count used)
  int32_t* count;      // entries written
};

// Merge of the key-split partial states of pass A or the fused verify pass
// (one thread per 4 channels of one (row, head)).
struct SplitMergeArgs {
  const float* ws_o;    // [n_splits, total_rows, Hq, D] normalised partial outputs
  const float* ws_lse;  // [n_splits, total_rows, Hq] partial LSE, base 2
  int32_t n_splits;
  int32_t split_len;
  int32_t total_rows;
  int32_t num_qo_heads;
  int32_t head_dim;
  int32_t batch_size;
  int32_t len_cap;      // keys a request can have: block-table capacity, and the planned splits
  int32_t verify;       // split 0 always holds a partial (the drafts of the fused pass)
  const int32_t* cache_seqlens;
  const int32_t* req_branch_indptr;
  const int32_t* branch_qo_indptr;
  void* o;
  int32_t o_bf16;
  float* lse;           // natural log (nullable)
};

// Elementwise merge of two attention states (the standalone merge_state).
struct MergeArgs {
  const float* o_a;
  const float* lse_a;
  const float* o_b;
  const float* lse_b;
  int64_t rows;  // num_rows * num_heads
  int32_t head_dim;
  void* o;
  int32_t o_bf16;
  float* lse;
};

// Debug hooks: gather one sequence's K/V, or one branch's visibility mask.
// Draft-KV append and commit of accepted drafts (the serving step's writes).
struct AppendArgs {
  KvView kv;
  int32_t head_dim;
  int32_t num_kv_heads;
  int32_t total_rows;
  int32_t num_branches;
  const int32_t* branch_qo_indptr;
  const int32_t* draft_page_table;
  int32_t draft_page_table_stride;
  const int32_t* draft_start;
  const void* k_new;  // [total_rows, Hkv, d] in the pool element type (strided)
  const void* v_new;
  int64_t new_row_stride;
  int64_t new_head_stride;
};

struct CommitArgs {
  KvView kv;
  int32_t head_dim;
  int32_t num_kv_heads;
  int32_t batch_size;
  int32_t num_branches;
  int32_t total_rows;
  int32_t max_accepted;
  const int32_t* page_table;
  int32_t page_table_stride;
  const int32_t* cache_seqlens;  // lengths before the commit
  int32_t* cache_seqlens_out;    // lengths after it (may alias cache_seqlens)
  const int32_t* branch_qo_indptr;
  const int32_t* draft_page_table;
  int32_t draft_page_table_stride;
  const int32_t* draft_start;
  const int32_t* accepted_indptr;  // [batch_size + 1]
  const int32_t* accepted_rows;    // global query rows, path order
};

struct DebugArgs {
  KvView kv;
  int32_t head_dim;
  int32_t num_kv_heads;
  int32_t batch_size;
  const int32_t* page_table;
  int32_t page_table_stride;
  const int32_t* cache_seqlens;
  const int32_t* req_branch_indptr;
  const int32_t* branch_qo_indptr;
  const int32_t* draft_page_table;
  int32_t draft_page_table_stride;
  const int32_t* draft_start;
  const uint64_t* draft_mask;
  int32_t draft_mask_words;
  int32_t which;
  int32_t index;
  int32_t kv_head;
  int32_t count;  // rows to produce (tokens for gather, query rows for the mask)
  int32_t cols;   // mask columns
  uint16_t* k_out;
  uint16_t* v_out;
  uint8_t* mask_out;
};

}  // namespace casc
