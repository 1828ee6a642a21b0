/*
 * cascade_attn.h -- C ABI of libcascade_attn.so: cascade attention for the
 * target-verify step of top-k tree speculative decoding, on AMD MI355X (gfx950).
 *
 * The operation (cascade attention page, zdszero.github.io):
 *   request i has a prefix of L_i cached tokens and topk_i branches; branch j
 *   holds S_j draft tokens.  Draft token s of branch j attends the request's
 *   prefix plus draft tokens 0..s of its own branch (section "topk > 1").
 *   The cascade computes this as
 *     pass A  one attention over the request's prefix, read once, for every
 *             query row of all its branches  -> (o_A, LSE_A)
 *     pass B  one attention per branch over its own draft tokens under the
 *             causal in-branch ancestor mask  -> (o_B, LSE_B)
 *     merge   LSE = ln(e^LSE_A + e^LSE_B),
 *             o = e^(LSE_A-LSE) o_A + e^(LSE_B-LSE) o_B
 *   (sections "splittability of standard attention" and "mathematical
 *   structure of the cascade scheme").  Scores are sm_scale * q.k; LSE values
 *   are natural logarithms.  An empty key set has o = 0, LSE = -inf.
 *
 * Paged KV (KV-cache tutorial page, sections 5.2-5.3 and 6.2): one layer's K
 * and V each live in a pool of fixed-size pages; a block-table row lists the
 * physical page of each logical page of a sequence.  Token at logical slot t
 * of row r is at page table[r][t / page_size], offset t % page_size.  Pages
 * may be shared between rows (prefix sharing); the library only reads them.
 * Query head h uses kv head h / (Hq / Hkv) (tutorial section 6.3, GQA).
 *
 * Conventions for every entry point:
 *  - All array pointers are device pointers owned by the caller.  The library
 *    never allocates, frees or synchronises; work is enqueued on `stream`
 *    (a hipStream_t passed as void*, NULL = the default stream).
 *  - Every argument check runs on the host before any HIP call; a failed check
 *    returns a status and launches nothing.  cascade_last_error() then holds
 *    a message (thread-local).
 *  - Array *contents* (page ids, lengths, indptr monotonicity, the host-side
 *    maxima in cascade_tree) are the caller's contract.  Kernels never read
 *    outside the pool for a page id outside [0, num_pages) or a row outside
 *    [0, total_rows): such keys/rows are skipped and a sticky device flag is
 *    raised, readable with cascade_device_error().
 *  - Outputs must not alias inputs.
 */
#ifndef CASCADE_ATTN_H
#define CASCADE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define CASCADE_API __attribute__((visibility("default")))
#else
#define CASCADE_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CASCADE_OK = 0,
  CASCADE_ERR_NULL = 1,        /* a required pointer is NULL                          */
  CASCADE_ERR_SHAPE = 2,       /* inconsistent sizes (e.g. Hq % Hkv != 0, negative)  */
  CASCADE_ERR_UNSUPPORTED = 3, /* head_dim, page size, stride or alignment not handled */
  CASCADE_ERR_WORKSPACE = 4,   /* workspace missing or smaller than required         */
  CASCADE_ERR_HIP = 5          /* a HIP runtime call failed (message in last_error)  */
} cascade_status;

typedef enum { CASCADE_F32 = 0, CASCADE_BF16 = 1 } cascade_dtype;

/* Element type of the K/V pools.  FP8 KV (KV-cache tutorial page, section
 * 4.5: FP8 KV cache with per-tensor or per-channel scales): each element is
 * an OCP FP8 E4M3 code (1 sign bit, 4 exponent bits with bias 7, 3 mantissa
 * bits; no infinities; 0x7F and 0xFF are NaN; largest finite 448), and
 * element (page, slot, g, c) stands for code_value * k_scale *
 * k_channel_scale[g * head_dim + c] in K (1 in place of the channel factor
 * when k_channel_scale is NULL), and likewise with the v_ scales in V. */
typedef enum { CASCADE_KV_BF16 = 0, CASCADE_KV_FP8_E4M3 = 1 } cascade_kv_dtype;

/* One layer's paged K and V.  Element (page, slot, kv_head, c) of K is at
 * element offset page*page_stride + slot*token_stride + kv_head*head_stride + c
 * from k (elements of 2 bytes for bf16, 1 byte for FP8).
 * Requirements: head_dim in {64, 128}; page_size a power of two in [16, 4096];
 * the three strides are multiples of 8 elements, token_stride >= head_dim;
 * k and v 16-byte aligned.  dtype is a cascade_kv_dtype (0 = bf16); for FP8,
 * k_scale and v_scale must be finite and > 0 (they and the channel scales
 * are ignored for bf16).
 * The default layout [num_pages, page_size, Hkv, head_dim] has
 * page_stride = page_size*Hkv*head_dim, token_stride = Hkv*head_dim,
 * head_stride = head_dim. */
typedef struct {
  const void *k;
  const void *v;
  int32_t num_pages;
  int32_t page_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  int64_t page_stride;
  int64_t token_stride;
  int64_t head_stride;
  int32_t dtype;
  float k_scale;
  float v_scale;
  /* FP8 only (ignored for bf16): optional per-channel scales, device fp32
   * arrays [num_kv_heads, head_dim] (element (g, c) at g * head_dim + c),
   * 16-byte aligned, NULL = all ones; borrowed for the call; the caller keeps
   * them finite and > 0.  K's channel scales are applied to the query row
   * (q . (k * s) = (q * s) . k; the scaled query is rounded to bf16, which is
   * exact when the channel scales are powers of two), V's to each normalised
   * output channel. */
  const float *k_channel_scale;
  const float *v_channel_scale;
} cascade_paged_kv;

/* Queries, bf16 [total_rows, Hq, head_dim]; element (row, h, c) at
 * q + row*row_stride + h*head_stride + c.  Strides are multiples of 8
 * elements, q is 16-byte aligned.  Rows are ordered request-major, then
 * branch, then draft position.  sm_scale is usually 1/sqrt(head_dim); it must be
 * finite and > 0 (CASCADE_ERR_SHAPE otherwise). */
typedef struct {
  const void *q;
  int64_t row_stride;
  int64_t head_stride;
  int32_t num_qo_heads;
  int32_t total_rows;
  float sm_scale;
} cascade_query;

/* The verify tree (all arrays int32 unless stated, device):
 *  page_table        [batch_size, page_table_stride]  prefix block table per request
 *                    (the per-request page table of pass A)
 *  cache_seqlens     [batch_size]    L_i >= 0
 *  req_branch_indptr [batch_size+1]  branches of request i are [indptr[i], indptr[i+1])
 *  branch_qo_indptr  [num_branches+1] query rows of branch j; its S_j = diff rows are
 *                    also its draft keys.  The rows of request i are contiguous:
 *                    [branch_qo_indptr[req_branch_indptr[i]], ...[req_branch_indptr[i+1]]).
 *  draft_page_table  [num_branches, draft_page_table_stride] per-branch block table
 *                    (the per-branch page table of pass B)
 *  draft_start       [num_branches] or NULL: draft token u of branch j sits at logical
 *                    slot draft_start[j] + u of its row (NULL means 0).
 *  draft_mask        uint64 [total_rows, W] or NULL (8-byte aligned), W =
 *                    draft_mask_words (0 is taken as 1).  NULL: every branch is a
 *                    chain, its position s attends its positions 0..s.  Else a
 *                    general draft tree (tree attention mask, tutorial page section
 *                    8.2): the row of branch j's position s attends branch j's draft
 *                    positions u whose bit u % 64 of word u / 64 is set (its ancestors
 *                    and itself; a request's tree is one branch holding all of its
 *                    nodes, numbered so that parents precede children).  Requires
 *                    max_draft_len <= 64 * W and W <= 64 (CASCADE_ERR_UNSUPPORTED
 *                    otherwise); bits at or past S_j must be zero.
 * Host-side maxima, used to size launches; the caller promises them:
 *  max_prefix_len    >= every L_i
 *  max_request_rows  >= the number of query rows of every request
 *  max_draft_len     >= every S_j */
typedef struct {
  int32_t batch_size;
  int32_t num_branches;
  const int32_t *page_table;
  int32_t page_table_stride;
  const int32_t *cache_seqlens;
  const int32_t *req_branch_indptr;
  const int32_t *branch_qo_indptr;
  const int32_t *draft_page_table;
  int32_t draft_page_table_stride;
  const int32_t *draft_start;
  int32_t max_prefix_len;
  int32_t max_request_rows;
  int32_t max_draft_len;
  const uint64_t *draft_mask;
  int32_t draft_mask_words;
} cascade_tree;

/* Bytes of workspace cascade_prefix_attn and cascade_verify_attn take for these
 * shapes: the partial states of a split prefix, required when the prefix pass
 * is split, then, for launches of more than 80 query rows per (request, kv
 * head) at head_dim 128, room for a work list that the call builds on the
 * device (the launch's work items, longest first).  The work list is
 * optional: a workspace that holds the partial states but not the list (or
 * none, when the prefix is unsplit) gives the same results with the items
 * taken in a fixed order.  0 when neither applies; 0 on invalid arguments. */
CASCADE_API size_t cascade_workspace_size(const cascade_query *q, const cascade_paged_kv *kv,
                              const cascade_tree *tree);

/* Pass A (cascade page, "mathematical structure", first attention): for every
 * request, all query rows of all its branches attend the L_i prefix tokens,
 * each page read once per (request, kv head).  Writes o_a float32
 * [total_rows, Hq, head_dim] and lse_a float32 [total_rows, Hq] (LSE_A = -inf,
 * o_A = 0 for L_i = 0).  Long prefixes are split into chunks whose partial
 * states go to `workspace` and are merged with the same LSE identity. */
CASCADE_API cascade_status cascade_prefix_attn(const cascade_query *q, const cascade_paged_kv *kv,
                                   const cascade_tree *tree, float *o_a, float *lse_a,
                                   void *workspace, size_t workspace_bytes, void *stream);

/* Pass B (same section, second attention): each branch's rows attend its own
 * S_j draft tokens; row s sees draft positions 0..s (the tree-attention
 * ancestor mask of the tutorial's section 8.2, itself included).  Writes o_b
 * float32 [total_rows, Hq, head_dim] and lse_b float32 [total_rows, Hq]. */
CASCADE_API cascade_status cascade_draft_attn(const cascade_query *q, const cascade_paged_kv *kv,
                                  const cascade_tree *tree, float *o_b, float *lse_b,
                                  void *stream);

/* The merge of two attention states over disjoint key sets (cascade page,
 * "splittability"): elementwise over num_rows*num_heads rows of head_dim.
 * o_a, o_b float32 [num_rows, num_heads, head_dim]; lse_a, lse_b float32
 * [num_rows, num_heads]; o in o_dtype with the same shape; lse (nullable)
 * float32.  A side with LSE = -inf contributes nothing; two such sides give
 * o = 0, LSE = -inf.  head_dim must be a multiple of 4; pointers 16-byte aligned. */
CASCADE_API cascade_status merge_state(const float *o_a, const float *lse_a, const float *o_b,
                           const float *lse_b, int64_t num_rows, int32_t num_heads,
                           int32_t head_dim, void *o, cascade_dtype o_dtype, float *lse,
                           void *stream);

/* The whole cascade in as few launches as the shapes allow: pass A, pass B and
 * the merge fused in one kernel when the prefix runs unsplit; otherwise a
 * first kernel runs pass A over the prefix splits (pass B joins the state of
 * split 0) and writes one partial state per split to the workspace, and a
 * second kernel merges the partial states with the same LSE identity.
 * o [total_rows, Hq, head_dim] in o_dtype, lse float32 (nullable). */
CASCADE_API cascade_status cascade_verify_attn(const cascade_query *q, const cascade_paged_kv *kv,
                                   const cascade_tree *tree, void *o, cascade_dtype o_dtype,
                                   float *lse, void *workspace, size_t workspace_bytes,
                                   void *stream);

/* cascade_verify_attn for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results, with the split-prefix workspace
 * taken from a file-scope device array of 32 MiB that the library holds on
 * each GPU it runs on until the process ends (its address is looked up once
 * per device, on the device current at the first call).  The call allocates
 * and frees nothing.  Shapes that need more workspace than the array holds
 * (cascade_workspace_size > 32 MiB) return CASCADE_ERR_WORKSPACE and launch
 * nothing.  Every call on one GPU shares that GPU's array: calls that overlap
 * in time on one GPU (other streams, other threads) race on it, so the
 * caller orders them.  The array's contents carry no meaning between calls
 * (every byte a call reads it first writes).  The stream must belong to the
 * current device. */
CASCADE_API cascade_status cascade_verify_attn_noalloc(const cascade_query *q, const cascade_paged_kv *kv,
                                           const cascade_tree *tree, void *o, cascade_dtype o_dtype,
                                           float *lse, void *stream);

/* Baseline (cascade page, naive expansion): the batch expanded into one
 * virtual request per branch; each reads its request's whole prefix and its
 * own drafts and runs one softmax.  Same outputs as cascade_verify_attn. */
CASCADE_API cascade_status naive_expand(const cascade_query *q, const cascade_paged_kv *kv,
                            const cascade_tree *tree, void *o, cascade_dtype o_dtype,
                            float *lse, void *stream);

CASCADE_API const char *cascade_status_string(cascade_status s);
CASCADE_API const char *cascade_last_error(void);

/* Test hooks, built on the same index helpers the attention kernels use.
 * cascade_debug_gather: which = 0 copies request `index`'s L_i prefix tokens,
 * which = 1 branch `index`'s S_j draft tokens, of kv head `kv_head`, into k_out
 * and v_out (bf16 [count, head_dim], device, sized by the caller).  FP8 codes
 * come out widened to bf16 (exact; scales not applied) by the conversion the
 * attention kernels use.
 * cascade_debug_mask: branch `branch`'s visibility over [its request's prefix ;
 * its drafts] as uint8 [S_j, L_i + S_j] (1 = visible), device, sized by the caller. */
CASCADE_API cascade_status cascade_debug_gather(const cascade_paged_kv *kv, const cascade_tree *tree,
                                    int32_t which, int32_t index, int32_t kv_head,
                                    void *k_out, void *v_out, void *stream);
CASCADE_API cascade_status cascade_debug_mask(const cascade_tree *tree, int32_t branch,
                                  uint8_t *mask_out, int32_t mask_cols, void *stream);

/* Reads (and with clear != 0 resets) the sticky device flag raised when a
 * kernel met a page id or row outside its bounds.  Synchronises the device. */
CASCADE_API cascade_status cascade_device_error(int32_t *flag_out, int32_t clear);

/* The serving step around verification (tutorial page, section 5.2: pages
 * through the block table; section 7, 7.1 and 7.6: the verify and rollback
 * loop, where rejected drafts are dropped by not advancing the length):
 *
 * cascade_append_draft_kv writes the K and V of every query row's draft token
 * into its page before the verify pass reads them: row r, position u of branch
 * j, goes to logical slot draft_start[j] + u of draft block-table row j.
 * k_new, v_new: [total_rows, num_kv_heads, head_dim] in the pool's element
 * type (bf16, or FP8 E4M3 codes that the caller quantised with the pool's
 * scales), element (r, g, c) at element offset r*new_row_stride +
 * g*new_head_stride + c (strides multiples of 8 elements, 16-byte aligned,
 * device); total_rows must be branch_qo_indptr[
 * num_branches].  Rows whose slot has no valid page are skipped and raise the
 * sticky device flag.  Asynchronous on stream; the pool is written in place.
 *
 * cascade_commit_accepted appends the accepted drafts to the prefixes after
 * verification: for request i the rows accepted_rows[accepted_indptr[i] ..
 * accepted_indptr[i+1]) (global query rows, in path order, device int32) have
 * their draft K/V copied to logical slots L_i, L_i + 1, ... of block-table row
 * i (those slots must already be mapped: the caller owns page allocation), then
 * cache_seqlens_out[i] = L_i + their count (cache_seqlens_out may be
 * t->cache_seqlens itself: the lengths are updated in place by a second
 * launch).  max_accepted >= every request's count.  The rows of a request are
 * copied in path order and every copy reads the value its source held before
 * the call, so destination L_i + k may be the draft slot of the k-th or of an
 * earlier accepted row (drafts continuing the prefix pages with
 * draft_start = L_i, and an accepted path that skips nodes, e.g. nodes
 * [0, 2, 5]); it must not be the draft slot of a later accepted row.
 * Rejected drafts cost nothing: their slots are rewritten by the next append.
 * Both calls are graph-capturable. */
CASCADE_API cascade_status cascade_append_draft_kv(const cascade_paged_kv *kv, const cascade_tree *t,
                                       int32_t total_rows, const void *k_new, const void *v_new,
                                       int64_t new_row_stride, int64_t new_head_stride, void *stream);
CASCADE_API cascade_status cascade_commit_accepted(const cascade_paged_kv *kv, const cascade_tree *t,
                                       int32_t total_rows, const int32_t *accepted_indptr,
                                       const int32_t *accepted_rows, int32_t max_accepted,
                                       int32_t *cache_seqlens_out, void *stream);

/* Measurement reference: a plain streaming read of `bytes` (multiple of 16) of
 * device memory at buf (16-byte aligned), nothing written except, in a case
 * that does not occur for real data, one word at sink (device, 4 bytes).
 * Asynchronous on stream. */
CASCADE_API cascade_status cascade_stream_read(const void *buf, size_t bytes, uint32_t *sink, void *stream);

/* Kernel timing, for measurement tools.  With enable != 0, every later
 * cascade_verify_attn call on this thread launches its kernels with HIP events
 * recorded by the command processor immediately around them (the first
 * kernel's start, the last kernel's end); enable = 0 turns it off.  The events
 * are created on the current device by the first enabling call.
 * cascade_last_verify_ms: the elapsed time between those two events of the
 * latest timed call, in ms; synchronises on the stop event.  Returns
 * CASCADE_ERR_SHAPE when no call has been timed since timing was enabled. */
CASCADE_API cascade_status cascade_kernel_timing(int32_t enable);
CASCADE_API cascade_status cascade_last_verify_ms(float *ms_out);

#ifdef __cplusplus
}
#endif

#endif /* CASCADE_ATTN_H */
