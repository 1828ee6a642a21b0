// C entry points of libcascade_attn.so: argument checks (all on the host,
// before any HIP call), launch planning, and dispatch to the kernels.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "../../include/cascade_attn.h"
#include "launch.h"

namespace {

thread_local std::string g_last_error;

cascade_status fail(cascade_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

cascade_status hip_fail(hipError_t e, const char* what) {
  return fail(CASCADE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

int ilog2(int x) {
  int r = 0;
  while ((1 << r) < x) ++r;
  return r;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Work items wanted per launch before the prefix is split: one per CU of an
// MI355X for the key-split kernel, two per CU for the pair kernel (which
// fits two workgroups on a CU); and the bounds on keys per split.
constexpr int kTargetItems = 256;
constexpr int kPairTargetItems = 512;
constexpr int kMinSplitKeys = 256;
// The pair kernel splits a prefix only into splits of at least this many keys
// (eight 32-key tiles per wave): a split's partial states cost a round trip
// through the workspace and a merge launch, which shorter splits do not earn
// back (GQA configuration, 8 requests x 1000 keys: 24.7 us unsplit in 16-row
// chunks against 26.4-28.1 us split in two or four).
constexpr int kPairMinSplitKeys = 1024;
constexpr int kMaxSplitKeys = 4096;
// The row-split kernel takes its items longest first from its work list, so
// it balances many items of unequal length: it splits a prefix only to reach
// four items per workgroup slot (two per CU), into splits of 1024 to 16384
// keys (ragged batch: 0.62 ms, against 0.66 ms with splits of at most 4096
// keys, whose partial states cost more than they balance).
constexpr int kRowTargetItems = 4 * kPairTargetItems;
constexpr int kRowMaxSplitKeys = 16384;
constexpr int kMaxRowBlocks = 5;

struct Plan {
  int group = 1;
  int rb = 1;        // 16-row blocks per chunk (key-split kernel, split merges)
  int n_chunks = 1;  // row chunks per (segment, kv head) of the key-split kernel
  int n_splits = 1;  // key splits of the prefix
  int split_len = 32;
  int64_t items = 0;  // segments * kv heads * chunks (key-split kernel)
  // Pass A and the fused verify pass on the pair kernel: chunks of at most
  // pair_rows rows, pair_chunks per (request, kv head).
  bool pair = false;
  int pair_chunks = 1;
  int pair_rows = 0;
  // Pass A, the fused verify pass and pass B on the row-split kernel: chunks
  // of kRowsPerItem rows, row_chunks per (request, kv head).
  bool rows_kernel = false;
  int row_chunks = 1;
};

void plan_rows(Plan& p, int64_t rows_per_segment) {
  const int64_t blocks = rows_per_segment > 0 ? cdiv(rows_per_segment, 16) : 1;
  p.rb = (int)(blocks < kMaxRowBlocks ? blocks : kMaxRowBlocks);
  p.n_chunks = (int)(rows_per_segment > 0 ? cdiv(rows_per_segment, 16 * p.rb) : 1);
}

// Key splits for `items` work items: enough to reach `target` items when the
// prefix is long enough, at most kMaxSplitKeys keys per split.
void plan_splits(Plan& p, int max_len, int64_t items, int64_t target, int min_split_keys = kMinSplitKeys,
                 int max_split_keys = kMaxSplitKeys) {
  const int len = max_len > 0 ? max_len : 1;
  int64_t n = 1;
  // An empty launch (no requests) has no items to fill the device with.
  if (len > 2 * min_split_keys && items > 0 && items < target) {
    n = cdiv(target, items);
    const int64_t cap = cdiv(len, min_split_keys);
    if (n > cap) n = cap;
  }
  if (cdiv(len, n) > max_split_keys) n = cdiv(len, max_split_keys);
  p.split_len = (int)(cdiv(cdiv(len, n), 32) * 32);
  p.n_splits = (int)cdiv(len, p.split_len);
}

bool kv_fp8(const cascade_paged_kv* kv) { return kv->dtype == CASCADE_KV_FP8_E4M3; }

// 64-bit words per row of a draft-tree mask (0 is taken as 1), and the most
// a launch accepts (4096 nodes per branch).
constexpr int kMaxMaskWords = 64;
int mask_words(const cascade_tree* t) { return t->draft_mask_words > 1 ? t->draft_mask_words : 1; }
int elem_bytes(const cascade_paged_kv* kv) { return kv_fp8(kv) ? 1 : 2; }

// Bytes from the start of a page to the end of its last (token, head) row.
int64_t page_extent_bytes(const cascade_paged_kv* kv) {
  return ((int64_t)(kv->page_size - 1) * kv->token_stride +
          (int64_t)(kv->num_kv_heads - 1) * kv->head_stride + kv->head_dim) * elem_bytes(kv);
}

casc::KvView kv_view(const cascade_paged_kv* kv) {
  casc::KvView v{};
  v.k = static_cast<const uint16_t*>(kv->k);
  v.v = static_cast<const uint16_t*>(kv->v);
  v.page_stride = kv->page_stride;
  v.token_stride = kv->token_stride;
  v.head_stride = kv->head_stride;
  v.num_pages = kv->num_pages;
  v.log2_page = ilog2(kv->page_size);
  v.page_bytes = (int32_t)page_extent_bytes(kv);
  v.elem_bytes = elem_bytes(kv);
  v.page_stride_b = (uint32_t)(kv->page_stride * elem_bytes(kv));
  v.token_stride_b = (uint32_t)(kv->token_stride * elem_bytes(kv));
  return v;
}

cascade_status check_kv(const cascade_paged_kv* kv) {
  if (!kv) return fail(CASCADE_ERR_NULL, "kv is NULL");
  if (!kv->k || !kv->v) return fail(CASCADE_ERR_NULL, "kv->k or kv->v is NULL");
  if (kv->num_kv_heads <= 0) return fail(CASCADE_ERR_SHAPE, "num_kv_heads must be > 0");
  if (kv->num_pages <= 0) return fail(CASCADE_ERR_SHAPE, "num_pages must be > 0");
  if (kv->dtype != CASCADE_KV_BF16 && kv->dtype != CASCADE_KV_FP8_E4M3)
    return fail(CASCADE_ERR_UNSUPPORTED, "kv dtype %d not supported (bf16 or fp8 e4m3)", (int)kv->dtype);
  if (kv_fp8(kv) && !(std::isfinite(kv->k_scale) && kv->k_scale > 0.f && std::isfinite(kv->v_scale) &&
                      kv->v_scale > 0.f))
    return fail(CASCADE_ERR_SHAPE, "fp8 kv needs finite k_scale and v_scale > 0");
  if (kv_fp8(kv) && !(aligned16(kv->k_channel_scale) && aligned16(kv->v_channel_scale)))
    return fail(CASCADE_ERR_UNSUPPORTED, "fp8 channel scales must be 16-byte aligned");
  if (kv->head_dim != 64 && kv->head_dim != 128)
    return fail(CASCADE_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", kv->head_dim);
  if (!is_pow2(kv->page_size) || kv->page_size < 16 || kv->page_size > 4096)
    return fail(CASCADE_ERR_UNSUPPORTED, "page_size %d not supported (power of two in [16, 4096])",
                kv->page_size);
  if (kv->page_stride < 0 || kv->token_stride < 0 || kv->head_stride < 0)
    return fail(CASCADE_ERR_SHAPE, "kv strides must be >= 0");
  if (kv->page_stride % 8 || kv->token_stride % 8 || kv->head_stride % 8)
    return fail(CASCADE_ERR_UNSUPPORTED, "kv strides must be multiples of 8 elements");
  if (kv->token_stride < kv->head_dim)
    return fail(CASCADE_ERR_UNSUPPORTED, "token_stride must be >= head_dim (rows of one kv head may not overlap)");
  if (!aligned16(kv->k) || !aligned16(kv->v))
    return fail(CASCADE_ERR_UNSUPPORTED, "kv->k and kv->v must be 16-byte aligned");
  if (page_extent_bytes(kv) >= (1ll << 30))
    return fail(CASCADE_ERR_UNSUPPORTED, "one page spans more than 1 GiB");
  if (kv->page_stride * elem_bytes(kv) >= (1ll << 31))
    return fail(CASCADE_ERR_UNSUPPORTED, "page_stride spans 2 GiB or more");
  return CASCADE_OK;
}

cascade_status check_query(const cascade_query* q, const cascade_paged_kv* kv) {
  if (!q) return fail(CASCADE_ERR_NULL, "q is NULL");
  if (!q->q && q->total_rows > 0) return fail(CASCADE_ERR_NULL, "q->q is NULL");
  if (q->num_qo_heads <= 0) return fail(CASCADE_ERR_SHAPE, "num_qo_heads must be > 0");
  if (q->num_qo_heads % kv->num_kv_heads)
    return fail(CASCADE_ERR_SHAPE, "num_qo_heads (%d) must be a multiple of num_kv_heads (%d)",
                q->num_qo_heads, kv->num_kv_heads);
  if (q->total_rows < 0) return fail(CASCADE_ERR_SHAPE, "total_rows must be >= 0");
  if (q->row_stride < 0 || q->head_stride < 0) return fail(CASCADE_ERR_SHAPE, "q strides must be >= 0");
  if (q->row_stride % 8 || q->head_stride % 8)
    return fail(CASCADE_ERR_UNSUPPORTED, "q strides must be multiples of 8 elements");
  if (q->q && !aligned16(q->q)) return fail(CASCADE_ERR_UNSUPPORTED, "q must be 16-byte aligned");
  // The kernels take the running row max over raw scores and scale it
  // afterwards, which is the max of the scaled scores only for a positive
  // scale; a zero scale would also turn masked (-inf) scores into NaN.
  if (!std::isfinite(q->sm_scale) || !(q->sm_scale > 0.f))
    return fail(CASCADE_ERR_SHAPE, "sm_scale must be finite and > 0");
  return CASCADE_OK;
}

cascade_status check_tree(const cascade_tree* t, const cascade_paged_kv* kv) {
  if (!t) return fail(CASCADE_ERR_NULL, "tree is NULL");
  if (t->batch_size < 0 || t->num_branches < 0) return fail(CASCADE_ERR_SHAPE, "negative batch_size/num_branches");
  if (t->max_prefix_len < 0 || t->max_request_rows < 0 || t->max_draft_len < 0)
    return fail(CASCADE_ERR_SHAPE, "negative maxima in tree");
  if (t->batch_size > 0) {
    if (!t->cache_seqlens || !t->req_branch_indptr || !t->branch_qo_indptr)
      return fail(CASCADE_ERR_NULL, "cache_seqlens, req_branch_indptr and branch_qo_indptr are required");
    if (t->max_prefix_len > 0 && !t->page_table) return fail(CASCADE_ERR_NULL, "page_table is NULL");
    if (t->num_branches < t->batch_size)
      return fail(CASCADE_ERR_SHAPE, "num_branches (%d) < batch_size (%d)", t->num_branches, t->batch_size);
  }
  if (t->num_branches > 0 && t->batch_size == 0)
    return fail(CASCADE_ERR_SHAPE, "branches without requests (batch_size = 0)");
  if (t->num_branches > 0 && !t->draft_page_table) return fail(CASCADE_ERR_NULL, "draft_page_table is NULL");
  if (t->page_table_stride < 0 || t->draft_page_table_stride < 0)
    return fail(CASCADE_ERR_SHAPE, "negative block-table stride");
  if ((int64_t)t->page_table_stride * kv->page_size < t->max_prefix_len)
    return fail(CASCADE_ERR_SHAPE, "page_table_stride * page_size (%lld) < max_prefix_len (%d)",
                (long long)t->page_table_stride * kv->page_size, t->max_prefix_len);
  if (t->num_branches > 0 && t->draft_start == nullptr &&
      (int64_t)t->draft_page_table_stride * kv->page_size < t->max_draft_len)
    return fail(CASCADE_ERR_SHAPE, "draft_page_table_stride * page_size < max_draft_len");
  if (t->draft_mask) {
    const int words = mask_words(t);
    if (t->draft_mask_words < 0 || words > kMaxMaskWords)
      return fail(CASCADE_ERR_UNSUPPORTED, "draft_mask_words %d not supported (0 .. %d)", (int)t->draft_mask_words,
                  kMaxMaskWords);
    if (t->max_draft_len > 64 * words)
      return fail(CASCADE_ERR_UNSUPPORTED,
                  "draft trees (draft_mask) are limited to 64 * draft_mask_words = %d nodes per branch",
                  64 * words);
    if (reinterpret_cast<uintptr_t>(t->draft_mask) & 7u)
      return fail(CASCADE_ERR_UNSUPPORTED, "draft_mask must be 8-byte aligned");
  }
  return CASCADE_OK;
}

cascade_status check_all(const cascade_query* q, const cascade_paged_kv* kv, const cascade_tree* t) {
  cascade_status s = check_kv(kv);
  if (s != CASCADE_OK) return s;
  if ((s = check_query(q, kv)) != CASCADE_OK) return s;
  if ((s = check_tree(t, kv)) != CASCADE_OK) return s;
  return CASCADE_OK;
}

casc::AttnArgs make_args(const cascade_query* q, const cascade_paged_kv* kv, const cascade_tree* t,
                         const Plan& p) {
  casc::AttnArgs a{};
  a.q = static_cast<const uint16_t*>(q->q);
  a.q_row_stride = q->row_stride;
  a.q_head_stride = q->head_stride;
  a.num_qo_heads = q->num_qo_heads;
  a.group = p.group;
  a.total_rows = q->total_rows;
  // FP8 pools: scores are sm_scale * k_scale * (q . codes), the V scale
  // multiplies the normalised output (a per-tensor scale factors out of both
  // sums).
  const double k_scale = kv_fp8(kv) ? (double)kv->k_scale : 1.0;
  a.scale_log2 = (float)((double)q->sm_scale * k_scale * 1.4426950408889634);
  a.v_scale = kv_fp8(kv) ? kv->v_scale : 1.f;
  a.k_cs = kv_fp8(kv) ? kv->k_channel_scale : nullptr;
  a.v_cs = kv_fp8(kv) ? kv->v_channel_scale : nullptr;
  a.kv = kv_view(kv);
  a.num_kv_heads = kv->num_kv_heads;
  a.batch_size = t->batch_size;
  a.page_table = t->page_table;
  a.page_table_stride = t->page_table_stride;
  a.cache_seqlens = t->cache_seqlens;
  a.req_branch_indptr = t->req_branch_indptr;
  a.branch_qo_indptr = t->branch_qo_indptr;
  a.draft_page_table = t->draft_page_table;
  a.draft_page_table_stride = t->draft_page_table_stride;
  a.draft_start = t->draft_start;
  a.draft_mask = t->draft_mask;
  a.draft_mask_words = mask_words(t);
  a.n_chunks = p.n_chunks;
  a.grid_splits = 1;
  a.n_splits = p.n_splits;
  a.split_len = p.split_len;
  return a;
}

// Query rows per (request, kv head) from which pass A, the fused verify pass
// and pass B run the row-split kernel (head dim 128, bf16 or FP8 pools): more
// than one key-split chunk holds.  Its workgroups share each K/V tile among
// four waves of 32 rows through LDS, and with a workspace its items come from
// a device-built work list, longest first and none empty: on the ragged batch
// (64 requests, 48 to 512 rows per kv head, prefixes of 512 to 32768 keys)
// 0.65 ms against 0.91 ms on the pair kernel in 48-row chunks.
constexpr int64_t kRowKernelMinRows = 16 * kMaxRowBlocks + 1;
// Rows per (request, kv head) from which the row-split kernel (bf16 pools)
// runs three workgroups per CU with three copy stages instead of two with
// four: many full 128-row items (prefix hit, fused: 2.52 -> 2.24 ms at
// h = 0, 1.87 -> 1.69 ms at h = 0.5), while batches of short items that
// stream from HBM (the ragged batch, at most 512 rows) keep the deeper copy
// pipeline (0.59 against 0.60 ms).
constexpr int64_t kRowThreeWaveRows = 1024;

// Plan of the per-request launches (pass A, pass B, verify).  At head_dim 128,
// pass A and the fused verify pass of requests with at most 16 * kMaxRowBlocks
// rows per kv head run on the pair kernel (chunks of up to kPairRows rows,
// two workgroups per CU, the chunks of a (request, kv head) sharing its
// prefix stream through one L2) -- except launches whose (request, kv head)
// pairs already fill the device with one chunk each: there the key-split
// kernel, one workgroup per CU holding all rows, measured faster (32 requests
// x 8 kv heads x 80 rows: 60.6 against 64.5 us over bf16 pools, 53.3 against
// 54.7 us over FP8 pools).  With too few (request, kv head) pairs to fill the
// device, a request's rows are cut in more chunks before its prefix is split;
// when even one 16-row block per chunk leaves at most a workgroup per CU (the
// GQA configuration: 8 requests x 8 kv heads x 48 rows, 192 chunks), the
// key-split kernel runs those 16-row chunks, its four waves sharing each
// chunk's prefix (19.9 us there, against 21.5 us on the pair kernel with
// 12-row chunks and 24.8 us with 16-row chunks padded to 48), and a prefix
// is split only past 2 * kPairMinSplitKeys keys.
Plan plan_request(const cascade_query* q, const cascade_paged_kv* kv, const cascade_tree* t) {
  Plan p;
  p.group = q->num_qo_heads / kv->num_kv_heads;
  const int64_t rows = (int64_t)t->max_request_rows * p.group;
  plan_rows(p, rows);
  const int64_t pairs = (int64_t)t->batch_size * kv->num_kv_heads;
  const bool thin = rows > 0 && rows <= 16 * kMaxRowBlocks && pairs * cdiv(rows, 16) <= kTargetItems;
  if (thin) {
    p.rb = 1;
    p.n_chunks = (int)cdiv(rows, 16);
  }
  p.items = pairs * p.n_chunks;
  const bool one_chunk_fills = rows <= 16 * kMaxRowBlocks && pairs >= kTargetItems;
  p.pair = !thin && kv->head_dim == 128 && rows > 0 && rows < kRowKernelMinRows && !one_chunk_fills;
  p.rows_kernel = kv->head_dim == 128 && rows >= kRowKernelMinRows;
  if (p.rows_kernel) {
    // Splits planned from the row-split kernel's own work items.
    p.row_chunks = (int)cdiv(rows, casc::kRowsPerItem);
    plan_splits(p, t->max_prefix_len, pairs * p.row_chunks, kRowTargetItems, kPairMinSplitKeys, kRowMaxSplitKeys);
  } else if (p.pair) {
    p.pair_chunks = (int)cdiv(rows, casc::kPairRows);
    // Few (request, kv head) pairs: smaller chunks (down to one 16-row block)
    // until the launch holds a workgroup per CU.
    while (pairs * p.pair_chunks < kTargetItems && cdiv(rows, p.pair_chunks + 1) >= 16) ++p.pair_chunks;
    p.pair_rows = (int)cdiv(rows, p.pair_chunks);
    plan_splits(p, t->max_prefix_len, pairs * p.pair_chunks, kPairTargetItems, kPairMinSplitKeys);
  } else {
    plan_splits(p, t->max_prefix_len, p.items, kTargetItems, thin ? kPairMinSplitKeys : kMinSplitKeys);
  }
  return p;
}

// Workgroups of one key split of the pair kernel: (request, kv head) pairs
// rounded up to a multiple of the 8 XCDs, times the row chunks.
int64_t pair_grid_per_split(const cascade_tree* t, const cascade_paged_kv* kv, const Plan& p) {
  return cdiv((int64_t)t->batch_size * kv->num_kv_heads, 8) * 8 * p.pair_chunks;
}

// Workspace: the split partial states (required when the prefix is split),
// then the row-split kernel's work list (optional: without room for it the
// launch takes its items in the fixed grid order).
struct WsLayout {
  size_t required = 0;  // partial states
  size_t bytes = 0;     // partial states and work list
  size_t lse_off = 0;
  size_t list_off = 0;  // work-list count, then the entries 256 bytes on
  int64_t list_entries = 0;
};

WsLayout ws_layout(const cascade_query* q, const cascade_paged_kv* kv, const cascade_tree* t, const Plan& p) {
  WsLayout w;
  size_t end = 0;
  if (p.n_splits > 1) {
    const size_t plane = (size_t)q->total_rows * q->num_qo_heads;
    const size_t o_bytes = (size_t)p.n_splits * plane * kv->head_dim * sizeof(float);
    w.lse_off = (o_bytes + 255) / 256 * 256;
    end = w.lse_off + (size_t)p.n_splits * plane * sizeof(float);
  }
  w.required = end;
  if (p.rows_kernel && t->batch_size > 0) {
    w.list_entries = (int64_t)t->batch_size * p.n_splits * p.row_chunks;
    w.list_off = (end + 255) / 256 * 256;
    end = w.list_off + 256 + (size_t)w.list_entries * sizeof(int32_t);
  }
  w.bytes = end;
  return w;
}

// The work list of a row-split launch in `ws`, or null when the workspace
// has no room for it.
void attach_work_list(casc::AttnArgs& a, const WsLayout& wl, void* ws, size_t ws_bytes) {
  if (wl.list_entries <= 0 || !ws || ws_bytes < wl.bytes) return;
  char* base = static_cast<char*>(ws) + wl.list_off;
  a.work_count = reinterpret_cast<int32_t*>(base);
  a.work_list = reinterpret_cast<int32_t*>(base + 256);
}

// Arguments of the split merge that follows a split prefix or verify pass.
casc::SplitMergeArgs split_merge_args(const cascade_query* q, const cascade_paged_kv* kv, const cascade_tree* t,
                                      const Plan& p, const casc::AttnArgs& a, bool verify) {
  casc::SplitMergeArgs m{};
  m.ws_o = a.ws_o;
  m.ws_lse = a.ws_lse;
  m.n_splits = p.n_splits;
  m.split_len = p.split_len;
  m.total_rows = q->total_rows;
  m.num_qo_heads = q->num_qo_heads;
  m.head_dim = kv->head_dim;
  m.batch_size = t->batch_size;
  const int64_t cap = (int64_t)t->page_table_stride * kv->page_size;
  const int64_t planned = (int64_t)p.n_splits * p.split_len;
  m.len_cap = (int32_t)(cap < planned ? cap : planned);
  m.verify = verify ? 1 : 0;
  m.cache_seqlens = t->cache_seqlens;
  m.req_branch_indptr = t->req_branch_indptr;
  m.branch_qo_indptr = t->branch_qo_indptr;
  m.o = a.o;
  m.o_bf16 = a.o_bf16;
  m.lse = a.lse;
  return m;
}

// Workgroups of the key-split kernel: `seg_items` (segment, kv head) pairs
// rounded up to a multiple of the 8 XCDs, times the row chunks and splits.
int64_t xcd_grid(int64_t seg_items, int n_chunks, int splits) { return cdiv(seg_items, 8) * 8 * n_chunks * splits; }

hipError_t launch(int mode, int head_dim, int rb, casc::AttnArgs a, int64_t seg_items, int splits, hipStream_t s,
                  hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr) {
  a.n_seg_items = (int32_t)seg_items;
  const int64_t grid = xcd_grid(seg_items, a.n_chunks, splits);
  if (seg_items <= 0 || grid <= 0) return hipSuccess;
  const bool fp8 = a.kv.elem_bytes == 1;
  if (head_dim == 64)
    return fp8 ? casc::launch_attn_d64_fp8(mode, rb, a, (int)grid, s, e0, e1)
               : casc::launch_attn_d64(mode, rb, a, (int)grid, s, e0, e1);
  return fp8 ? casc::launch_attn_d128_fp8(mode, rb, a, (int)grid, s, e0, e1)
             : casc::launch_attn_d128(mode, rb, a, (int)grid, s, e0, e1);
}


// Pass A, the fused verify pass or pass B (`mode`), unsplit or one launch of
// the splits: the row-split kernel (head dim 128, row-heavy
// requests) over chunks of up to kRowsPerItem query rows, else the key-split
// kernel of the plan.
hipError_t launch_row_modes(int mode, const cascade_paged_kv* kv,
                               const cascade_tree* t, const Plan& p, casc::AttnArgs a, int splits,
                               hipStream_t s, hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr) {
  if (p.pair && (mode == casc::kModePrefix || mode == casc::kModeVerify)) {
    a.n_chunks = p.pair_chunks;
    a.chunk_rows = p.pair_rows;
    const int64_t grid = pair_grid_per_split(t, kv, p) * splits;
    if (grid <= 0) return hipSuccess;
    return kv_fp8(kv) ? casc::launch_pair_d128_fp8(mode, a, (int)grid, s, e0, e1)
                      : casc::launch_pair_d128(mode, a, (int)grid, s, e0, e1);
  }
  if (!p.rows_kernel)
    return launch(mode, kv->head_dim, p.rb, a, (int64_t)t->batch_size * kv->num_kv_heads, splits, s, e0, e1);
  a.n_chunks = p.row_chunks;
  a.n_seg_items = (int32_t)((int64_t)t->batch_size * kv->num_kv_heads);
  int64_t grid = xcd_grid(a.n_seg_items, a.n_chunks, splits);
  if (a.work_list) {
    casc::WorkListArgs w{};
    w.batch_size = t->batch_size;
    w.cache_seqlens = t->cache_seqlens;
    w.req_branch_indptr = t->req_branch_indptr;
    w.branch_qo_indptr = t->branch_qo_indptr;
    w.num_branches = t->num_branches;
    w.group = p.group;
    w.n_chunks = a.n_chunks;
    w.n_splits = a.n_splits;
    w.split_len = a.split_len;
    w.drafts = mode != casc::kModePrefix;
    // Work buckets of 2^shift tiles: the longest item below 256 buckets.
    const int64_t most = cdiv(p.split_len, 32) + cdiv((int64_t)t->max_request_rows, 32);
    while ((most >> w.bucket_shift) >= 255) ++w.bucket_shift;
    w.list = const_cast<int32_t*>(a.work_list);
    w.count = const_cast<int32_t*>(a.work_count);
    const hipError_t e = casc::launch_worklist(w, s, e0);
    if (e != hipSuccess) return e;
    e0 = nullptr;
    grid = (int64_t)t->batch_size * a.n_splits * a.n_chunks * kv->num_kv_heads;
  }
  if (grid <= 0) return hipSuccess;
  // Launches of full items (at least kRowThreeWaveRows rows per pair: a
  // prefix-hit suffix prefill) run three workgroups per CU.
  const bool three_wave = (int64_t)t->max_request_rows * p.group >= kRowThreeWaveRows;
  return kv_fp8(kv) ? casc::launch_rows_d128_fp8(mode, a, (int)grid, s, e0, e1)
                    : casc::launch_rows_d128(mode, three_wave, a, (int)grid, s, e0, e1);
}

// Kernel timing of cascade_verify_attn (per thread; see the header).
struct KernelTiming {
  bool enabled = false;
  bool recorded = false;
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
thread_local KernelTiming g_timing;

cascade_status check_grid(int64_t grid);
cascade_status check_plan_grid(const cascade_tree* t, const cascade_paged_kv* kv, const Plan& p) {
  const int64_t pair = p.pair ? pair_grid_per_split(t, kv, p) * p.n_splits : 0;
  const int64_t ks = xcd_grid((int64_t)t->batch_size * kv->num_kv_heads, p.n_chunks, p.n_splits);
  return check_grid(pair > ks ? pair : ks);
}
cascade_status check_grid(int64_t grid) {
  if (grid > INT32_MAX) return fail(CASCADE_ERR_SHAPE, "launch too large (%lld work items)", (long long)grid);
  return CASCADE_OK;
}

}  // namespace

extern "C" {

const char* cascade_status_string(cascade_status s) {
  switch (s) {
    case CASCADE_OK: return "ok";
    case CASCADE_ERR_NULL: return "null pointer";
    case CASCADE_ERR_SHAPE: return "inconsistent shape";
    case CASCADE_ERR_UNSUPPORTED: return "unsupported configuration";
    case CASCADE_ERR_WORKSPACE: return "workspace too small";
    case CASCADE_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* cascade_last_error(void) { return g_last_error.c_str(); }

size_t cascade_workspace_size(const cascade_query* q, const cascade_paged_kv* kv, const cascade_tree* t) {
  if (check_all(q, kv, t) != CASCADE_OK) return 0;
  return ws_layout(q, kv, t, plan_request(q, kv, t)).bytes;
}

cascade_status cascade_prefix_attn(const cascade_query* q, const cascade_paged_kv* kv,
                                   const cascade_tree* t, float* o_a, float* lse_a, void* ws,
                                   size_t ws_bytes, void* stream) {
  cascade_status st = check_all(q, kv, t);
  if (st != CASCADE_OK) return st;
  if (q->total_rows > 0 && (!o_a || !lse_a)) return fail(CASCADE_ERR_NULL, "o_a and lse_a are required");
  if (o_a && !aligned16(o_a)) return fail(CASCADE_ERR_UNSUPPORTED, "o_a must be 16-byte aligned");
  const Plan p = plan_request(q, kv, t);
  const WsLayout wl = ws_layout(q, kv, t, p);
  if (wl.required > 0 && (!ws || ws_bytes < wl.required))
    return fail(CASCADE_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", wl.required, ws ? ws_bytes : 0);
  if (ws && !aligned16(ws)) return fail(CASCADE_ERR_UNSUPPORTED, "workspace must be 16-byte aligned");
  if ((st = check_plan_grid(t, kv, p)) != CASCADE_OK) return st;
  if (q->total_rows == 0 || t->batch_size == 0) return CASCADE_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  casc::AttnArgs a = make_args(q, kv, t, p);
  attach_work_list(a, wl, ws, ws_bytes);
  a.o = o_a;
  a.o_bf16 = 0;
  a.lse = lse_a;
  hipError_t e;
  if (p.n_splits > 1) {
    a.ws_o = static_cast<float*>(ws);
    a.ws_lse = reinterpret_cast<float*>(static_cast<char*>(ws) + wl.lse_off);
    a.grid_splits = p.n_splits;
    e = launch_row_modes(casc::kModePrefix, kv, t, p, a, p.n_splits, s);
    if (e != hipSuccess) return hip_fail(e, "prefix pass launch");
    e = casc::launch_split_merge(split_merge_args(q, kv, t, p, a, false), s, nullptr);
    if (e != hipSuccess) return hip_fail(e, "prefix split merge launch");
  } else {
    e = launch_row_modes(casc::kModePrefix, kv, t, p, a, 1, s);
    if (e != hipSuccess) return hip_fail(e, "prefix pass launch");
  }
  return CASCADE_OK;
}

cascade_status cascade_draft_attn(const cascade_query* q, const cascade_paged_kv* kv,
                                  const cascade_tree* t, float* o_b, float* lse_b, void* stream) {
  cascade_status st = check_all(q, kv, t);
  if (st != CASCADE_OK) return st;
  if (q->total_rows > 0 && (!o_b || !lse_b)) return fail(CASCADE_ERR_NULL, "o_b and lse_b are required");
  if (o_b && !aligned16(o_b)) return fail(CASCADE_ERR_UNSUPPORTED, "o_b must be 16-byte aligned");
  Plan p = plan_request(q, kv, t);
  p.n_splits = 1;
  if ((st = check_grid(xcd_grid((int64_t)t->batch_size * kv->num_kv_heads, p.n_chunks, 1))) != CASCADE_OK) return st;
  if (q->total_rows == 0 || t->batch_size == 0) return CASCADE_OK;
  casc::AttnArgs a = make_args(q, kv, t, p);
  a.o = o_b;
  a.o_bf16 = 0;
  a.lse = lse_b;
  const hipError_t e = launch_row_modes(casc::kModeDraft, kv, t, p, a, 1, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "draft pass launch");
  return CASCADE_OK;
}

cascade_status merge_state(const float* o_a, const float* lse_a, const float* o_b, const float* lse_b,
                           int64_t num_rows, int32_t num_heads, int32_t head_dim, void* o,
                           cascade_dtype o_dtype, float* lse, void* stream) {
  if (num_rows < 0 || num_heads < 0 || head_dim <= 0) return fail(CASCADE_ERR_SHAPE, "bad merge shape");
  if (head_dim % 4) return fail(CASCADE_ERR_UNSUPPORTED, "head_dim must be a multiple of 4");
  if (o_dtype != CASCADE_F32 && o_dtype != CASCADE_BF16) return fail(CASCADE_ERR_UNSUPPORTED, "bad o_dtype");
  if (num_rows == 0 || num_heads == 0) return CASCADE_OK;
  if (!o_a || !lse_a || !o_b || !lse_b || !o) return fail(CASCADE_ERR_NULL, "merge_state input or output is NULL");
  if (!aligned16(o_a) || !aligned16(o_b) || !aligned16(o))
    return fail(CASCADE_ERR_UNSUPPORTED, "o_a, o_b and o must be 16-byte aligned");
  casc::MergeArgs a{};
  a.o_a = o_a;
  a.lse_a = lse_a;
  a.o_b = o_b;
  a.lse_b = lse_b;
  a.rows = num_rows * num_heads;
  a.head_dim = head_dim;
  a.o = o;
  a.o_bf16 = o_dtype == CASCADE_BF16;
  a.lse = lse;
  const hipError_t e = casc::launch_merge(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "merge_state launch");
  return CASCADE_OK;
}

static cascade_status verify_impl(const cascade_query* q, const cascade_paged_kv* kv,
                                   const cascade_tree* t, void* o, cascade_dtype o_dtype, float* lse,
                                   void* ws, size_t ws_bytes, void* stream) {
  cascade_status st = check_all(q, kv, t);
  if (st != CASCADE_OK) return st;
  if (o_dtype != CASCADE_F32 && o_dtype != CASCADE_BF16) return fail(CASCADE_ERR_UNSUPPORTED, "bad o_dtype");
  if (q->total_rows > 0 && !o) return fail(CASCADE_ERR_NULL, "o is NULL");
  if (o && !aligned16(o)) return fail(CASCADE_ERR_UNSUPPORTED, "o must be 16-byte aligned");
  const Plan p = plan_request(q, kv, t);
  const WsLayout wl = ws_layout(q, kv, t, p);
  if (wl.required > 0 && (!ws || ws_bytes < wl.required))
    return fail(CASCADE_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", wl.required, ws ? ws_bytes : 0);
  if (ws && !aligned16(ws)) return fail(CASCADE_ERR_UNSUPPORTED, "workspace must be 16-byte aligned");
  if ((st = check_plan_grid(t, kv, p)) != CASCADE_OK) return st;
  if (q->total_rows == 0 || t->batch_size == 0) return CASCADE_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  casc::AttnArgs a = make_args(q, kv, t, p);
  attach_work_list(a, wl, ws, ws_bytes);
  a.o = o;
  a.o_bf16 = o_dtype == CASCADE_BF16;
  a.lse = lse;
  hipError_t e;
  hipEvent_t e0 = g_timing.enabled ? g_timing.start : nullptr;
  hipEvent_t e1 = g_timing.enabled ? g_timing.stop : nullptr;
  if (p.n_splits > 1) {
    a.ws_o = static_cast<float*>(ws);
    a.ws_lse = reinterpret_cast<float*>(static_cast<char*>(ws) + wl.lse_off);
    a.grid_splits = p.n_splits;
    e = launch_row_modes(casc::kModeVerify, kv, t, p, a, p.n_splits, s, e0, nullptr);
    if (e != hipSuccess) return hip_fail(e, "verify prefix launch");
    e = casc::launch_split_merge(split_merge_args(q, kv, t, p, a, true), s, e1);
    if (e != hipSuccess) return hip_fail(e, "verify merge launch");
  } else {
    e = launch_row_modes(casc::kModeVerify, kv, t, p, a, 1, s, e0, e1);
    if (e != hipSuccess) return hip_fail(e, "verify launch");
  }
  if (g_timing.enabled) g_timing.recorded = true;
  return CASCADE_OK;
}

cascade_status cascade_verify_attn(const cascade_query* q, const cascade_paged_kv* kv,
                                   const cascade_tree* t, void* o, cascade_dtype o_dtype, float* lse,
                                   void* ws, size_t ws_bytes, void* stream) {
  return verify_impl(q, kv, t, o, o_dtype, lse, ws, ws_bytes, stream);
}

cascade_status cascade_verify_attn_noalloc(const cascade_query* q, const cascade_paged_kv* kv,
                                           const cascade_tree* t, void* o, cascade_dtype o_dtype,
                                           float* lse, void* stream) {
  cascade_status st = check_all(q, kv, t);
  if (st != CASCADE_OK) return st;
  const size_t need = ws_layout(q, kv, t, plan_request(q, kv, t)).bytes;
  if (need > casc::kScratchBytes)
    return fail(CASCADE_ERR_WORKSPACE,
                "these shapes need %zu bytes of workspace; the built-in workspace holds %zu "
                "(use cascade_verify_attn with a caller workspace)",
                need, casc::kScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = casc::scratch_for_current_device(&ws);
    if (e != hipSuccess) return hip_fail(e, "built-in workspace address");
  }
  return verify_impl(q, kv, t, o, o_dtype, lse, ws, need > 0 ? casc::kScratchBytes : 0, stream);
}

cascade_status naive_expand(const cascade_query* q, const cascade_paged_kv* kv, const cascade_tree* t,
                            void* o, cascade_dtype o_dtype, float* lse, void* stream) {
  cascade_status st = check_all(q, kv, t);
  if (st != CASCADE_OK) return st;
  if (o_dtype != CASCADE_F32 && o_dtype != CASCADE_BF16) return fail(CASCADE_ERR_UNSUPPORTED, "bad o_dtype");
  if (q->total_rows > 0 && !o) return fail(CASCADE_ERR_NULL, "o is NULL");
  if (o && !aligned16(o)) return fail(CASCADE_ERR_UNSUPPORTED, "o must be 16-byte aligned");
  Plan p;
  p.group = q->num_qo_heads / kv->num_kv_heads;
  plan_rows(p, (int64_t)t->max_draft_len * p.group);
  p.items = (int64_t)t->num_branches * kv->num_kv_heads * p.n_chunks;
  p.n_splits = 1;
  p.split_len = 32;
  if ((st = check_grid(xcd_grid((int64_t)t->num_branches * kv->num_kv_heads, p.n_chunks, 1))) != CASCADE_OK) return st;
  if (q->total_rows == 0 || t->num_branches == 0) return CASCADE_OK;
  casc::AttnArgs a = make_args(q, kv, t, p);
  a.o = o;
  a.o_bf16 = o_dtype == CASCADE_BF16;
  a.lse = lse;
  const hipError_t e = launch(casc::kModeNaive, kv->head_dim, p.rb, a, (int64_t)t->num_branches * kv->num_kv_heads,
                              1, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "naive expand launch");
  return CASCADE_OK;
}

cascade_status cascade_debug_gather(const cascade_paged_kv* kv, const cascade_tree* t, int32_t which,
                                    int32_t index, int32_t kv_head, void* k_out, void* v_out, void* stream) {
  cascade_status st = check_kv(kv);
  if (st != CASCADE_OK) return st;
  if (!t) return fail(CASCADE_ERR_NULL, "tree is NULL");
  if (which != 0 && which != 1) return fail(CASCADE_ERR_SHAPE, "which must be 0 (prefix) or 1 (draft)");
  if (kv_head < 0 || kv_head >= kv->num_kv_heads) return fail(CASCADE_ERR_SHAPE, "kv_head out of range");
  if (which == 0 && (index < 0 || index >= t->batch_size)) return fail(CASCADE_ERR_SHAPE, "request out of range");
  if (which == 1 && (index < 0 || index >= t->num_branches)) return fail(CASCADE_ERR_SHAPE, "branch out of range");
  if (which == 0 && (!t->page_table || !t->cache_seqlens)) return fail(CASCADE_ERR_NULL, "page_table is NULL");
  if (which == 1 && (!t->draft_page_table || !t->branch_qo_indptr)) return fail(CASCADE_ERR_NULL, "draft tables are NULL");
  if (!k_out || !v_out) return fail(CASCADE_ERR_NULL, "k_out / v_out is NULL");
  if (!aligned16(k_out) || !aligned16(v_out)) return fail(CASCADE_ERR_UNSUPPORTED, "outputs must be 16-byte aligned");
  // The token count lives on the device: fetch it (this hook synchronises).
  int32_t count = 0;
  hipError_t e;
  if (which == 0) {
    e = hipMemcpy(&count, t->cache_seqlens + index, sizeof(int32_t), hipMemcpyDeviceToHost);
  } else {
    int32_t ends[2];
    e = hipMemcpy(ends, t->branch_qo_indptr + index, 2 * sizeof(int32_t), hipMemcpyDeviceToHost);
    count = ends[1] - ends[0];
  }
  if (e != hipSuccess) return hip_fail(e, "reading sequence length");
  if (count < 0) return fail(CASCADE_ERR_SHAPE, "negative sequence length");
  casc::DebugArgs a{};
  a.kv = kv_view(kv);
  a.head_dim = kv->head_dim;
  a.num_kv_heads = kv->num_kv_heads;
  a.batch_size = t->batch_size;
  a.page_table = t->page_table;
  a.page_table_stride = t->page_table_stride;
  a.cache_seqlens = t->cache_seqlens;
  a.req_branch_indptr = t->req_branch_indptr;
  a.branch_qo_indptr = t->branch_qo_indptr;
  a.draft_page_table = t->draft_page_table;
  a.draft_page_table_stride = t->draft_page_table_stride;
  a.draft_start = t->draft_start;
  a.draft_mask = t->draft_mask;
  a.draft_mask_words = mask_words(t);
  a.which = which;
  a.index = index;
  a.kv_head = kv_head;
  a.count = count;
  a.k_out = static_cast<uint16_t*>(k_out);
  a.v_out = static_cast<uint16_t*>(v_out);
  e = casc::launch_debug_gather(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "debug gather launch");
  return CASCADE_OK;
}

cascade_status cascade_debug_mask(const cascade_tree* t, int32_t branch, uint8_t* mask_out,
                                  int32_t mask_cols, void* stream) {
  if (!t) return fail(CASCADE_ERR_NULL, "tree is NULL");
  if (branch < 0 || branch >= t->num_branches) return fail(CASCADE_ERR_SHAPE, "branch out of range");
  if (!t->cache_seqlens || !t->req_branch_indptr || !t->branch_qo_indptr)
    return fail(CASCADE_ERR_NULL, "tree arrays are NULL");
  if (!mask_out) return fail(CASCADE_ERR_NULL, "mask_out is NULL");
  if (mask_cols < 0) return fail(CASCADE_ERR_SHAPE, "mask_cols must be >= 0");
  if (t->draft_mask && (reinterpret_cast<uintptr_t>(t->draft_mask) & 7u))
    return fail(CASCADE_ERR_UNSUPPORTED, "draft_mask must be 8-byte aligned");
  if (t->draft_mask && (t->draft_mask_words < 0 || mask_words(t) > kMaxMaskWords))
    return fail(CASCADE_ERR_UNSUPPORTED, "draft_mask_words %d not supported (0 .. %d)", (int)t->draft_mask_words,
                kMaxMaskWords);
  int32_t ends[2];
  hipError_t e = hipMemcpy(ends, t->branch_qo_indptr + branch, 2 * sizeof(int32_t), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "reading branch length");
  casc::DebugArgs a{};
  a.batch_size = t->batch_size;
  a.cache_seqlens = t->cache_seqlens;
  a.req_branch_indptr = t->req_branch_indptr;
  a.branch_qo_indptr = t->branch_qo_indptr;
  a.draft_mask = t->draft_mask;
  a.draft_mask_words = mask_words(t);
  a.index = branch;
  a.count = ends[1] - ends[0];
  a.cols = mask_cols;
  a.mask_out = mask_out;
  e = casc::launch_debug_mask(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "debug mask launch");
  return CASCADE_OK;
}

cascade_status cascade_device_error(int32_t* flag_out, int32_t clear) {
  if (!flag_out) return fail(CASCADE_ERR_NULL, "flag_out is NULL");
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_fail(e, "synchronise");
  int flags = 0;
  hipError_t (*const readers[])(int*, int) = {casc::read_error_d64, casc::read_error_d128,
                                              casc::read_error_d64_fp8, casc::read_error_d128_fp8,
                                              casc::read_error_small, casc::read_error_pair_d128,
                                              casc::read_error_pair_d128_fp8};
  for (auto* rd : readers) {
    int v = 0;
    if ((e = rd(&v, clear)) != hipSuccess) return hip_fail(e, "read error word");
    flags |= v;
  }
  *flag_out = flags;
  return CASCADE_OK;
}

cascade_status cascade_append_draft_kv(const cascade_paged_kv* kv, const cascade_tree* t, int32_t total_rows,
                                       const void* k_new, const void* v_new, int64_t new_row_stride,
                                       int64_t new_head_stride, void* stream) {
  cascade_status st = check_kv(kv);
  if (st != CASCADE_OK) return st;
  if ((st = check_tree(t, kv)) != CASCADE_OK) return st;
  if (total_rows < 0) return fail(CASCADE_ERR_SHAPE, "total_rows must be >= 0");
  if (total_rows == 0) return CASCADE_OK;
  if (t->num_branches <= 0) return fail(CASCADE_ERR_SHAPE, "rows without branches");
  if (!k_new || !v_new) return fail(CASCADE_ERR_NULL, "k_new / v_new is NULL");
  if (!aligned16(k_new) || !aligned16(v_new)) return fail(CASCADE_ERR_UNSUPPORTED, "k_new / v_new must be 16-byte aligned");
  if (new_row_stride % 8 || new_head_stride % 8 || new_row_stride < 0 || new_head_stride < 0)
    return fail(CASCADE_ERR_UNSUPPORTED, "k_new / v_new strides must be non-negative multiples of 8 elements");
  casc::AppendArgs a{};
  a.kv = kv_view(kv);
  a.head_dim = kv->head_dim;
  a.num_kv_heads = kv->num_kv_heads;
  a.total_rows = total_rows;
  a.num_branches = t->num_branches;
  a.branch_qo_indptr = t->branch_qo_indptr;
  a.draft_page_table = t->draft_page_table;
  a.draft_page_table_stride = t->draft_page_table_stride;
  a.draft_start = t->draft_start;
  a.k_new = k_new;
  a.v_new = v_new;
  a.new_row_stride = new_row_stride;
  a.new_head_stride = new_head_stride;
  const hipError_t e = casc::launch_append_kv(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "append launch");
  return CASCADE_OK;
}

cascade_status cascade_commit_accepted(const cascade_paged_kv* kv, const cascade_tree* t, int32_t total_rows,
                                       const int32_t* accepted_indptr, const int32_t* accepted_rows,
                                       int32_t max_accepted, int32_t* cache_seqlens_out, void* stream) {
  cascade_status st = check_kv(kv);
  if (st != CASCADE_OK) return st;
  if ((st = check_tree(t, kv)) != CASCADE_OK) return st;
  if (total_rows < 0 || max_accepted < 0) return fail(CASCADE_ERR_SHAPE, "total_rows / max_accepted must be >= 0");
  if (t->batch_size == 0) return CASCADE_OK;
  if (!accepted_indptr || !cache_seqlens_out) return fail(CASCADE_ERR_NULL, "accepted_indptr / cache_seqlens_out is NULL");
  if (max_accepted > 0 && !accepted_rows) return fail(CASCADE_ERR_NULL, "accepted_rows is NULL");
  if (max_accepted > 0 && !t->page_table) return fail(CASCADE_ERR_NULL, "page_table is NULL");
  if ((int64_t)t->batch_size * max_accepted * kv->num_kv_heads * 16 > (int64_t)INT32_MAX * 256)
    return fail(CASCADE_ERR_SHAPE, "commit too large");
  casc::CommitArgs a{};
  a.kv = kv_view(kv);
  a.head_dim = kv->head_dim;
  a.num_kv_heads = kv->num_kv_heads;
  a.batch_size = t->batch_size;
  a.num_branches = t->num_branches;
  a.total_rows = total_rows;
  a.max_accepted = max_accepted;
  a.page_table = t->page_table;
  a.page_table_stride = t->page_table_stride;
  a.cache_seqlens = t->cache_seqlens;
  a.cache_seqlens_out = cache_seqlens_out;
  a.branch_qo_indptr = t->branch_qo_indptr;
  a.draft_page_table = t->draft_page_table;
  a.draft_page_table_stride = t->draft_page_table_stride;
  a.draft_start = t->draft_start;
  a.accepted_indptr = accepted_indptr;
  a.accepted_rows = accepted_rows;
  const hipError_t e = casc::launch_commit(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "commit launch");
  return CASCADE_OK;
}

cascade_status cascade_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (bytes == 0) return CASCADE_OK;
  if (!buf || !sink) return fail(CASCADE_ERR_NULL, "buf / sink is NULL");
  if (!aligned16(buf) || bytes % 16) return fail(CASCADE_ERR_UNSUPPORTED, "buf must be 16-byte aligned, bytes a multiple of 16");
  const hipError_t e = casc::launch_stream_read(buf, bytes, sink, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "stream read launch");
  return CASCADE_OK;
}

cascade_status cascade_kernel_timing(int32_t enable) {
  if (enable && !g_timing.start) {
    hipError_t e = hipEventCreate(&g_timing.start);
    if (e == hipSuccess) e = hipEventCreate(&g_timing.stop);
    if (e != hipSuccess) return hip_fail(e, "timing event creation");
  }
  g_timing.enabled = enable != 0;
  g_timing.recorded = false;
  return CASCADE_OK;
}

cascade_status cascade_last_verify_ms(float* ms_out) {
  if (!ms_out) return fail(CASCADE_ERR_NULL, "ms_out is NULL");
  if (!g_timing.recorded) return fail(CASCADE_ERR_SHAPE, "no timed cascade_verify_attn call");
  hipError_t e = hipEventSynchronize(g_timing.stop);
  if (e == hipSuccess) e = hipEventElapsedTime(ms_out, g_timing.start, g_timing.stop);
  if (e != hipSuccess) return hip_fail(e, "timing event query");
  return CASCADE_OK;
}

}  // extern "C"
