// Device-side helpers shared by every kernel of the library: vector types,
// the paged-KV address computation, the draft-key visibility rule, and the
// sticky bounds flag.  Built for gfx950 (CDNA4, wave64) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "args.h"

namespace casc {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
// Read-only tables (block tables, lengths) seen through the constant address
// space: uniform reads of them compile to scalar loads, which complete on
// their own counter instead of behind the vector loads of K and V.
typedef const __attribute__((address_space(4))) int32_t cint32;
__device__ __forceinline__ cint32* as_const(const int32_t* p) { return (cint32*)(uintptr_t)p; }

// Sticky error word of this translation unit (bit flags below); read and
// cleared by the host through hipMemcpyFromSymbol / hipMemcpyToSymbol.
static __device__ int g_device_error;

// Orders one wave's LDS writes before its later LDS reads from other lanes.
// A wave's LDS instructions execute in order, so this only keeps the compiler
// from moving them across the point.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// Bit flags of the sticky device error word.
constexpr int kErrPage = 1;   // a block-table entry outside [0, num_pages)
constexpr int kErrRow = 2;    // a query row outside [0, total_rows)
constexpr int kErrLen = 4;    // a sequence longer than its block-table row can hold


// Logical slot `slot` of block-table row `table_row` for kv head `g`: the page
// is table_row[slot / P] and the token sits at slot % P inside it (paged KV,
// block table mapping logical to physical pages).  Returns -1 when the page id
// lies outside the pool.
__device__ __forceinline__ int64_t paged_offset(const KvView& kv, const int32_t* table_row,
                                                int32_t slot, int32_t g) {
  const int32_t page = table_row[slot >> kv.log2_page];
  if ((uint32_t)page >= (uint32_t)kv.num_pages) return -1;
  const int32_t in_page = slot & ((1 << kv.log2_page) - 1);
  return (int64_t)page * kv.page_stride + (int64_t)in_page * kv.token_stride +
         (int64_t)g * kv.head_stride;
}

// Branch j in [jb, je) whose query rows contain global row `row`
// (branch_qo_indptr is non-decreasing).
__device__ __forceinline__ int branch_of_row(const int32_t* qo, int jb, int je, int row) {
  int lo = jb, hi = je - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (qo[mid] <= row) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Request i with req_branch_indptr[i] <= j < req_branch_indptr[i+1].
__device__ __forceinline__ int request_of_branch(const int32_t* rb, int batch, int j) {
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (rb[mid] <= j) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Draft-key visibility (tree attention restricted to chains: a node sees its
// ancestors and itself).  Tokens are numbered within one row segment; a query
// at token t whose branch starts at token bs sees draft key token kt iff kt
// lies in its own branch at or before it.
__device__ __forceinline__ bool draft_visible(int t, int bs, int kt) {
  return (kt >= bs) & (kt <= t);  // bitwise: a select, not a branch, per key
}
// The same for a general draft tree (tree attention mask): the row's ancestor
// set `anc` over its branch's nodes (bit u: node u, i.e. token bs + u).
__device__ __forceinline__ bool draft_visible_tree(uint64_t anc, int bs, int kt) {
  const int u = kt - bs;
  return (u >= 0) & (u < 64) & (((anc >> (u & 63)) & 1ull) != 0ull);
}
// Trees of more than 64 nodes keep a row's ancestor set in `words` 64-bit
// words (bit u % 64 of word u / 64: node u).  A tile of keys from token
// `base` on sees the 64-node window of the set that starts at node
// ws = max(base - bs, 0): tree_window returns it (bit v: node ws + v, zeros
// past the last word), and draft_visible_tree(window, bs + ws, kt) decides
// every key kt of the tile.  tree_window1: the same for a one-word set held
// in a register.
__device__ __forceinline__ uint64_t tree_window(const uint64_t* row_mask, int words, int ws) {
  const int i = ws >> 6, sh = ws & 63;
  const uint64_t lo = i < words ? row_mask[i] : 0ull;
  const uint64_t hi = i + 1 < words ? row_mask[i + 1] : 0ull;
  return (lo >> sh) | ((hi << 1) << (63 - sh));
}
__device__ __forceinline__ uint64_t tree_window1(uint64_t anc, int ws) { return ws < 64 ? anc >> ws : 0ull; }

// Element offset (kv head excluded) of logical slot `slot` of draft
// block-table row `row` (`stride` entries), or -1 when the slot lies outside
// the row or its page id outside the pool.  The draft-key tables of the
// attention kernels, the draft gather hook and the serving-step writes all
// resolve draft slots through this function.
__device__ __forceinline__ int64_t draft_slot_offset(const KvView& kv, const int32_t* row, int32_t stride,
                                                     int32_t slot) {
  if (slot < 0 || (slot >> kv.log2_page) >= stride) return -1;
  const int32_t page = row[slot >> kv.log2_page];
  if ((uint32_t)page >= (uint32_t)kv.num_pages) return -1;
  return (int64_t)page * kv.page_stride + (int64_t)(slot & ((1 << kv.log2_page) - 1)) * kv.token_stride;
}

// Physical offset of draft token `kt` (numbered from the first row of branch
// jb) of kv head g.  Branch j's token u is at logical slot draft_start[j] + u
// of draft block-table row j (dstride entries).  -1 when the slot lies past
// the row or the page id is outside the pool.
__device__ __forceinline__ int64_t draft_offset(const KvView& kv, const int32_t* qo,
                                                const int32_t* dpt, int32_t dstride,
                                                const int32_t* dstart, int jb, int je,
                                                int kt, int g) {
  const int row = qo[jb] + kt;
  const int j = branch_of_row(qo, jb, je, row);
  const int u = row - qo[j];
  const int slot = (dstart ? dstart[j] : 0) + u;
  const int64_t off = draft_slot_offset(kv, dpt + (int64_t)j * dstride, dstride, slot);
  return off < 0 ? -1 : off + (int64_t)g * kv.head_stride;
}

// Largest element offset at which a whole key row of one kv head starts
// inside the pool.  A draft-key load clamps its offset to [0, this], so even
// an offset read from a table entry that was never written stays inside the
// pool (it reads a wrong row, never an unmapped address).
__device__ __forceinline__ int64_t pool_last_row(const KvView& kv, int num_kv_heads) {
  return (int64_t)(kv.num_pages - 1) * kv.page_stride + (int64_t)((1 << kv.log2_page) - 1) * kv.token_stride +
         (int64_t)(num_kv_heads - 1) * kv.head_stride;
}
__device__ __forceinline__ int64_t clamp_row(int64_t off, int64_t last) {
  return off < 0 ? 0 : (off > last ? last : off);
}

// Buffer descriptor over a byte range (gfx9-family raw buffer: stride 0,
// dword 3 = 0x00020000).  A lane whose 16-byte read does not lie inside
// `bytes` reads zeros, so a partially valid tile needs neither branches nor
// selects.
constexpr int kBufFlags = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kBufFlags);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}
__device__ __forceinline__ u32x2 buf_load8(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, 0));
}

// Prefix tiles start at multiples of 32 slots and pages hold >= 16 tokens,
// so each 16-key half of a tile lies in one page.  The half's buffer
// descriptor starts at its first key's row (slot `first` of page `page`) and
// ends after the row of its last valid key (`nvalid` keys), kv head and head
// dim included (`tail_bytes` = bytes from a key row's start to the end of the
// kv head's elements), so lanes addressing keys past the end -- and every key
// of a half whose page id is -1 (none, or outside the pool) -- read zeros.
// K and V pools share their strides, so one span serves both descriptors.
// The attention kernels and the prefix gather hook build their prefix loads
// from prefix_half_span, half_rsrc and prefix_lane_offset.
struct HalfSpan {
  uint64_t off;  // byte offset of the half's first key row in a pool
  int bytes;     // descriptor range
};
__device__ __forceinline__ HalfSpan prefix_half_span(const KvView& kv, int page, int first, int nvalid,
                                                     int tail_bytes) {
  const bool ok = page >= 0 && nvalid > 0;
  const uint32_t slot = (uint32_t)(first & ((1 << kv.log2_page) - 1));
  const uint64_t off = ok ? (uint64_t)(uint32_t)page * kv.page_stride_b + (uint64_t)slot * kv.token_stride_b : 0;
  // Every input is wave-uniform (a tile's keys are the same for all lanes);
  // stating it keeps the descriptor in scalar registers -- a descriptor the
  // compiler takes for divergent costs a loop over lanes around every load.
  HalfSpan h;
  h.off = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(off >> 32)) << 32) |
          (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)off);
  h.bytes = __builtin_amdgcn_readfirstlane(ok ? (nvalid - 1) * (int)kv.token_stride_b + tail_bytes : 0);
  return h;
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t half_rsrc(const void* pool, const HalfSpan& h) {
  return page_rsrc(static_cast<const unsigned char*>(pool) + h.off, h.bytes);
}

// Byte offset, inside its half's descriptor, of 8-channel chunk `chunk` of
// the key `key` places after the half's first key.
template <int EB>
__device__ __forceinline__ int prefix_lane_offset(const KvView& kv, int key, int64_t head_off, int chunk) {
  return (int)(((int64_t)key * kv.token_stride + head_off + chunk * 8) * EB);
}
// A block-table entry as a page id: -1 for ids outside [0, num_pages).
__device__ __forceinline__ int checked_page(int id, int num_pages) {
  return (uint32_t)id < (uint32_t)num_pages ? id : -1;
}

// Eight consecutive K or V channels as they sit in the pool: eight bf16
// values (16 bytes), or eight FP8 E4M3 codes (8 bytes; KV-cache page,
// section 4.5 -- FP8 KV with a per-tensor scale).
template <bool KV8> struct KvChunk { typedef u32x4 T; };
template <> struct KvChunk<true> { typedef u32x2 T; };

__device__ __forceinline__ u32x4 buf_load_chunk(__amdgpu_buffer_rsrc_t r, int byte_off, u32x4*) {
  return buf_load16(r, byte_off);
}
__device__ __forceinline__ u32x2 buf_load_chunk(__amdgpu_buffer_rsrc_t r, int byte_off, u32x2*) {
  return buf_load8(r, byte_off);
}

// One chunk of eight channels at element offset `elem_off` of a pool (the
// draft-key loads, whose keys resolve their rows one by one; the offset is
// clamped into the pool by the caller).
template <typename Raw, int EB>
__device__ __forceinline__ Raw load_key_chunk(const void* pool, int64_t elem_off) {
  return *reinterpret_cast<const Raw*>(static_cast<const unsigned char*>(pool) + elem_off * EB);
}

// The eight channels as bf16.  E4M3 (1 sign, 4 exponent bits with bias 7,
// 3 mantissa bits; no infinities) embeds exactly in bf16, so the widening
// conversion (scale 1) rounds nothing; the per-tensor scales are applied in
// fp32 outside (the K scale with the softmax scale, the V scale on the
// normalised output).  Byte b of the chunk becomes element b.
__device__ __forceinline__ u32x4 widen_bf16(u32x4 x) { return x; }
__device__ __forceinline__ u32x4 widen_bf16(u32x2 x) {
  u32x4 r;
  r[0] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[0], 1.0f, false));
  r[1] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[0], 1.0f, true));
  r[2] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[1], 1.0f, false));
  r[3] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[1], 1.0f, true));
  return r;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Round-to-nearest-even float -> bf16 bits.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Two floats to two bf16 (RNE) in one register, lo in the low half: one
// v_cvt_pk_bf16_f32 with both operands.
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
__device__ __forceinline__ unsigned int pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(unsigned int, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// FP8 pools with per-channel K scales: q . (k * s) = (q * s) . k, so the
// eight bf16 query channels of a 16-byte chunk are multiplied by their
// channel scales (cs: 8 floats, 16-byte aligned) and rounded back to bf16
// (nearest even) as they are loaded.
__device__ __forceinline__ u32x4 scale_q_chunk(u32x4 q, const float* cs) {
  const f32x4 s0 = *reinterpret_cast<const f32x4*>(cs);
  const f32x4 s1 = *reinterpret_cast<const f32x4*>(cs + 4);
  const float s[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = __builtin_bit_cast(float, q[i] << 16);
    const float hi = __builtin_bit_cast(float, q[i] & 0xffff0000u);
    r[i] = pack_bf16x2(lo * s[2 * i], hi * s[2 * i + 1]);
  }
  return r;
}

}  // namespace casc
