// Row-split attention kernel for row-heavy launches (pass A, pass B and the
// fused verify pass), head_dim 128, bf16 or FP8 E4M3 pools (KV8: 8-byte code
// chunks per load, widened to bf16 when staged; the K scale is in the
// softmax scale, the V scale is applied to the normalised output).
//
// One workgroup of kRowWaves = 4 waves (one per SIMD; two workgroups share a
// CU, so every SIMD runs two waves of independent workgroups) handles one
// work item
//   (request, kv head g, chunk of at most kRowsPerItem query rows, key split).
// The chunk's rows -- the request's query tokens times the query heads that
// share kv head g -- are dealt out to the waves, at most 16 * RBW per wave
// (RBW MFMA row blocks sharing every K and V fragment the wave reads), so
// every wave keeps its own rows' complete online softmax state and no state
// is merged across waves.  The waves of a workgroup go through the same
// 32-key tiles in lock step:
//   * bf16 pools: the tiles are copied from HBM straight into LDS (buffer
//     loads into LDS, 16 bytes a lane; the 64 lanes of a wave fill four whole
//     256-byte key rows of one page per copy) into NS stages, NS - 1 tiles
//     ahead; per step each wave waits for its own copies of the current tile,
//     the workgroup meets at one barrier, the stage the previous tile left
//     gets the tile NS - 1 ahead, and the current tile is computed.  No
//     register holds a tile in flight;
//   * FP8 pools: each thread loads its 8-byte code chunks DEPTH tiles ahead
//     into a ring of registers, and per step widens the next tile into one of
//     two LDS stages while the current one is computed out of the other;
//   * a wave reads K back as MFMA A-fragments (S^T = K Q^T with
//     v_mfma_f32_16x16x32_bf16, its rows' Q as B-fragments in registers),
//     updates its rows' base-2 online softmax, and reads V back transposed
//     (ds_read_b64_tr_b16) for O^T += V^T P^T; P^T stays in the lanes that
//     computed S^T.
// In the fused verify launch the request's draft keys (pass B, under the
// in-branch ancestor mask) follow the prefix tiles as further steps of the
// same online softmax, so passes A and B meet in one state: the merge of the
// two passes is the online softmax itself (cascade page, splittability: the
// same LSE identity).  A request with one branch whose slots lie in its
// draft-page row streams them through the same ring loop, in pass B and in
// the fused launch; other requests reach their draft keys through per-key
// offset tables.
#pragma once

#include "attn_kernel.h"

namespace casc {

// A 16-byte-per-lane copy global -> LDS: lane i's 16 bytes at `voff` in the
// buffer land at LDS byte `lds` + 16 i.  Written out so that the compiler
// does not order every later LDS read behind every copy in flight (it cannot
// tell the stages apart); the key loop waits for the copies itself.  No
// register is written.
__device__ __forceinline__ void lds_copy16(__amdgpu_buffer_rsrc_t r, uint32_t lds, int voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(lds), "v"(voff), "s"(r)
               : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const uint16_t* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint16_t*)p;
}

// Mask kind of a key range, as a type for the key loop.
template <int K>
struct KeyKind {
  static constexpr int value = K;
};

// NS: LDS stages of the bf16 copies (NS - 1 tiles in flight).  NS = 4: two
// workgroups per CU (64 KB of stages each).  NS = 3: three workgroups per CU
// -- 48 KB of stages, a 256-key draft table and at most 168 VGPRs (a few
// values spill), so that every SIMD runs three waves: for launches with many
// full 128-row items (a prefix-hit suffix prefill: 10-12 % faster), while
// batches of short HBM-bound items keep the deeper copy pipeline.  FP8 pools
// run the register ring at two workgroups per CU.
template <int MODE, int DEPTH, int RBW, bool KV8, int NS>
__global__ void __launch_bounds__(64 * kRowWaves) __attribute__((amdgpu_waves_per_eu(NS == 3 ? 3 : 2, NS == 3 ? 3 : 2)))
rows_kernel(const AttnArgs a) {
  static_assert(MODE == kModePrefix || MODE == kModeVerify || MODE == kModeDraft, "pass A, verify, pass B");
  static_assert(DEPTH % 2 == 0, "the two LDS stages of the register ring alternate within the unrolled ring");
  static_assert(kRowsPerItem == kRowWaves * 16 * RBW, "RBW 16-row blocks per wave");
  constexpr int ROWS_W = 16 * RBW;  // query rows per wave
  constexpr int D = 128;
  constexpr int KS = D / 32;   // k-steps of the Q K^T contraction
  constexpr int DB = D / 16;   // 16-channel blocks of the head dim
  constexpr int CPR = D / 8;   // 8-channel chunks per key row (16)
  // Stage layout: the K tile's 32 rows, then the V tile's, 256 bytes each
  // with no padding.  The 16-byte chunks of a row are XOR-swizzled by the
  // key -- K: chunk c of key k at slot c ^ (k & 15); V: at slot c ^ 2(k & 3) --
  // so that a K-fragment read (one chunk of 16 keys) and a transposed V read
  // (two chunks of 4 keys) each touch every bank once.
  constexpr int ROWE = D;             // bf16 elements per LDS row
  constexpr int STAGE = 64 * ROWE;    // bf16 elements of one stage: K tile, then V tile
  // bf16 pools are copied global -> LDS directly (buffer loads into LDS):
  // NS stages, NS - 1 tiles in flight.  FP8 codes are widened in registers
  // on the way (two stages, a register ring of DEPTH tiles).
  constexpr bool kDma = !KV8;
  static_assert(NS == 3 || NS == 4, "three or four copy stages");
  static_assert(!KV8 || NS == 4, "FP8 pools run the register ring");
  // Bytes per pool element; a chunk of 8 channels as loaded (16 bytes of
  // bf16, or 8 bytes of FP8 E4M3 codes widened to bf16 when staged).
  constexpr int EB = KV8 ? 1 : 2;
  typedef typename KvChunk<KV8>::T Raw;
  // The workgroup's NT threads cover a tile's 32 keys x 16 chunks of K (and
  // of V); thread tid holds chunks tid + q*NT, q < CPT.
  constexpr int NT = 64 * kRowWaves;
  constexpr int CPT = 512 / NT;
  static_assert(CPT * NT == 512, "whole tiles per workgroup");
  struct Tile {
    Raw k[CPT], v[CPT];
  };
  struct Pages {
    int p[CPT];
  };
  constexpr bool kVerify = MODE == kModeVerify;
  constexpr bool kDraft = MODE == kModeDraft;
  constexpr bool kTables = kVerify || kDraft;
  constexpr int NBCAP = 128;   // branches of a request resolved in LDS
  constexpr int KEYCAP = NS == 3 ? 256 : 512;  // draft keys of a chunk resolved in LDS

  // One LDS object per stage, so that the compiler can tell the stages apart
  // when it orders reads of one stage against copies into another.
  __shared__ __attribute__((aligned(16))) uint16_t stg0[STAGE];
  __shared__ __attribute__((aligned(16))) uint16_t stg1[STAGE];
  __shared__ __attribute__((aligned(16))) uint16_t stg2[kDma ? STAGE : 8];
  __shared__ __attribute__((aligned(16))) uint16_t stg3[kDma && NS > 3 ? STAGE : 8];
  uint16_t* const stg[4] = {stg0, stg1, stg2, stg3};
  __shared__ int64_t t_doff[kTables ? KEYCAP : 1];
  __shared__ int t_bnd[kTables ? NBCAP + 1 : 1];
  __shared__ int t_dst[kTables ? NBCAP : 1];
  __shared__ int t_rbs[kTables ? kRowsPerItem : 1];

  const int tid = (int)threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;
  const int g4 = lane >> 4;

  // ---- work item: key splits slowest; within a split, workgroup u goes to
  // XCD u % 8 (round-robin dispatch) and u / 8 walks the row chunks of one
  // (request, kv head) pair, then the next pair of that XCD.  The chunks of a
  // pair then run side by side on one L2 and stream the same key tiles at
  // about the same time, so the tiles come from HBM once per XCD, not once
  // per chunk.
  // With a work list (launches that have a workspace), workgroup u takes
  // entry u / Hkv for kv head u % Hkv instead: the items come longest first
  // and none is empty, and with 8 kv heads XCD x takes kv head x of every
  // entry, so the XCDs get the same work in the same order.
  int split, chunk, g, req;
  if (a.work_list) {
    const int u = (int)blockIdx.x;
    const int e = u / a.num_kv_heads;
    if (e >= *as_const(a.work_count)) return;
    g = u - e * a.num_kv_heads;
    const int c = as_const(a.work_list)[e];
    chunk = c % a.n_chunks;
    const int rs = c / a.n_chunks;
    split = rs % a.n_splits;
    req = rs / a.n_splits;
  } else {
    const int per_split = (int)gridDim.x / a.grid_splits;
    split = (int)blockIdx.x / per_split;
    const int u = (int)blockIdx.x - split * per_split;
    const int v8 = u >> 3;
    // Pass B is causal: a chunk's keys end at its last token, so later chunks
    // are longer (in pass B and in the fused verify).  They are handed out
    // longest first, so that the short ones fill in behind them instead of
    // the long ones forming the launch's tail.
    chunk = (kDraft || kVerify) ? a.n_chunks - 1 - v8 % a.n_chunks : v8 % a.n_chunks;
    const int item = (v8 / a.n_chunks) * 8 + (u & 7);
    if (item >= a.n_seg_items) return;
    g = item % a.num_kv_heads;
    req = item / a.num_kv_heads;
  }
  split = __builtin_amdgcn_readfirstlane(split);
  chunk = __builtin_amdgcn_readfirstlane(chunk);
  g = __builtin_amdgcn_readfirstlane(g);
  req = __builtin_amdgcn_readfirstlane(req);
  cint32* crb = as_const(a.req_branch_indptr);
  cint32* cqo = as_const(a.branch_qo_indptr);
  const int jb = crb[req];
  const int je = crb[req + 1];
  const int L_in = as_const(a.cache_seqlens)[req];
  cint32* pt_row = as_const(a.page_table + (int64_t)req * a.page_table_stride);
  const int nb = je - jb;
  // A key split at or past the request's length has no keys (split 0 always
  // runs: it holds the drafts of the fused launch and the row checks).
  if (split != 0 && (int64_t)split * a.split_len >= L_in) return;
  const int tok0 = cqo[jb];
  const int tok1 = cqo[je];
  asm volatile("" ::"s"(L_in));
  if (tok0 < 0 || tok1 < tok0 || tok1 > a.total_rows) {
    if (tid == 0) atomicOr(&g_device_error, kErrRow);
    return;
  }
  const int nrows = (tok1 - tok0) * a.group;
  const int row0 = chunk * kRowsPerItem;
  if (chunk == 0 && split == 0 && tid == 0 && nrows > a.n_chunks * kRowsPerItem)
    atomicOr(&g_device_error, kErrRow);  // rows past the planned chunks are not computed
  if (row0 >= nrows) return;
  const int nrc = min(nrows - row0, kRowsPerItem);  // rows of this chunk
  const int tok_first = row0 / a.group;
  const int tok_last = (row0 + nrc - 1) / a.group;
  const int dhi = tok_last + 1;  // draft keys the chunk's rows can see end here

  // Pass B of a request with a single branch (a prefix-hit suffix, a draft
  // tree): its draft keys are consecutive slots of one block-table row
  // (token x at slot ds0 + x), so the key loop streams them like a prefix,
  // from the 32-slot boundary at or below ds0; the keys in front of the
  // branch are staged as zeros and masked.  Other requests take their draft
  // tiles through per-key offset tables (the draft phase below).
  // The fused verify launch streams such a branch the same way after the
  // prefix (split 0).
  bool slot_mode = false;
  int ds0 = 0;
  int p0 = 0, p1 = 0;
  const int64_t dcap = (int64_t)a.draft_page_table_stride << a.kv.log2_page;
  if (kDraft || (kVerify && split == 0)) {
    if (nb == 1 && dcap > 0) {
      ds0 = a.draft_start ? as_const(a.draft_start)[jb] : 0;
      slot_mode = ds0 >= 0 && ds0 < dcap;
    }
  }
  // Key range of a slot-mode branch: slots [ds0 & ~31, ds0 + dhi) of its row.
  auto slot_range = [&](int& q0, int& q1) {
    int64_t se = (int64_t)ds0 + dhi;
    if (se > dcap) {
      if (tid == 0) atomicOr(&g_device_error, kErrPage);
      se = dcap;
    }
    q0 = ds0 & ~31;
    q1 = (int)se;
  };
  if constexpr (kDraft) {
    if (slot_mode) {
      pt_row = as_const(a.draft_page_table + (int64_t)jb * a.draft_page_table_stride);
      slot_range(p0, p1);
    }
  }
  // A request whose keys all fall in split 0 writes its final output (the
  // split merge leaves its rows alone).
  bool partial = false;
  if constexpr (!kDraft) {
  int L = L_in;
  {
    const int cap = a.page_table_stride << a.kv.log2_page;
    if (L > cap) {
      if (tid == 0) atomicOr(&g_device_error, kErrLen);
      L = cap;
    }
    if (L < 0) L = 0;
    const int planned = a.n_splits * a.split_len;
    if (L > planned) {
      if (tid == 0) atomicOr(&g_device_error, kErrLen);
      L = planned;
    }
  }
  // Uniform by construction; stated so that the buffer descriptors built
  // from them live in scalar registers (the flag stores above are per lane).
  L = __builtin_amdgcn_readfirstlane(L);
  p0 = split * a.split_len;
  p1 = min(L, p0 + a.split_len);
  if (a.n_splits > 1 && p0 >= L && (MODE == kModePrefix || split != 0)) return;
  if (p1 < p0) p1 = p0;
  partial = a.n_splits > 1 && L > a.split_len;
  }
  p0 = __builtin_amdgcn_readfirstlane(p0);
  p1 = __builtin_amdgcn_readfirstlane(p1);
  int nt = (p1 - p0 + 31) >> 5;  // tiles of the key loop
  // Key loop tiles as the mask sees them: prefix keys [p0, p1), or the draft
  // tokens of a slot-mode branch (slot - ds0, negative in front of it; the
  // slots in front of the branch are staged as zeros).
  int kshift = kDraft ? ds0 : 0;
  int kend = kDraft ? dhi : p1;
  int front = kDraft ? ds0 : p0;

  const KvView kv = a.kv;
  const float c2 = a.scale_log2;
  const int64_t head_off = (int64_t)g * kv.head_stride;

  // ---- this lane's rows: wave w holds chunk rows [ROWS_W w, ROWS_W (w+1)) --
  // Rows fill whole waves from wave 0 on (waves past the last row only load
  // and stage): spreading them thinner would pad every 16-row block and make
  // more waves read each tile out of LDS.  Row block rb of the wave: rows
  // ROWS_W w + 16 rb + l16.
  const bool wave_rows = w * ROWS_W < nrc;  // uniform
  bool rvalid[RBW];
  int rtok[RBW];
  int64_t orow[RBW];
  bf16x8 qf[RBW][KS];  // Q B-fragments: channels ks*32 + g4*8 .. +8 of the row
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    const int rw = w * ROWS_W + rb * 16 + l16;
    rvalid[rb] = rw < nrc;
    const int rho = row0 + (rvalid[rb] ? rw : 0);  // row within (request, kv head)
    rtok[rb] = rho / a.group;                      // request token of the row
    const int hq = g * a.group + (rho - rtok[rb] * a.group);
    orow[rb] = (int64_t)(tok0 + rtok[rb]) * a.num_qo_heads + hq;
    const uint16_t* qp = a.q + (int64_t)(tok0 + rtok[rb]) * a.q_row_stride + (int64_t)hq * a.q_head_stride + g4 * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[rb][ks] = rvalid[rb] ? *reinterpret_cast<const bf16x8*>(qp + ks * 32) : bf16x8{};
      if constexpr (KV8) {
        if (a.k_cs)
          qf[rb][ks] = __builtin_bit_cast(
              bf16x8, scale_q_chunk(__builtin_bit_cast(u32x4, qf[rb][ks]), a.k_cs + (int64_t)g * D + ks * 32 + g4 * 8));
      }
    }
  }

  // ---- prefix tile loads -------------------------------------------------
  // Chunk e = tid + q*NT of a tile is chunk e % 16 of key e / 16: the wave's
  // four keys of chunk q lie in the tile's 16-key half e / 256, whose page id
  // is wave-uniform, at the same place in the half for every q.  The half's
  // buffer descriptors start at its first key and end after the row of its
  // last valid key, so keys past `p1` (and bad pages) read zeros.
  auto half_of = [&](int q) { return (w * 64 + q * NT) >> 8; };
  const int lane_off = prefix_lane_offset<EB>(kv, (w * 4 + g4) & 15, head_off, l16);
  // Page ids outside the pool are noted here and flagged once at the end: a
  // store in the key loop would count on the same counter as the K/V loads
  // and blur the loop's wait counts.
  bool bad_page = false;
  auto page_of = [&](int tile) -> Pages {  // page ids of this wave's halves of a tile, -1 if none
    Pages pg;
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int first = p0 + tile * 32 + half_of(q) * 16;
      int id = first < p1 ? pt_row[first >> kv.log2_page] : -1;
      id = __builtin_amdgcn_readfirstlane(id);
      bad_page |= id >= kv.num_pages;
      pg.p[q] = checked_page(id, kv.num_pages);
    }
    return pg;
  };
  const int tail_bytes = (int)((head_off + D) * EB);
  auto load_tile = [&](int tile, const Pages& pg, Tile& tl) {
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int first = p0 + tile * 32 + half_of(q) * 16;
      const int nvalid = min(max(p1 - first, 0), 16);
      const HalfSpan h = prefix_half_span(kv, pg.p[q], first, nvalid, tail_bytes);
      tl.k[q] = buf_load_chunk(half_rsrc(kv.k, h), lane_off, (Raw*)nullptr);
      tl.v[q] = buf_load_chunk(half_rsrc(kv.v, h), lane_off, (Raw*)nullptr);
    }
  };
  // bf16 pools: a tile copied straight into a stage.  Lane (g4, l16) of wave
  // w fills slot l16 of key 4w + g4 of each 16-key half: K chunk
  // l16 ^ (4w + g4) and V chunk l16 ^ 2 g4 (the swizzles, with k & 15 =
  // 4w + g4 and k & 3 = g4); the 64 lanes' 16 bytes land side by side, four
  // whole rows per copy.  Keys past the range read zeros through the
  // descriptors; `front_zero` also zeroes the keys of tile 0 in front of
  // `front` (an offset past every descriptor).
  const int dma_off_k = prefix_lane_offset<EB>(kv, w * 4 + g4, head_off, l16 ^ (w * 4 + g4));
  const int dma_off_v = prefix_lane_offset<EB>(kv, w * 4 + g4, head_off, l16 ^ (g4 << 1));
  auto dma_tile = [&](int tile, const Pages& pg, uint16_t* st, bool front_zero) {
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int first = p0 + tile * 32 + half_of(q) * 16;
      const int nvalid = min(max(p1 - first, 0), 16);
      const HalfSpan h = prefix_half_span(kv, pg.p[q], first, nvalid, tail_bytes);
      const bool zero = front_zero && first + w * 4 + g4 < front;
      const int row = half_of(q) * 16 + w * 4;
      lds_copy16(half_rsrc(kv.k, h), lds_addr(st + row * ROWE), zero ? 0x7ffffff0 : dma_off_k);
      lds_copy16(half_rsrc(kv.v, h), lds_addr(st + (32 + row) * ROWE), zero ? 0x7ffffff0 : dma_off_v);
    }
  };
  // Thread tid's chunks of a tile into a stage (chunk q zeroed where bit q of
  // `keep` is clear).
  auto skey = [&](int q) { return (tid + q * NT) >> 4; };
  const int sch = tid & 15;
  constexpr int kKeepAll = (1 << CPT) - 1;
  auto stage = [&](const Tile& tl, int keep, uint16_t* st) {
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      u32x4 k = widen_bf16(tl.k[q]), v = widen_bf16(tl.v[q]);
      if (!((keep >> q) & 1)) {
        k = u32x4{0u, 0u, 0u, 0u};
        v = u32x4{0u, 0u, 0u, 0u};
      }
      const int key = skey(q);
      *reinterpret_cast<u32x4*>(st + key * ROWE + ((sch ^ (key & 15)) << 3)) = k;
      *reinterpret_cast<u32x4*>(st + (32 + key) * ROWE + ((sch ^ ((key & 3) << 1)) << 3)) = v;
    }
  };

  // DEPTH tiles requested before the first one is staged; `pgn` holds the
  // pages of the next tile to be requested.
  Tile ring[kDma ? 1 : DEPTH];
  Pages pgn = page_of(0);
  auto request_first = [&]() {
    if constexpr (kDma) {
#pragma unroll
      for (int k = 0; k < NS - 1; ++k) {
        dma_tile(k, pgn, stg[k], k == 0);
        pgn = page_of(k + 1);
      }
    } else {
#pragma unroll
      for (int k = 0; k < DEPTH; ++k) {
        load_tile(k, pgn, ring[k]);
        pgn = page_of(k + 1);
      }
    }
  };
  request_first();

  // ---- tree tables (fused verify split 0, pass B not in slot mode) ---------
  const bool drafts = (kVerify && split == 0 && !slot_mode) || (kDraft && !slot_mode);
  const bool lds_bnd = nb <= NBCAP;
  int dlo = 0;
  // The first draft tile: requested right after the tables at two
  // workgroups per CU; after the key loop at three (no registers held
  // across the loop).
  constexpr bool kEarlyDraft = NS == 4;
  Tile dt;
  int dkeep = 0;
  auto branch_at = [&](int x) -> int {  // local branch of request token x
    if (lds_bnd) {
      int lo = 0, hi = nb - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (t_bnd[mid] - tok0 <= x) lo = mid; else hi = mid - 1;
      }
      return lo;
    }
    return branch_of_row(a.branch_qo_indptr, jb, je, tok0 + x) - jb;
  };
  auto branch_start = [&](int jl) { return (lds_bnd ? t_bnd[jl] : a.branch_qo_indptr[jb + jl]) - tok0; };
  auto branch_dstart = [&](int jl) {
    return lds_bnd ? t_dst[jl] : (a.draft_start ? a.draft_start[jb + jl] : 0);
  };
  const int64_t last_row = pool_last_row(kv, a.num_kv_heads);
  // Keys base + skey(q) of a draft tile (request tokens), chunk tid % 16;
  // zeros for keys past dhi and for bad slots or pages (flagged).
  auto load_draft = [&](int base, Tile& tl, int& keep) {
    keep = 0;
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int x = base + skey(q);
      int64_t off = -2;  // element offset of the key's row (kv head included)
      if (x < dhi) {
        if (x - dlo < KEYCAP) {
          off = t_doff[x - dlo];
          if (off >= 0) off += head_off;
        } else {
          off = draft_offset(kv, a.branch_qo_indptr, a.draft_page_table, a.draft_page_table_stride,
                             a.draft_start, jb, je, x, g);
        }
        if (off == -1) atomicOr(&g_device_error, kErrPage);
      }
      const bool ok = off >= 0;
      keep |= ok ? (1 << q) : 0;
      const int64_t e = clamp_row(off, last_row) + sch * 8;
      tl.k[q] = ok ? load_key_chunk<Raw, EB>(kv.k, e) : Raw{};
      tl.v[q] = ok ? load_key_chunk<Raw, EB>(kv.v, e) : Raw{};
    }
  };
  if constexpr (kTables) {
    if (drafts) {
      if (lds_bnd) {
        for (int t = tid; t <= nb; t += NT) t_bnd[t] = a.branch_qo_indptr[jb + t];
        for (int t = tid; t < nb; t += NT) t_dst[t] = a.draft_start ? a.draft_start[jb + t] : 0;
      }
      __syncthreads();
      dlo = __builtin_amdgcn_readfirstlane(branch_start(branch_at(tok_first)));
      for (int t = tid; t <= tok_last - tok_first; t += NT) t_rbs[t] = branch_start(branch_at(tok_first + t));
      const int nk = min(dhi - dlo, KEYCAP);
      const int dstride = a.draft_page_table_stride;
      for (int t = tid; t < nk; t += NT) {
        const int x = dlo + t;
        const int jl = branch_at(x);
        const int slot = branch_dstart(jl) + (x - branch_start(jl));
        t_doff[t] = draft_slot_offset(kv, a.draft_page_table + (int64_t)(jb + jl) * dstride, dstride, slot);
      }
      __syncthreads();
      if constexpr (kEarlyDraft) load_draft(dlo, dt, dkeep);
    }
  }

  // ---- the key loop ---------------------------------------------------------
  float m[RBW], l[RBW];
  f32x4 o[RBW][DB];
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    m[rb] = kNegInf;
    l[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  auto kfrag = [&](const uint16_t* st, int kb, int ks) -> bf16x8 {
    const int key = kb * 16 + l16;
    return *reinterpret_cast<const bf16x8*>(st + key * ROWE + (((ks * 4 + g4) ^ (key & 15)) << 3));
  };
  auto vt_frag = [&](const uint16_t* st, int db) -> bf16x8 {
    const int row = 4 * g4 + (l16 >> 2);
    const int c = 2 * db + ((l16 & 3) >> 1);
    const uint16_t* vb = st + (32 + row) * ROWE + ((c ^ ((row & 3) << 1)) << 3) + 4 * (l16 & 1);
    const i16x4 lo = lds_read_tr16(vb);
    const i16x4 hi = lds_read_tr16(vb + 16 * ROWE);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // The lane's row's draft visibility (fused verify): request token, start of
  // its branch, ancestor set for general trees.
  int rbs[RBW] = {};
  uint64_t ranc[RBW] = {};
  const bool tree = a.draft_mask != nullptr;
  // One tile out of a stage into the lane's row state.  kind 0: prefix keys
  // [base, end); kind 1: draft keys under the ancestor rule.
  auto compute = [&](const uint16_t* st, int base, int end, int kind) {
    f32x4 s[RBW][2];
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) s[rb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // The matrix phases run at raised wave priority: when the waves of a
    // SIMD (independent workgroups) both have work, the one with MFMAs to
    // issue goes first and the others' softmax fills in behind it.
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 kf = kfrag(st, kb, ks);
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb) s[rb][kb] = mfma16(kf, qf[rb][ks], s[rb][kb]);
      }
    __builtin_amdgcn_s_setprio(0);
    // At two workgroups per CU (registers to spare) each row block's P.V
    // follows its own softmax, the tile's V fragments read out of the stage
    // beforehand, so that the first block's P.V runs while the second block's
    // weights are formed (ragged batch: 0.56 against 0.59 ms).  At three, the
    // P.V of both blocks follows both softmaxes (held V fragments would spill).
    constexpr bool kPvPerBlock = NS == 4 && !KV8;
    bf16x8 pf[RBW];
    bf16x8 vfr[kPvPerBlock ? DB : 1];
    if constexpr (kPvPerBlock) {
#pragma unroll
      for (int db = 0; db < DB; ++db) vfr[db] = vt_frag(st, db);
    }
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) {
      // One uniform branch per tile picks the rule (tree masks or chains).
      if (kind == 1 && tree) {
        // The tree's window for this tile (see tree_window).
        const int ws = max(base - rbs[rb], 0);
        const uint64_t win =
            a.draft_mask_words == 1
                ? tree_window1(ranc[rb], ws)
                : tree_window(a.draft_mask + (int64_t)(tok0 + rtok[rb]) * a.draft_mask_words, a.draft_mask_words, ws);
        const int wbs = rbs[rb] + ws;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = base + kb * 16 + g4 * 4 + i;
            const bool vis = (key < end) & draft_visible_tree(win, wbs, key);
            s[rb][kb][i] = vis ? s[rb][kb][i] : kNegInf;
          }
      } else if (kind == 1) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = base + kb * 16 + g4 * 4 + i;
            const bool vis = (key < end) & draft_visible(rtok[rb], rbs[rb], key);
            s[rb][kb][i] = vis ? s[rb][kb][i] : kNegInf;
          }
      } else if (base + 32 > end) {
        // The tile's last keys lie past `end`: key base + kb*16 + g4*4 + i is
        // kept iff g4*4 < end - base - kb*16 - i (a uniform bound per key).
        const int n = end - base;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) s[rb][kb][i] = g4 * 4 < n - (kb * 16 + i) ? s[rb][kb][i] : kNegInf;
      }
      // Online softmax in base 2; the carried max is raised only past a slack.
      const float lm = fmaxf(fmaxf(fmaxf(s[rb][0][0], s[rb][0][1]), fmaxf(s[rb][0][2], s[rb][0][3])),
                             fmaxf(fmaxf(s[rb][1][0], s[rb][1][1]), fmaxf(s[rb][1][2], s[rb][1][3])));
      if (__any(lm * c2 > m[rb] + kMaxSlack)) {
        const float mx = rowgroup_max(lm) * c2;
        const float mnew = mx > m[rb] + kMaxSlack ? mx : m[rb];
        const float ms = mnew == kNegInf ? 0.f : mnew;
        const float alpha = mnew == m[rb] ? 1.f : fast_exp2(m[rb] - ms);
        const bool resc = mnew != m[rb] && m[rb] != kNegInf;
        m[rb] = mnew;
        l[rb] *= alpha;
        if (__any(resc)) {
#pragma unroll
          for (int db = 0; db < DB; ++db) o[rb][db] *= alpha;
        }
      }
      const float ms = m[rb] == kNegInf ? 0.f : m[rb];
      float p[8];
      float sum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[kb * 4 + i] = fast_exp2(s[rb][kb][i] * c2 - ms);
          sum += p[kb * 4 + i];
        }
      l[rb] += sum;
      const u32x4 pk = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                        pack_bf16x2(p[6], p[7])};
      pf[rb] = __builtin_bit_cast(bf16x8, pk);
      if constexpr (kPvPerBlock) {
#pragma unroll
        for (int db = 0; db < DB; ++db) o[rb][db] = mfma16(vfr[db], pf[rb], o[rb][db]);
      }
    }
    if constexpr (!kPvPerBlock) {
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16x8 vf = vt_frag(st, db);
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb) o[rb][db] = mfma16(vf, pf[rb], o[rb][db]);
      }
      __builtin_amdgcn_s_setprio(0);
    }
  };

  // Request token of the wave's first row (its rows' tokens are not smaller).
  const int wave_tok = (row0 + w * ROWS_W) / a.group;
  // Slot-mode branches: every row's branch starts at request token 0.
  if ((kDraft || kVerify) && slot_mode && tree) {
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb)
      if (rvalid[rb]) ranc[rb] = a.draft_mask[(int64_t)(tok0 + rtok[rb]) * a.draft_mask_words];
  }
  // The key loop over the current key range, its first DEPTH tiles requested:
  // tile 0 into stage 0 (slots in front of `front` as zeros); its slot then
  // requests tile DEPTH.
  // The range's mask kind (0: prefix keys, 1: draft keys) is a compile-time
  // tag, so each instantiation keeps one masking rule per tile.
  // Step t: stage tile t+1 (slot (t+1) % DEPTH) into stage (t+1) & 1, request
  // tile t+1+DEPTH into that slot, compute tile t out of stage t & 1, barrier.
  // Tiles past the range are empty: no memory access, zeros staged.
  // Whole rings of DEPTH steps, with no exit inside a ring: every back edge
  // then carries the same ring state as the entry, and each stage waits for
  // its own slot only.  Steps past the last tile stage zeros and compute
  // nothing.
  // bf16: step t waits for this wave's copies of tile t (at most the NS - 2
  // later tiles' four copies each still in flight), meets the other waves at
  // the barrier, copies tile t+NS-1 into the stage tile t-1 left, and
  // computes tile t.  Whole rings of NS steps; steps past the range copy
  // nothing useful (zeros) and compute nothing.  The loop ends with every
  // copy landed.
  auto key_loop_dma = [&](auto kind_tag) {
    constexpr int KIND = decltype(kind_tag)::value;
    constexpr int kWaitTile = 4 * (NS - 2) | (7 << 4) | (15 << 8);  // s_waitcnt vmcnt(4 (NS - 2))
    constexpr int kWait0 = 0 | (7 << 4) | (15 << 8);  // s_waitcnt vmcnt(0)
    // Every load in flight lands first (the query rows and tables, and the
    // first NS - 1 tiles): the compiler, which cannot count the copies, then
    // has no load of its own left to wait for inside the loop.
    __builtin_amdgcn_s_waitcnt(kWait0);
    for (int t0 = 0; t0 < nt; t0 += NS) {
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        const int t = t0 + k;
        __builtin_amdgcn_s_waitcnt(kWaitTile);
        __syncthreads();
        dma_tile(t + NS - 1, pgn, stg[(k + NS - 1) % NS], false);
        pgn = page_of(t + NS);
        if (wave_rows && t < nt) {
          const int tb = p0 + t * 32 - kshift;
          const bool open = KIND == 1 && slot_mode && !tree && tb >= 0 && tb + 32 <= wave_tok + 1;
          compute(stg[k], tb, open ? tb + 32 : kend, open ? 0 : KIND);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(kWait0);
    __syncthreads();
  };
  auto key_loop = [&](auto kind_tag) {
    constexpr int KIND = decltype(kind_tag)::value;
    {
      int keep = 0;
#pragma unroll
      for (int q = 0; q < CPT; ++q) keep |= p0 + skey(q) >= front ? (1 << q) : 0;
      stage(ring[0], keep, stg[0]);
    }
    load_tile(DEPTH, pgn, ring[0]);
    pgn = page_of(DEPTH + 1);
    __syncthreads();
    for (int t0 = 0; t0 < nt; t0 += DEPTH) {
#pragma unroll
      for (int k = 0; k < DEPTH; ++k) {
        const int t = t0 + k;
        const int sn = (k + 1) % DEPTH;
        stage(ring[sn], kKeepAll, stg[(k + 1) & 1]);
        load_tile(t + 1 + DEPTH, pgn, ring[sn]);
        pgn = page_of(t + 2 + DEPTH);
        if (wave_rows && t < nt) {
          // A slot-mode chain tile that ends at or before the wave's first
          // row token is visible to all of the wave's rows: no mask.
          const int tb = p0 + t * 32 - kshift;
          const bool open = KIND == 1 && slot_mode && !tree && tb >= 0 && tb + 32 <= wave_tok + 1;
          compute(stg[k & 1], tb, open ? tb + 32 : kend, open ? 0 : KIND);
        }
        __syncthreads();
      }
    }
  };
  if constexpr (kDma) {
    key_loop_dma(KeyKind<kDraft ? 1 : 0>{});
  } else {
    key_loop(KeyKind<kDraft ? 1 : 0>{});
  }

  // ---- fused verify, slot mode: the branch's draft keys as a second range ---
  if constexpr (kVerify) {
    if (split == 0 && slot_mode) {
      pt_row = as_const(a.draft_page_table + (int64_t)jb * a.draft_page_table_stride);
      slot_range(p0, p1);
      p0 = __builtin_amdgcn_readfirstlane(p0);
      p1 = __builtin_amdgcn_readfirstlane(p1);
      nt = (p1 - p0 + 31) >> 5;
      kshift = ds0;
      kend = dhi;
      front = ds0;
      pgn = page_of(0);
      request_first();
      if constexpr (kDma) {
        key_loop_dma(KeyKind<1>{});
      } else {
        key_loop(KeyKind<1>{});
      }
    }
  }

  // ---- pass B through the offset tables: the chunk's visible draft tiles ---
  if constexpr (kTables) {
    if (drafts) {
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb)
        if (rvalid[rb]) {
          rbs[rb] = t_rbs[rtok[rb] - tok_first];
          if (tree) ranc[rb] = a.draft_mask[(int64_t)(tok0 + rtok[rb]) * a.draft_mask_words];
        }
      for (int base = dlo; base < dhi; base += 32) {
        if (!kEarlyDraft || base != dlo) load_draft(base, dt, dkeep);
        stage(dt, dkeep, stg[0]);
        __syncthreads();
        if (wave_rows) compute(stg[0], base, dhi, 1);
        __syncthreads();
      }
    }
  }
  mfma_drain();
  if (bad_page && lane == 0) atomicOr(&g_device_error, kErrPage);

  // ---- output ----------------------------------------------------------------
  const int64_t plane = (int64_t)a.total_rows * a.num_qo_heads;
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    l[rb] = rowgroup_sum(l[rb]);
    if (!rvalid[rb]) continue;
    const float lse2 = l[rb] > 0.f ? m[rb] + fast_log2(l[rb]) : kNegInf;
    // FP8 pools: the V scale multiplies every normalised output once, here,
    // and per-channel V scales each output channel.
    const float f = l[rb] > 0.f ? (KV8 ? a.v_scale : 1.f) / l[rb] : 0.f;
    if constexpr (KV8) {
      if (a.v_cs) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
          o[rb][db] *= *reinterpret_cast<const f32x4*>(a.v_cs + (int64_t)g * D + db * 16 + g4 * 4);
      }
    }
    if (partial) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<f32x4*>(a.ws_o + (split * plane + orow[rb]) * D + db * 16 + g4 * 4) = o[rb][db] * f;
      if (g4 == 0) a.ws_lse[split * plane + orow[rb]] = lse2;
      continue;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const f32x4 x = o[rb][db] * f;
      const int c = db * 16 + g4 * 4;
      if (a.o_bf16) {
        *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a.o) + orow[rb] * D + c) =
            u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
      } else {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.o) + orow[rb] * D + c) = x;
      }
    }
    if (g4 == 0 && a.lse) a.lse[orow[rb]] = lse2 * kLn2;
  }
}

}  // namespace casc
