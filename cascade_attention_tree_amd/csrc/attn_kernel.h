// Paged attention kernels of the cascade verify path (gfx950, wave64, MFMA bf16).
//
// One workgroup = 4 waves (one per SIMD) handles one work item
//   (segment, kv head g, row chunk, key split)
// where a segment is a request (pass A, pass B, verify) or a branch (naive
// expansion).  The rows of an item are the segment's query tokens times the
// query heads that share kv head g (GQA), token-major, in chunks of at most
// 16*RB rows.  The whole chunk is one dense row tile, so each K/V tile read
// from HBM serves all topk*S*group query rows of the request at once.
//
// Inside the workgroup every wave keeps all rows of the chunk and takes every
// 4th 32-key tile.  Per tile a wave
//   * has the tile's K and V rows in registers (loaded one iteration earlier:
//     whole 256-byte key rows per group of lanes, through the block table),
//     writes them to its own LDS stage and issues the loads of its next tile,
//   * reads K back as MFMA A-fragments and computes S^T = K Q^T with
//     v_mfma_f32_16x16x32_bf16 (keys on M, rows on N),
//   * updates a base-2 online softmax per row; the cross-lane row max is only
//     formed when some lane's own max exceeds the carried max by the slack,
//   * reads V back transposed (ds_read_b64_tr_b16) as the A-fragments of
//     O^T += V^T P^T.  P^T is already in B-fragment layout in the lanes that
//     computed S^T, so P never moves between lanes.
//
// Before the key loop the workgroup resolves everything that depends on the
// tree layout into small LDS tables (branch starts of its tokens, physical
// offsets of the draft keys it can see), so that no chain of dependent global
// loads sits on the path of the key loop or of the epilogue.
//
// The four waves then merge their states with the LSE identity; each wave
// ends up owning a quarter of the head dimension.  Depending on the mode the
// merged state is written as a pass state, as a split partial (merged later
// by the split-merge kernel), or as the final output.
#pragma once

#include "device_common.h"

namespace casc {

// A row's running max is only raised when a tile exceeds it by more than this
// (base-2 units).  Weights exp2(s - m) then stay below 2^kMaxSlack, and the O
// accumulator is rescaled only when some row's max really moves.  The result
// is the same softmax; only which common factor is carried differs.
constexpr float kMaxSlack = 8.0f;

// LSE merge of two states given as base-2 log-sum-exps:
//   lse = log2(2^a + 2^b), weights 2^(a - lse) and 2^(b - lse).
__device__ __forceinline__ void merge_weights(float a, float b, float& wa, float& wb, float& lse) {
  const float mx = fmaxf(a, b);
  if (mx == kNegInf) {
    wa = 0.f;
    wb = 0.f;
    lse = kNegInf;
    return;
  }
  lse = mx + fast_log2(fast_exp2(a - mx) + fast_exp2(b - mx));
  wa = fast_exp2(a - lse);
  wb = fast_exp2(b - lse);
}

__device__ __forceinline__ f32x4 wsum(float wa, f32x4 a, float wb, f32x4 b) {
  f32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = (wa == 0.f ? 0.f : wa * a[i]) + (wb == 0.f ? 0.f : wb * b[i]);
  return r;
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Wait states after the last MFMA of a loop whose accumulators are read past
// the loop exit: 24 issue slots, more than any MFMA result latency.
__device__ __forceinline__ void mfma_drain() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Max and sum over lanes l, l^16, l^32, l^48 -- the four key groups that hold
// one row of an S^T block -- with the row swaps of CDNA4 (VALU only).  A swap
// of a register with a copy of itself leaves rows {0,1} (resp. {2,3}, or the
// two halves) of the same lanes in the two results; every lane ends with the
// same value, combined in the same order.  Both results pass through an empty
// asm: without it the optimizer folds a combine of the two results of the
// swap into its first result.
__device__ __forceinline__ void swap_rows16(float x, float& p, float& q) {
  unsigned u = __builtin_bit_cast(unsigned, x), c = u;
  asm volatile("" : "+v"(c));
  const auto r = __builtin_amdgcn_permlane16_swap(u, c, false, false);
  unsigned r0 = r[0], r1 = r[1];
  asm volatile("" : "+v"(r0), "+v"(r1));
  p = __builtin_bit_cast(float, r0);
  q = __builtin_bit_cast(float, r1);
}
__device__ __forceinline__ void swap_rows32(float x, float& p, float& q) {
  unsigned u = __builtin_bit_cast(unsigned, x), c = u;
  asm volatile("" : "+v"(c));
  const auto r = __builtin_amdgcn_permlane32_swap(u, c, false, false);
  unsigned r0 = r[0], r1 = r[1];
  asm volatile("" : "+v"(r0), "+v"(r1));
  p = __builtin_bit_cast(float, r0);
  q = __builtin_bit_cast(float, r1);
}
__device__ __forceinline__ float rowgroup_max(float x) {
  float p, q;
  swap_rows16(x, p, q);
  swap_rows32(fmaxf(p, q), p, q);
  return fmaxf(p, q);
}
__device__ __forceinline__ float rowgroup_sum(float x) {
  float p, q;
  swap_rows16(x, p, q);
  swap_rows32(p + q, p, q);
  return p + q;
}

typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Transposing LDS read: within each group of 16 lanes, lane i receives
// element (i & 3) of the 4-element vectors addressed by lanes i/4, 4 + i/4,
// 8 + i/4, 12 + i/4 (in that order).
__device__ __forceinline__ i16x4 lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

// A wave index as a type (merge code specialised per wave).
template <int W>
struct WaveIndex {
  static constexpr int value = W;
};

// KV8: the pools hold FP8 E4M3 codes (half the bytes per key); each chunk is
// widened to bf16 when staged, so everything from the LDS stage on is shared.
template <int D, int RB, int MODE, bool KV8 = false>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
attn_kernel(const AttnArgs a) {
  constexpr int KS = D / 32;        // k-steps of the Q K^T contraction
  constexpr int DB = D / 16;        // 16-channel blocks of the head dim
  constexpr int DBW = DB / 4;       // blocks each wave owns after the combine
  constexpr int ROWS = RB * 16;
  constexpr int NI = D / 16;        // 16-byte loads per lane for one 32-key tile of K (or V)
  constexpr int CPR = D / 8;        // 16-byte chunks per key row
  constexpr int TPI = 64 / CPR;     // key rows covered by one row-shaped load
  // Bytes per pool element, and one chunk of 8 channels as loaded.
  constexpr int EB = KV8 ? 1 : 2;
  typedef typename KvChunk<KV8>::T Raw;
  // LDS row stride (bf16) of staged K and V tiles.  D + 16 puts consecutive
  // rows 8 banks apart: the A-fragment reads (16 B of 8 consecutive keys per
  // pass) and the transposed V reads (8 B of 4 consecutive keys x 4 column
  // quads per 16 lanes) touch distinct banks, and rows stay 16-byte aligned.
  constexpr int RS = D + 16;
  constexpr int STAGE = 2 * 32 * RS;  // bf16 elements per wave: the K tile, then the V tile
  constexpr int XSLOT = RB * DBW * 64 * 4;  // floats per (owner, source) exchange slot
  constexpr int STAGE_BYTES = 4 * STAGE * 2;
  constexpr int XBYTES = 12 * XSLOT * 4;
  constexpr int UNION_BYTES = STAGE_BYTES > XBYTES ? STAGE_BYTES : XBYTES;
  static_assert(MODE >= kModePrefix && MODE <= kModeNaive, "pass A, pass B, verify or naive expansion");
  constexpr bool kDraftKeys = MODE == kModeDraft || MODE == kModeNaive || MODE == kModeVerify;
  // In the fused verify launch the request's draft tiles are taken by one
  // wave, after its share of the prefix tiles, into its own online softmax
  // state; the wave merge below then combines pass A and pass B with the same
  // LSE identity as the prefix partial states.  Wave 3 has the fewest prefix
  // tiles (tiles go round-robin from wave 0).
  constexpr int kDraftWave = 3;
  // Large row tiles keep Q in LDS (read per tile as B-fragments) so that the
  // architectural VGPRs stay free for K/V in flight and the softmax.
  constexpr bool kQInLds = RB * KS >= 16;
  constexpr int QSTR = D + 8;  // padded LDS row stride of Q: rows land 4 banks apart
  constexpr int QBYTES = kQInLds ? ROWS * QSTR * 2 : 0;
  constexpr int MLBYTES = 4 * ROWS * 2 * 4;
  // Tree tables: branches of one segment, and draft keys of one chunk, whose
  // lookups are resolved in LDS; larger segments fall back to global lookups.
  constexpr int NBCAP = 128;
  constexpr int KEYCAP = 512;
  constexpr int TBYTES = kDraftKeys ? KEYCAP * 8 + ((2 * NBCAP + 1 + ROWS) * 4 + 15) / 16 * 16 : 0;

  __shared__ __attribute__((aligned(16))) unsigned char smem[UNION_BYTES + QBYTES + MLBYTES + TBYTES];
  uint16_t* qs = reinterpret_cast<uint16_t*>(smem + UNION_BYTES);                // [ROWS][QSTR]
  float* ml = reinterpret_cast<float*>(smem + UNION_BYTES + QBYTES);             // [4][ROWS][m, l]
  int64_t* t_doff = reinterpret_cast<int64_t*>(smem + UNION_BYTES + QBYTES + MLBYTES);  // [KEYCAP]
  int* t_bnd = reinterpret_cast<int*>(t_doff + KEYCAP);  // [NBCAP + 1] branch_qo_indptr window
  int* t_dst = t_bnd + NBCAP + 1;                        // [NBCAP] draft_start window
  int* t_rbs = t_dst + NBCAP;                            // [ROWS] branch start per chunk token

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15;
  const int g4 = lane >> 4;

  // ---- work item -------------------------------------------------------
  // Key splits vary slowest, so that every XCD gets a like share of each
  // split's (uneven) work when requests differ in length and row count.
  // Within a split, workgroup u goes to XCD u % 8 (round-robin dispatch) and
  // u / 8 walks the row chunks of one (segment, kv head) pair, then the next
  // pair of that XCD: the chunks of a pair run side by side on one L2, which
  // serves every chunk after the first its prefix tiles.
  const int per_split = (int)gridDim.x / a.grid_splits;
  const int split = (int)blockIdx.x / per_split;
  const int u = (int)blockIdx.x - split * per_split;
  const int v8 = u >> 3;
  const int chunk = v8 % a.n_chunks;
  const int item = (v8 / a.n_chunks) * 8 + (u & 7);
  if (item >= a.n_seg_items) return;
  const int g = item % a.num_kv_heads;
  const int seg = item / a.num_kv_heads;

  const int32_t* __restrict__ qo = a.branch_qo_indptr;
  cint32* cqo = as_const(qo);
  int req, jb, je;
  if constexpr (MODE == kModeNaive) {
    jb = seg;
    je = seg + 1;
    // The request owning branch `seg`: the requests whose first branch is at
    // or before it, minus one (req_branch_indptr is non-decreasing).
    int cnt = 0;
    for (int i0 = 0; i0 < a.batch_size; i0 += 256) {
      const int i = i0 + (int)threadIdx.x;
      cnt += __syncthreads_count(i < a.batch_size && a.req_branch_indptr[i] <= seg);
    }
    req = __builtin_amdgcn_readfirstlane(cnt > 0 ? cnt - 1 : 0);
  } else {
    cint32* crb = as_const(a.req_branch_indptr);
    req = seg;
    jb = crb[seg];
    je = crb[seg + 1];
  }
  // The request's length and the block-table entries of this wave's first
  // prefix tile are requested together with the branch range, so that the
  // first K/V loads wait for one round trip of small loads, not a chain.
  const int L_in = as_const(a.cache_seqlens)[req];
  cint32* pt_row = as_const(a.page_table + (int64_t)req * a.page_table_stride);
  int pt_first[2] = {-1, -1};
  if constexpr (MODE == kModePrefix || MODE == kModeVerify) {
    const int stride = a.page_table_stride;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int idx = (split * a.split_len + w * 32 + kb * 16) >> a.kv.log2_page;
      if (stride > 0) pt_first[kb] = pt_row[idx < stride ? idx : stride - 1];  // clamped: used only if in range
    }
  }
  // A key split that starts at or past the request's length has no keys
  // (split 0 always runs: it holds the drafts of the fused launch and the
  // row checks).  Such a workgroup leaves after the first round of small
  // loads instead of the second: launches planned from the longest request
  // hold many of them when lengths vary.
  if constexpr (MODE == kModePrefix || MODE == kModeVerify) {
    if (split != 0 && (int64_t)split * a.split_len >= L_in) return;
  }
  int L = L_in;
  {
    const int cap = a.page_table_stride << a.kv.log2_page;
    if (L > cap) {
      if (threadIdx.x == 0) atomicOr(&g_device_error, kErrLen);
      L = cap;
    }
    if (L < 0) L = 0;
    if constexpr (MODE != kModeNaive && MODE != kModeDraft) {
      // Keys past the planned splits would be neither computed nor merged.
      const int planned = a.n_splits * a.split_len;
      if (L > planned) {
        if (threadIdx.x == 0) atomicOr(&g_device_error, kErrLen);
        L = planned;
      }
    }
  }

  const KvView kv = a.kv;
  const float c2 = a.scale_log2;
  const int64_t head_off = (int64_t)g * kv.head_stride;
  // ---- per-tile building blocks ----------------------------------------

  // A tile's K and V arrive in registers, 16 bytes per lane and load, in one
  // of two shapes, and are written to the wave's LDS stage by (key, chunk):
  //  * row shape (prefix tiles): load n covers keys n*TPI .. +TPI, lane reads
  //    chunk lane % CPR of key n*TPI + lane / CPR -- whole key rows, so a load
  //    reads contiguous runs (one 1 KB run per load for head-major pages);
  //  * fragment shape (draft tiles, whose keys resolve their pages lane by
  //    lane): load kb*KS + ks holds key kb*16 + l16, chunk ks*4 + g4.
  // Prefix tiles start at a multiple of 32 and pages hold >= 16 tokens, so
  // each 16-key half of a tile lies in one page whose id pg[kb] is
  // wave-uniform (-1: no key in that half, or an id outside the pool).  The
  // half's buffer descriptors start at its first key and end after the row
  // of its last valid key, so keys past `end` (and bad pages) read zeros and
  // the loads need no per-lane bounds arithmetic: load n of a lane reads at
  // the fixed byte offset lane_off[n % NV] (key (n*TPI) % 16 + lane / CPR of
  // the half, chunk lane % CPR; rows are token_stride >= head_dim apart).
  constexpr int NV = 16 / TPI;
  int lane_off[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) lane_off[i] = prefix_lane_offset<EB>(kv, i * TPI + lane / CPR, head_off, lane % CPR);
  const int tail_bytes = (int)((head_off + D) * EB);
  auto load_rows = [&](const int (&pg)[2], int base, int end, Raw (&kr)[NI], Raw (&vr)[NI]) {
    __amdgpu_buffer_rsrc_t rk[2], rv[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int first = base + kb * 16;
      const int nvalid = min(max(end - first, 0), 16);
      const HalfSpan h = prefix_half_span(kv, pg[kb], first, nvalid, tail_bytes);
      rk[kb] = half_rsrc(kv.k, h);
      rv[kb] = half_rsrc(kv.v, h);
    }
#pragma unroll
    for (int n = 0; n < NI; ++n) {
      const int kb = (n * TPI) / 16;
      kr[n] = buf_load_chunk(rk[kb], lane_off[n % NV], (Raw*)nullptr);
      vr[n] = buf_load_chunk(rv[kb], lane_off[n % NV], (Raw*)nullptr);
    }
  };
  auto page_id = [&](int id) {  // -1 (and the error flag) for ids outside the pool
    if (id >= kv.num_pages) {
      if (lane == 0) atomicOr(&g_device_error, kErrPage);
    }
    return __builtin_amdgcn_readfirstlane(checked_page(id, kv.num_pages));  // uniform by construction
  };
  auto prefix_pages = [&](int base, int end, int (&pg)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int first = base + kb * 16;
      pg[kb] = page_id(first < end ? pt_row[first >> kv.log2_page] : -1);
    }
  };

  // ---- prefix range of the key loop; its first tile is requested now -----
  int p0 = 0, p1 = 0;
  if constexpr (MODE == kModePrefix || MODE == kModeVerify) {
    p0 = split * a.split_len;
    p1 = min(L, p0 + a.split_len);
    // No keys in this split: no partial (split 0 of a verify launch also
    // holds the draft tiles, so it always writes one).
    if (a.n_splits > 1 && p0 >= L && (MODE == kModePrefix || split != 0)) return;
    if (p1 < p0) p1 = p0;
  } else if constexpr (MODE == kModeNaive) {
    p1 = L;
  }
  const int npt = (p1 - p0 + 31) >> 5;

  // Writes a tile's K and V rows into the wave's stage (row = key, RS stride).
  auto stage = [&](const Raw (&kr)[NI], const Raw (&vr)[NI], bool rows, int ok, uint16_t* st) {
#pragma unroll
    for (int r = 0; r < NI; ++r) {
      int key, ch;
      u32x4 v = widen_bf16(vr[r]);
      if (rows) {
        key = r * TPI + lane / CPR;
        ch = lane % CPR;
      } else {
        key = (r / KS) * 16 + l16;
        ch = (r % KS) * 4 + g4;
        if (!((ok >> (r / KS)) & 1)) v = u32x4{0u, 0u, 0u, 0u};
      }
      *reinterpret_cast<u32x4*>(st + key * RS + ch * 8) = widen_bf16(kr[r]);
      *reinterpret_cast<u32x4*>(st + 32 * RS + key * RS + ch * 8) = v;
    }
  };

  // The first prefix tile goes out now, one round trip of small loads after
  // the start (its block-table entries came with the request's length); Q
  // follows once the branch range has given the rows.
  Raw kr[NI], vr[NI];
  int pg[2] = {-1, -1};
  if (w < npt) {
    if constexpr (MODE == kModePrefix || MODE == kModeVerify) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) pg[kb] = page_id(p0 + w * 32 + kb * 16 < p1 ? pt_first[kb] : -1);
    } else {
      prefix_pages(p0 + w * 32, p1, pg);
    }
    load_rows(pg, p0 + w * 32, p1, kr, vr);
  }

  const int tok0 = cqo[jb];
  const int tok1 = cqo[je];
  // Keeps the length load in the same round trip as the branch-range loads
  // (otherwise it is sunk past the checks below).
  asm volatile("" ::"s"(L_in));
  if (tok0 < 0 || tok1 < tok0 || tok1 > a.total_rows) {
    if (threadIdx.x == 0) atomicOr(&g_device_error, kErrRow);
    return;
  }
  const int ntok = tok1 - tok0;
  const int nrows = ntok * a.group;
  const int row0 = chunk * ROWS;
  if (chunk == 0 && split == 0 && threadIdx.x == 0 && nrows > a.n_chunks * ROWS)
    atomicOr(&g_device_error, kErrRow);  // rows past the planned chunks are not computed
  if (row0 >= nrows) return;
  const int row_end = min(nrows, row0 + ROWS);

  // Segment tokens of this chunk's rows, and the draft keys [dlo, dhi) they
  // can see (dlo, the start of the first row's branch, is set below).
  const int tok_first = row0 / a.group;
  const int tok_last = (row_end - 1) / a.group;
  const int dhi = tok_last + 1;

  // ---- rows of this lane (column l16 of each 16-row block of S^T / O^T) --
  // Recomputed where needed rather than kept live across the key loop.
  auto row_valid = [&](int rb) { return row0 + rb * 16 + l16 < nrows; };
  auto row_tok = [&](int rb) {  // segment token of the row (tok_first for padding rows)
    const int rho = row0 + rb * 16 + l16;
    return rho < nrows ? rho / a.group : tok_first;
  };
  auto row_out = [&](int rb) -> int64_t {  // index of (row, head) in [total_rows, Hq]
    const int rho = row0 + rb * 16 + l16;
    const int t = rho / a.group;
    return (int64_t)(tok0 + t) * a.num_qo_heads + g * a.group + (rho - t * a.group);
  };
  // Per row: its segment token, its branch's first token, and with a draft
  // tree its ancestor mask.
  int rtok[RB] = {}, rbs[RB] = {};
  uint64_t ranc[RB] = {};
  const bool tree = a.draft_mask != nullptr;
  auto load_row_masks = [&]() {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      rtok[rb] = row_tok(rb);
      rbs[rb] = t_rbs[rtok[rb] - tok_first];
      if (tree) ranc[rb] = a.draft_mask[(int64_t)(tok0 + rtok[rb]) * a.draft_mask_words];
    }
  };
  // The window of row block rb's ancestor set for a tile from token `base`
  // on (a one-word set from its register, more words from memory), and the
  // token of the window's first node.
  auto tree_win = [&](int rb, int base, uint64_t& win, int& wbs) {
    const int ws = max(base - rbs[rb], 0);
    win = a.draft_mask_words == 1
              ? tree_window1(ranc[rb], ws)
              : tree_window(a.draft_mask + (int64_t)(tok0 + rtok[rb]) * a.draft_mask_words, a.draft_mask_words, ws);
    wbs = rbs[rb] + ws;
  };

  // ---- Q rows of the chunk (into registers now, into LDS below) ---------
  constexpr int kQChunks = D / 8;
  constexpr int QIT = (ROWS * kQChunks + 255) / 256;
  u32x4 qtmp[kQInLds ? QIT : 1];
  if constexpr (kQInLds) {
#pragma unroll
    for (int it = 0; it < QIT; ++it) {
      const int idx = (int)threadIdx.x + it * 256;
      const int r = idx / kQChunks, c = idx % kQChunks;
      const int rho = row0 + r;
      qtmp[it] = u32x4{0u, 0u, 0u, 0u};
      if (idx < ROWS * kQChunks && rho < nrows) {
        const int t = rho / a.group;
        const int h = g * a.group + (rho - t * a.group);
        qtmp[it] = *reinterpret_cast<const u32x4*>(a.q + (int64_t)(tok0 + t) * a.q_row_stride +
                                                   (int64_t)h * a.q_head_stride + c * 8);
        if constexpr (KV8) {
          if (a.k_cs) qtmp[it] = scale_q_chunk(qtmp[it], a.k_cs + (int64_t)g * D + c * 8);
        }
      }
    }
  }

  // ---- tree tables: their loads go out ahead of the first tile ------------
  // In the fused verify launch only the draft wave (of split 0) reads the
  // tables, so it alone builds them, ordered at wave level; the draft and
  // naive launches build them with the whole workgroup.
  constexpr bool kWaveTables = MODE == kModeVerify;
  constexpr int TNT = kWaveTables ? 64 : 256;       // threads building the tables
  constexpr int TLD = (NBCAP + 1 + TNT - 1) / TNT;  // window entries per thread
  const int nb = je - jb;
  const bool lds_bnd = nb <= NBCAP;
  const int tid = kWaveTables ? lane : (int)threadIdx.x;
  bool builder = kDraftKeys;
  if constexpr (kWaveTables) builder = w == kDraftWave && split == 0;
  int tb_reg[TLD], td_reg[TLD];
  if constexpr (kDraftKeys) {
    if (builder && lds_bnd) {
#pragma unroll
      for (int i = 0; i < TLD; ++i) {
        const int t = tid + i * TNT;
        tb_reg[i] = t <= nb ? qo[jb + t] : 0;
        td_reg[i] = t < nb && a.draft_start ? a.draft_start[jb + t] : 0;
      }
    }
  }

  // ---- tree tables ---------------------------------------------------------
  // t_bnd / t_dst: branch_qo_indptr[jb .. je] and draft_start[jb .. je) of the
  // segment's branches; t_rbs: branch start of each token of the chunk;
  // t_doff: element offset (head excluded) of draft key dlo + t, -1 when its
  // slot lies past its draft block-table row or its page outside the pool.
  int dlo = 0;
  auto branch_at = [&](int x) -> int {  // local branch index of segment token x
    if (lds_bnd) {
      int lo = 0, hi = nb - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (t_bnd[mid] - tok0 <= x) lo = mid; else hi = mid - 1;
      }
      return lo;
    }
    return branch_of_row(qo, jb, je, tok0 + x) - jb;
  };
  auto branch_start = [&](int jl) { return (lds_bnd ? t_bnd[jl] : qo[jb + jl]) - tok0; };
  auto branch_dstart = [&](int jl) {
    return lds_bnd ? t_dst[jl] : (a.draft_start ? a.draft_start[jb + jl] : 0);
  };
  if constexpr (kDraftKeys) {
    if (builder && lds_bnd) {
#pragma unroll
      for (int i = 0; i < TLD; ++i) {
        const int t = tid + i * TNT;
        if (t <= nb) t_bnd[t] = tb_reg[i];
        if (t < nb) t_dst[t] = td_reg[i];
      }
    }
    if constexpr (kWaveTables) {
      wave_lds_sync();
    } else {
      __syncthreads();
    }
    if (builder) {
      dlo = __builtin_amdgcn_readfirstlane(branch_start(branch_at(tok_first)));
      for (int t = tid; t <= tok_last - tok_first; t += TNT) t_rbs[t] = branch_start(branch_at(tok_first + t));
      const int nk = min(dhi - dlo, KEYCAP);
      const int dstride = a.draft_page_table_stride;
      for (int t = tid; t < nk; t += TNT) {
        const int x = dlo + t;
        const int jl = branch_at(x);
        const int slot = branch_dstart(jl) + (x - branch_start(jl));
        t_doff[t] = draft_slot_offset(kv, a.draft_page_table + (int64_t)(jb + jl) * dstride, dstride, slot);
      }
    }
    if constexpr (kWaveTables) wave_lds_sync();  // t_rbs and t_doff before the draft wave reads them
  }
  if constexpr (kQInLds) {
#pragma unroll
    for (int it = 0; it < QIT; ++it) {
      const int idx = (int)threadIdx.x + it * 256;
      if (idx < ROWS * kQChunks)
        *reinterpret_cast<u32x4*>(qs + (idx / kQChunks) * QSTR + (idx % kQChunks) * 8) = qtmp[it];
    }
  }
  if constexpr (kQInLds || (kDraftKeys && !kWaveTables)) __syncthreads();

  // Q B-fragments: lane holds row rb*16 + l16, channels ks*32 + g4*8 .. +8.
  bf16x8 qf[kQInLds ? 1 : RB][KS];
  if constexpr (!kQInLds) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int rho = row0 + rb * 16 + l16;
      const int t = row_tok(rb);
      const uint16_t* qp = a.q + (int64_t)(tok0 + t) * a.q_row_stride +
                           (int64_t)(g * a.group + (rho - t * a.group)) * a.q_head_stride + g4 * 8;
      const bool ok = row_valid(rb);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        qf[rb][ks] = ok ? *reinterpret_cast<const bf16x8*>(qp + ks * 32) : bf16x8{};
        if constexpr (KV8) {
          if (a.k_cs)
            qf[rb][ks] = __builtin_bit_cast(
                bf16x8, scale_q_chunk(__builtin_bit_cast(u32x4, qf[rb][ks]), a.k_cs + (int64_t)g * D + ks * 32 + g4 * 8));
        }
      }
    }
  }
  auto qfrag = [&](int rb, int ks) -> bf16x8 {
    if constexpr (kQInLds) {
      return *reinterpret_cast<const bf16x8*>(qs + (rb * 16 + l16) * QSTR + ks * 32 + g4 * 8);
    } else {
      return qf[rb][ks];
    }
  };

  // Draft tiles: keys are segment tokens [base, base+32); off[kb] is the
  // offset of key base + kb*16 + l16 (-2: no key, -1: bad slot or page).
  auto draft_offsets = [&](int base, int end, int64_t (&off)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = base + kb * 16 + l16;
      int64_t o = -2;
      if (key < end) {
        if (key - dlo < KEYCAP) {
          o = t_doff[key - dlo];
          if (o >= 0) o += head_off;
        } else {
          o = draft_offset(kv, qo, a.draft_page_table, a.draft_page_table_stride, a.draft_start, jb, je,
                           key, g);
        }
        if (o == -1) atomicOr(&g_device_error, kErrPage);
      }
      off[kb] = o;
    }
  };
  // Lanes without a key load nothing (all such lanes of all workgroups would
  // otherwise hit one row) and hold zeros; their K is masked later and their
  // V is zero (bit kb of `ok` also zeroes it when staged).
  const int64_t last_row = pool_last_row(kv, a.num_kv_heads);
  auto load_draft_at = [&](const int64_t (&off)[2], Raw (&kr)[NI], Raw (&vr)[NI], int& ok) {
    ok = 0;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bool valid = off[kb] >= 0;
      ok |= valid ? (1 << kb) : 0;
      if (valid) {
        const int64_t o2 = clamp_row(off[kb], last_row) + g4 * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          kr[kb * KS + ks] = load_key_chunk<Raw, EB>(kv.k, o2 + ks * 32);
          vr[kb * KS + ks] = load_key_chunk<Raw, EB>(kv.v, o2 + ks * 32);
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          kr[kb * KS + ks] = Raw{};
          vr[kb * KS + ks] = Raw{};
        }
      }
    }
  };
  auto load_draft = [&](int base, int end, Raw (&kr)[NI], Raw (&vr)[NI], int& ok) {
    int64_t off[2];
    draft_offsets(base, end, off);
    load_draft_at(off, kr, vr, ok);
  };


  // S^T for one tile: s[rb][kb] holds keys kb*16 + 4*g4 + i of row rb*16 + l16.
  auto kfrag = [&](const uint16_t* st, int kb, int ks) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(st + (kb * 16 + l16) * RS + (ks * 4 + g4) * 8);
  };
  auto scores = [&](const uint16_t* st, f32x4 (&s)[RB][2]) {
    bf16x8 kf[2][KS];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kf[kb][ks] = kfrag(st, kb, ks);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) acc = mfma16(kf[kb][ks], qfrag(rb, ks), acc);
        s[rb][kb] = acc;
      }
    }
    // Copy the scores out of the MFMA destinations here, in the block that
    // issued the MFMAs, so that every read of them is ordered behind the
    // required MFMA wait states even when a branch follows.
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) asm volatile("" : "+v"(s[rb][kb]));
  };

  // Prefix keys: only the bound `end`.  Key base + kb*16 + g4*4 + i is kept
  // iff g4*4 < end - base - kb*16 - i: a uniform bound per key, so no key
  // index is formed per lane.
  auto mask_prefix = [&](int base, int end, f32x4 (&s)[RB][2]) {
    const int n = end - base;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) s[rb][kb][i] = g4 * 4 < n - (kb * 16 + i) ? s[rb][kb][i] : kNegInf;
  };
  // Draft keys: the bound `end` and the in-branch ancestor rule (rtok / rbs
  // must have been loaded by load_row_masks).
  auto mask_draft = [&](int base, int end, f32x4 (&s)[RB][2]) {
    // One uniform branch per tile picks the rule (tree masks or chains).
    if (tree) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        uint64_t win;
        int wbs;
        tree_win(rb, base, win, wbs);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = base + kb * 16 + g4 * 4 + i;
            const bool vis = (key < end) & draft_visible_tree(win, wbs, key);
            s[rb][kb][i] = vis ? s[rb][kb][i] : kNegInf;
          }
        }
      }
    } else {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = base + kb * 16 + g4 * 4 + i;
            const bool vis = (key < end) & draft_visible(rtok[rb], rbs[rb], key);
            s[rb][kb][i] = vis ? s[rb][kb][i] : kNegInf;
          }
        }
      }
    }
  };

  // Online softmax update in base 2.  m is the carried max (raised only past
  // the slack), l the lane's partial row sum (its 8 keys of each tile, fp32),
  // alpha the factor the accumulator must be scaled by, pf the weights as P^T
  // B-fragments.  Returns whether this lane needs a rescale.
  // A row's max only moves when the max over its 32 keys exceeds m + slack;
  // each lane checks its own 8 keys first, and only when some lane of the
  // wave finds such a key are the row maxima formed across lanes.
  // First half: the carried max and alpha.
  auto softmax_max = [&](const f32x4 (&s)[RB][2], float (&m)[RB], float (&alpha)[RB]) -> bool {
    float lm[RB];
    bool raise = false;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      lm[rb] = fmaxf(fmaxf(fmaxf(s[rb][0][0], s[rb][0][1]), fmaxf(s[rb][0][2], s[rb][0][3])),
                     fmaxf(fmaxf(s[rb][1][0], s[rb][1][1]), fmaxf(s[rb][1][2], s[rb][1][3])));
      raise |= lm[rb] * c2 > m[rb] + kMaxSlack;
    }
    bool rescale = false;
    if (__any(raise)) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const float mx = rowgroup_max(lm[rb]) * c2;
        const float mold = m[rb];
        const float mnew = mx > mold + kMaxSlack ? mx : mold;
        const float ms = mnew == kNegInf ? 0.f : mnew;
        alpha[rb] = mnew == mold ? 1.f : fast_exp2(mold - ms);
        rescale |= mnew != mold && mold != kNegInf;
        m[rb] = mnew;
      }
    } else {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) alpha[rb] = 1.f;
    }
    return rescale;
  };
  // Second half: the weights as P^T fragments and the row sums (straight-line
  // VALU code, so that matrix instructions can be interleaved with it).
  auto softmax_exp = [&](const f32x4 (&s)[RB][2], const float (&m)[RB], float (&l)[RB],
                         const float (&alpha)[RB], bf16x8 (&pf)[RB]) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float ms = m[rb] == kNegInf ? 0.f : m[rb];
      float p[8];
      float sum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[kb * 4 + i] = fast_exp2(s[rb][kb][i] * c2 - ms);
          sum += p[kb * 4 + i];
        }
      }
      l[rb] = l[rb] * alpha[rb] + sum;
      const u32x4 pk = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                        pack_bf16x2(p[6], p[7])};
      pf[rb] = __builtin_bit_cast(bf16x8, pk);
    }
  };
  auto softmax = [&](const f32x4 (&s)[RB][2], float (&m)[RB], float (&l)[RB], float (&alpha)[RB],
                     bf16x8 (&pf)[RB]) -> bool {
    const bool rescale = softmax_max(s, m, alpha);
    softmax_exp(s, m, l, alpha, pf);
    return rescale;
  };

  // V^T A-fragment of channel block db: lane holds channel db*16 + l16 of keys
  // kb*16 + 4*g4 + j (k slot kb*4 + j), the key order of P^T.  Lane a of each
  // 16-lane group addresses key row 4*g4 + a/4, channels db*16 + 4*(a%4) ..+4;
  // the transposing read hands lane l16 element l16%4 of lanes l16/4 + 4j.
  auto vt_frag = [&](const uint16_t* st, int db) -> bf16x8 {
    const uint16_t* vb = st + 32 * RS + (4 * g4 + (l16 >> 2)) * RS + db * 16 + 4 * (l16 & 3);
    const i16x4 lo = lds_read_tr16(vb);
    const i16x4 hi = lds_read_tr16(vb + 16 * RS);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // Merged pass state of this lane's rows for the channel blocks this wave
  // owns: acc[rb][dbl] normalised output, lse2[rb] base-2 LSE.
  f32x4 acc[RB][DBW];
  float lse2[RB];

  int d0 = 0, d1 = 0;
  if constexpr (MODE == kModeDraft || MODE == kModeNaive) {
    d0 = dlo;
    d1 = dhi;
  }
  const int ndt = (d1 - d0 + 31) >> 5;
  const int nt = npt + ndt;
  if constexpr (MODE == kModeDraft || MODE == kModeNaive) load_row_masks();

  float m[RB], l[RB];
  f32x4 o[RB][DB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m[rb] = kNegInf;
    l[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  uint16_t* st = reinterpret_cast<uint16_t*>(smem) + w * STAGE;

  // Tile tau covers prefix keys p0 + 32*tau .. for tau < npt, then draft
  // tokens d0 + 32*(tau - npt) .. .  pg always holds the pages of the next
  // prefix tile to be loaded.
  auto pages_of = [&](int tau, int (&pg)[2]) {
    if (tau < npt) {
      prefix_pages(p0 + tau * 32, p1, pg);
    } else {
      pg[0] = -1;
      pg[1] = -1;
    }
  };
  int ok = 3;
  auto issue = [&](int tau) {
    if (tau < npt) {
      load_rows(pg, p0 + tau * 32, p1, kr, vr);
      ok = 3;
    } else {
      load_draft(d0 + (tau - npt) * 32, d1, kr, vr, ok);
    }
  };
  // Prefix-only launches (pass A, verify) prefetch without branches: past the
  // wave's last tile the "next" tile is the current one again (L2-resident,
  // never used), so the load sequence and its wait counts are the same every
  // iteration.
  constexpr bool kPrefixOnly = MODE == kModePrefix || MODE == kModeVerify;
  if (w < nt) {
    if (w >= npt) issue(w);  // a draft tile (prefix tiles were requested above)
    pages_of(w + 4 < nt ? w + 4 : w, pg);
  }
  // The draft wave of a verify launch: its first draft tile is requested in
  // place of the prefetch past its last prefix tile.
  const bool verify_drafts = MODE == kModeVerify && split == 0 && dlo < dhi && w == kDraftWave;
  if (verify_drafts && w >= nt) load_draft(dlo, dhi, kr, vr, ok);
  // Each tile's P·V is issued one iteration late, in one block with the
  // next tile's softmax exponentials, so that the matrix pipe works through
  // it while the VALU computes the weights (one wave per SIMD has no other
  // wave to overlap with).  The deferred tile keeps its P^T fragments, its
  // V^T fragments (read out of the stage before the stage is overwritten)
  // and the rescale the following softmax asks for; the rescale is applied
  // before that tile's P·V, since its P is relative to the raised max.
  // Before the first tile the deferred operands are zeros: an exact no-op.
  bf16x8 pv_p[RB], pv_v[DB];
  float pv_alpha[RB];
  bool pv_rescale = false;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) pv_p[rb] = bf16x8{};
  auto rescale_o = [&](const float (&alpha)[RB]) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int db = 0; db < DB; ++db) o[rb][db] *= alpha[rb];
  };
  for (int tau = w; tau < nt; tau += 4) {
    const int nxt = tau + 4;
    const bool is_prefix = tau < npt;
    const int base = is_prefix ? p0 + tau * 32 : d0 + (tau - npt) * 32;
    const int end = is_prefix ? p1 : d1;
    // V of the deferred tile leaves the stage (zeros before the first tile).
    const bool first = tau == w;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const bf16x8 vf = vt_frag(st, db);
      pv_v[db] = first ? bf16x8{} : vf;
    }
    // Stage this tile, then reuse its registers for the next tile's loads,
    // which then have a whole iteration to land.
    stage(kr, vr, is_prefix, ok, st);
    if constexpr (kPrefixOnly) {
      if (verify_drafts && nxt >= nt) {
        load_draft(dlo, dhi, kr, vr, ok);
      } else {
        const int ld = nxt < nt ? nxt : tau;
        load_rows(pg, p0 + ld * 32, p1, kr, vr);
        pages_of(nxt + 4 < nt ? nxt + 4 : ld, pg);
      }
    } else {
      if (nxt < nt) issue(nxt);
      if (nxt + 4 < nt) pages_of(nxt + 4, pg);
    }
    if (pv_rescale) rescale_o(pv_alpha);
    f32x4 s[RB][2];
    scores(st, s);
    if (!is_prefix) {
      mask_draft(base, end, s);
    } else if (base + 32 > end) {
      mask_prefix(base, end, s);
    }
    float alpha[RB];
    const bool resc = __any(softmax_max(s, m, alpha));
    bf16x8 pf[RB];
    softmax_exp(s, m, l, alpha, pf);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) o[rb][db] = mfma16(pv_v[db], pv_p[rb], o[rb][db]);
    // The compiler interleaves these matrix instructions with the VALU
    // work around them: fixed patterns of one MFMA per 2, 3 or 5 VALU
    // instructions measured 1-2 % slower on the verify kernel.
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      pv_p[rb] = pf[rb];
      pv_alpha[rb] = alpha[rb];
    }
    pv_rescale = resc;
  }
  // The last tile's P·V (its V is still in the stage).
  if (w < nt) {
    mfma_drain();
    if (pv_rescale) rescale_o(pv_alpha);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const bf16x8 vf = vt_frag(st, db);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) o[rb][db] = mfma16(vf, pv_p[rb], o[rb][db]);
    }
    mfma_drain();
  }
  if (verify_drafts) {
    // Pass B of the chunk's rows into this wave's state: its visible draft
    // tiles (usually one), under the in-branch ancestor mask.
    load_row_masks();
    for (int base = dlo; base < dhi; base += 32) {
      if (base != dlo) load_draft(base, dhi, kr, vr, ok);
      stage(kr, vr, false, ok, st);
      f32x4 s[RB][2];
      scores(st, s);
      mask_draft(base, dhi, s);
      float alpha[RB];
      bf16x8 pf[RB];
      if (__any(softmax(s, m, l, alpha, pf))) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int db = 0; db < DB; ++db) o[rb][db] *= alpha[rb];
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16x8 vf = vt_frag(st, db);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) o[rb][db] = mfma16(vf, pf[rb], o[rb][db]);
      }
    }
  }

  mfma_drain();

  // ---- merge the four waves' states (LSE identity) ----------------------
  // Each wave publishes its rows' (m, l); after the barrier (which also ends
  // every wave's use of its stage) it sends its unscaled O blocks to their
  // owners and forms the merge weights of its rows; after the second barrier
  // owner ow of channel blocks [ow*DBW, ow*DBW + DBW) sums the four waves'
  // blocks, each times its weight 2^(m_w - M) / sum_w' l_w' 2^(m_w' - M).
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) l[rb] = rowgroup_sum(l[rb]);
  if (g4 == 0) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      ml[(w * ROWS + rb * 16 + l16) * 2 + 0] = m[rb];
      ml[(w * ROWS + rb * 16 + l16) * 2 + 1] = l[rb];
    }
  }
  __syncthreads();
  float* xbuf = reinterpret_cast<float*>(smem);
  auto slot = [](int owner, int src) { return owner * 3 + (src < owner ? src : src - 1); };
#pragma unroll
  for (int ow = 0; ow < 4; ++ow) {
    if (ow == w) continue;
    float* dst = xbuf + slot(ow, w) * XSLOT;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int dbl = 0; dbl < DBW; ++dbl)
        *reinterpret_cast<f32x4*>(dst + ((rb * DBW + dbl) * 64 + lane) * 4) = o[rb][ow * DBW + dbl];
  }
  float wt[RB][4];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = rb * 16 + l16;
    float mw[4], lw[4];
#pragma unroll
    for (int w2 = 0; w2 < 4; ++w2) {
      mw[w2] = ml[(w2 * ROWS + r) * 2];
      lw[w2] = ml[(w2 * ROWS + r) * 2 + 1];
    }
    const float M = fmaxf(fmaxf(mw[0], mw[1]), fmaxf(mw[2], mw[3]));
    const float ms = M == kNegInf ? 0.f : M;
    float e[4], tot = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < 4; ++w2) {
      e[w2] = fast_exp2(mw[w2] - ms);
      tot += lw[w2] * e[w2];
    }
    // FP8 pools: the V scale multiplies every normalised output once, here.
    const float inv = tot > 0.f ? (KV8 ? a.v_scale : 1.f) / tot : 0.f;
#pragma unroll
    for (int w2 = 0; w2 < 4; ++w2) wt[rb][w2] = e[w2] * inv;
    lse2[rb] = tot > 0.f ? M + fast_log2(tot) : kNegInf;
  }
  __syncthreads();
  // The owner's own blocks stay in registers: one specialisation per wave
  // index (a uniform branch), so no block is selected lane by lane.
  auto combine = [&](auto owner) {
    constexpr int OW = decltype(owner)::value;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int dbl = 0; dbl < DBW; ++dbl) {
        f32x4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) {
          const f32x4 x = w2 == OW ? o[rb][OW * DBW + dbl]
                                   : *reinterpret_cast<const f32x4*>(
                                         xbuf + slot(OW, w2) * XSLOT + ((rb * DBW + dbl) * 64 + lane) * 4);
#pragma unroll
          for (int i = 0; i < 4; ++i) sum[i] = fmaf(wt[rb][w2], x[i], sum[i]);
        }
        acc[rb][dbl] = sum;
      }
    }
  };
  switch (w) {
    case 0: combine(WaveIndex<0>{}); break;
    case 1: combine(WaveIndex<1>{}); break;
    case 2: combine(WaveIndex<2>{}); break;
    default: combine(WaveIndex<3>{}); break;
  }

  // Split prefix passes stop at a partial state; everything else is final,
  // including a request whose keys all fall in split 0 (the split merge
  // leaves its rows alone).
  bool partial = false;
  if constexpr (MODE == kModePrefix || MODE == kModeVerify) partial = a.n_splits > 1 && L > a.split_len;

  // ---- output ----------------------------------------------------------------
  // Row addresses and values are formed first and the stores issued back to
  // back, one uniform branch per output kind: no store waits for an earlier
  // one to release its registers.
  const int64_t plane = (int64_t)a.total_rows * a.num_qo_heads;
  int64_t orow[RB];
  bool rv[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    rv[rb] = row_valid(rb);
    orow[rb] = rv[rb] ? row_out(rb) : 0;
  }
  const int cw = w * DBW * 16 + g4 * 4;  // first channel of this lane's blocks
  if constexpr (KV8) {
    // Per-channel V scales multiply each normalised output channel.
    if (a.v_cs) {
#pragma unroll
      for (int dbl = 0; dbl < DBW; ++dbl) {
        const f32x4 vs = *reinterpret_cast<const f32x4*>(a.v_cs + (int64_t)g * D + cw + dbl * 16);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) acc[rb][dbl] *= vs;
      }
    }
  }
  if (partial) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if (!rv[rb]) continue;
      float* dst = a.ws_o + (split * plane + orow[rb]) * D + cw;
#pragma unroll
      for (int dbl = 0; dbl < DBW; ++dbl) *reinterpret_cast<f32x4*>(dst + dbl * 16) = acc[rb][dbl];
      if (w == 0 && g4 == 0) a.ws_lse[split * plane + orow[rb]] = lse2[rb];
    }
    return;
  }
  if (a.o_bf16) {
    u32x2 pk[RB][DBW];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int dbl = 0; dbl < DBW; ++dbl)
        pk[rb][dbl] = u32x2{pack_bf16x2(acc[rb][dbl][0], acc[rb][dbl][1]),
                            pack_bf16x2(acc[rb][dbl][2], acc[rb][dbl][3])};
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if (!rv[rb]) continue;
      uint16_t* dst = reinterpret_cast<uint16_t*>(a.o) + orow[rb] * D + cw;
#pragma unroll
      for (int dbl = 0; dbl < DBW; ++dbl) *reinterpret_cast<u32x2*>(dst + dbl * 16) = pk[rb][dbl];
    }
  } else {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if (!rv[rb]) continue;
      float* dst = reinterpret_cast<float*>(a.o) + orow[rb] * D + cw;
#pragma unroll
      for (int dbl = 0; dbl < DBW; ++dbl) *reinterpret_cast<f32x4*>(dst + dbl * 16) = acc[rb][dbl];
    }
  }
  if (w == 0 && g4 == 0 && a.lse) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
      if (rv[rb]) a.lse[orow[rb]] = lse2[rb] * kLn2;
  }
}

}  // namespace casc
