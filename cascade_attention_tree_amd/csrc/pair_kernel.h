// Paged attention kernel of pass A and the fused verify pass for requests
// with few query rows per kv head (head_dim 128, bf16 or FP8 E4M3 pools):
// two workgroups per CU.
//
// A (request, kv head) item's rows -- the request's query tokens times the
// query heads that share kv head g (GQA) -- are cut into n_chunks chunks of
// at most 16*RB rows, one workgroup of 4 waves each.  The chunks of an item
// are dispatched one after another to the same XCD, so they stream the
// item's prefix pages in step and the second read of every K/V tile is
// served by that XCD's L2: HBM still sees each page about once.  Small row
// chunks keep a wave's state (RB 16-row blocks of O, 96 registers at RB 3)
// small enough for two waves per SIMD, so one wave's softmax and loads run
// in the gaps of the other's dependent chain.
//
// Inside the workgroup every wave keeps all rows of the chunk and takes every
// 4th 32-key tile.  Per tile a wave
//   * loads K straight into MFMA A-fragments (lane l16 + 16 g4 reads the
//     16 bytes of key kb*16 + l16, channels ks*32 + g4*8 .. +8: S^T = K Q^T
//     contracts over channels, which lie contiguous in a key row), and V in
//     whole rows, one tile ahead, through per-half-page buffer descriptors;
//   * writes V into its LDS stage and reads it back transposed
//     (ds_read_b64_tr_b16) as the A-fragments of O^T += V^T P^T;
//   * keeps Q in LDS (B-fragments, read per tile) and a base-2 online softmax
//     per row with a slack on the carried max.
// Wave 3, which has the fewest prefix tiles, takes the request's visible
// draft tiles after its prefix tiles, under the in-branch ancestor mask, into
// its own state (pass B).  The four waves then merge their states with the
// LSE identity (cascade page, splittability of standard attention), which
// also merges pass A with pass B.
#pragma once

#include "attn_kernel.h"

namespace casc {

// 16-row MFMA blocks per chunk of the pair kernel.
constexpr int kPairRowBlocks = kPairRows / 16;

template <int RB, int MODE, bool KV8>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
pair_kernel(const AttnArgs a) {
  static_assert(MODE == kModePrefix || MODE == kModeVerify, "pass A or the fused verify pass");
  constexpr int D = 128;
  constexpr int KS = D / 32;     // k-steps of the Q K^T contraction
  constexpr int DB = D / 16;     // 16-channel blocks of the head dim
  constexpr int DBW = DB / 4;    // blocks each wave owns after the merge
  constexpr int ROWS = RB * 16;
  constexpr int CPR = D / 8;     // 8-channel chunks per key row
  constexpr int TPI = 64 / CPR;  // key rows covered by one row-shaped load
  constexpr int NL = 2 * KS;     // loads of 16 (bf16) or 8 (FP8) bytes per lane for a tile's K, and V
  constexpr int EB = KV8 ? 1 : 2;
  typedef typename KvChunk<KV8>::T Raw;
  constexpr int RS = D + 16;  // V stage row stride (bf16): rows 8 banks apart
  constexpr int VSTAGE = 32 * RS;
  constexpr int VBYTES = 4 * VSTAGE * 2;
  constexpr int XSLOT = RB * DBW * 64 * 4;  // floats one wave sends to one owner
  constexpr int XBYTES = 4 * XSLOT * 4;     // one exchange round: a slot per owner
  constexpr int UNION = VBYTES > XBYTES ? VBYTES : XBYTES;
  constexpr int QSTR = D + 8;  // Q rows land 4 banks apart
  constexpr int QBYTES = ROWS * QSTR * 2;
  constexpr int MLBYTES = 4 * ROWS * 2 * 4;
  constexpr bool kVerify = MODE == kModeVerify;
  constexpr int NBCAP = 128;   // branches of a request resolved in LDS
  constexpr int KEYCAP = 512;  // draft keys of a chunk resolved in LDS
  constexpr int TBYTES = kVerify ? KEYCAP * 8 + ((2 * NBCAP + 1 + ROWS) * 4 + 15) / 16 * 16 : 0;
  constexpr int kDraftWave = 3;

  __shared__ __attribute__((aligned(16))) unsigned char smem[UNION + QBYTES + MLBYTES + TBYTES];
  uint16_t* qs = reinterpret_cast<uint16_t*>(smem + UNION);                 // [ROWS][QSTR]
  float* ml = reinterpret_cast<float*>(smem + UNION + QBYTES);              // [4][ROWS][m, l]
  int64_t* t_doff = reinterpret_cast<int64_t*>(smem + UNION + QBYTES + MLBYTES);  // [KEYCAP]
  int* t_bnd = reinterpret_cast<int*>(t_doff + KEYCAP);  // [NBCAP + 1]
  int* t_dst = t_bnd + NBCAP + 1;                        // [NBCAP]
  int* t_rbs = t_dst + NBCAP;                            // [ROWS]

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15;
  const int g4 = lane >> 4;

  // ---- work item ------------------------------------------------------------
  // Key splits vary slowest.  Within a split, workgroup u goes to XCD u % 8
  // (round-robin dispatch); u / 8 walks the chunks of one item, then the next
  // item of that XCD, so an item's chunks run side by side on one L2.
  const int n_items = a.batch_size * a.num_kv_heads;
  const int per_split = (int)gridDim.x / a.grid_splits;
  const int split = (int)blockIdx.x / per_split;
  const int u = (int)blockIdx.x - split * per_split;
  const int v8 = u >> 3;
  const int chunk = v8 % a.n_chunks;
  const int item = (v8 / a.n_chunks) * 8 + (u & 7);
  if (item >= n_items) return;
  const int g = item % a.num_kv_heads;
  const int req = item / a.num_kv_heads;

  cint32* cqo = as_const(a.branch_qo_indptr);
  cint32* crb = as_const(a.req_branch_indptr);
  const int jb = crb[req];
  const int je = crb[req + 1];
  const int L_in = as_const(a.cache_seqlens)[req];
  cint32* pt_row = as_const(a.page_table + (int64_t)req * a.page_table_stride);
  int pt_first[2] = {-1, -1};
  {
    const int stride = a.page_table_stride;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int idx = (split * a.split_len + w * 32 + kb * 16) >> a.kv.log2_page;
      if (stride > 0) pt_first[kb] = pt_row[idx < stride ? idx : stride - 1];  // used only if in range
    }
  }
  // A key split at or past the request's length has no keys (split 0 always
  // runs: it holds the drafts of the fused launch and the row checks).
  if (split != 0 && (int64_t)split * a.split_len >= L_in) return;
  const int tok0 = cqo[jb];
  const int tok1 = cqo[je];
  asm volatile("" ::"s"(L_in));
  if (tok0 < 0 || tok1 < tok0 || tok1 > a.total_rows) {
    if (threadIdx.x == 0) atomicOr(&g_device_error, kErrRow);
    return;
  }
  const int nrows = (tok1 - tok0) * a.group;
  const int row0 = chunk * a.chunk_rows;
  if (chunk == 0 && split == 0 && threadIdx.x == 0 && nrows > a.n_chunks * a.chunk_rows)
    atomicOr(&g_device_error, kErrRow);  // rows past the planned chunks are not computed
  if (row0 >= nrows) return;
  const int row_end = min(nrows, row0 + a.chunk_rows);

  int L = L_in;
  {
    const int cap = a.page_table_stride << a.kv.log2_page;
    if (L > cap) {
      if (threadIdx.x == 0) atomicOr(&g_device_error, kErrLen);
      L = cap;
    }
    if (L < 0) L = 0;
    const int planned = a.n_splits * a.split_len;
    if (L > planned) {
      if (threadIdx.x == 0) atomicOr(&g_device_error, kErrLen);
      L = planned;
    }
  }

  const KvView kv = a.kv;
  const float c2 = a.scale_log2;
  const int64_t head_off = (int64_t)g * kv.head_stride;
  const int tok_first = row0 / a.group;
  const int tok_last = (row_end - 1) / a.group;
  const int dhi = tok_last + 1;

  auto row_valid = [&](int rb) { return row0 + rb * 16 + l16 < row_end; };
  auto row_tok = [&](int rb) {
    const int rho = row0 + rb * 16 + l16;
    return rho < row_end ? rho / a.group : tok_first;
  };
  auto row_out = [&](int rb) -> int64_t {
    const int rho = row0 + rb * 16 + l16;
    const int t = rho / a.group;
    return (int64_t)(tok0 + t) * a.num_qo_heads + g * a.group + (rho - t * a.group);
  };

  // ---- loads ------------------------------------------------------------------
  // V, row shape: load n covers keys n*TPI .. +TPI of the tile, lane reads
  // chunk lane % CPR of key n*TPI + lane / CPR (whole key rows).
  // K, fragment shape: load kb*KS + ks holds chunk ks*4 + g4 of key kb*16 + l16.
  int voff[16 / TPI];
#pragma unroll
  for (int i = 0; i < 16 / TPI; ++i) voff[i] = prefix_lane_offset<EB>(kv, i * TPI + lane / CPR, head_off, lane % CPR);
  const int koff = prefix_lane_offset<EB>(kv, l16, head_off, g4);
  // The two halves' spans of a tile (one per 16 keys), shared by its K and V.
  const int tail_bytes = (int)((head_off + D) * EB);
  auto spans = [&](const int (&pg)[2], int base, int end, HalfSpan (&hs)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int first = base + kb * 16;
      hs[kb] = prefix_half_span(kv, pg[kb], first, min(max(end - first, 0), 16), tail_bytes);
    }
  };
  auto load_v = [&](const HalfSpan (&hs)[2], Raw (&vr)[NL]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const __amdgpu_buffer_rsrc_t r = half_rsrc(kv.v, hs[kb]);
#pragma unroll
      for (int i = 0; i < 16 / TPI; ++i) vr[kb * (16 / TPI) + i] = buf_load_chunk(r, voff[i], (Raw*)nullptr);
    }
  };
  auto load_k = [&](const HalfSpan (&hs)[2], Raw (&kr)[NL]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const __amdgpu_buffer_rsrc_t r = half_rsrc(kv.k, hs[kb]);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kr[kb * KS + ks] = buf_load_chunk(r, koff + ks * 32 * EB, (Raw*)nullptr);
    }
  };
  auto page_id = [&](int id) {  // -1 (and the error flag) for ids outside the pool
    if (id >= kv.num_pages) {
      if (lane == 0) atomicOr(&g_device_error, kErrPage);
    }
    return __builtin_amdgcn_readfirstlane(checked_page(id, kv.num_pages));
  };

  // ---- prefix range of this split; the first tile is requested now ---------
  int p0 = split * a.split_len;
  int p1 = min(L, p0 + a.split_len);
  if (a.n_splits > 1 && p0 >= L && (MODE == kModePrefix || split != 0)) return;
  if (p1 < p0) p1 = p0;
  const int npt = (p1 - p0 + 31) >> 5;

  // ---- Q rows of the chunk (registers now, LDS below) -----------------------
  constexpr int QIT = (ROWS * CPR + 255) / 256;
  u32x4 qtmp[QIT];
#pragma unroll
  for (int it = 0; it < QIT; ++it) {
    const int idx = (int)threadIdx.x + it * 256;
    const int r = idx / CPR, c = idx % CPR;
    const int rho = row0 + r;
    qtmp[it] = u32x4{0u, 0u, 0u, 0u};
    if (idx < ROWS * CPR && rho < row_end) {
      const int t = rho / a.group;
      const int h = g * a.group + (rho - t * a.group);
      qtmp[it] = *reinterpret_cast<const u32x4*>(a.q + (int64_t)(tok0 + t) * a.q_row_stride +
                                                 (int64_t)h * a.q_head_stride + c * 8);
      if constexpr (KV8) {
        if (a.k_cs) qtmp[it] = scale_q_chunk(qtmp[it], a.k_cs + (int64_t)g * D + c * 8);
      }
    }
  }

  // ---- tree tables (fused verify, split 0): built by the draft wave alone ---
  const int nb = je - jb;
  const bool lds_bnd = nb <= NBCAP;
  const bool builder = kVerify && w == kDraftWave && split == 0;
  constexpr int TLD = (NBCAP + 1 + 63) / 64;
  int tb_reg[TLD], td_reg[TLD];
  if constexpr (kVerify) {
    if (builder && lds_bnd) {
#pragma unroll
      for (int i = 0; i < TLD; ++i) {
        const int t = lane + i * 64;
        tb_reg[i] = t <= nb ? a.branch_qo_indptr[jb + t] : 0;
        td_reg[i] = t < nb && a.draft_start ? a.draft_start[jb + t] : 0;
      }
    }
  }

  Raw kr[NL], vr[NL];
  int pg[2] = {-1, -1};
  HalfSpan hs[2];
  if (w < npt) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) pg[kb] = page_id(p0 + w * 32 + kb * 16 < p1 ? pt_first[kb] : -1);
    spans(pg, p0 + w * 32, p1, hs);
    load_v(hs, vr);
    load_k(hs, kr);
  }

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
    return branch_of_row(a.branch_qo_indptr, jb, je, tok0 + x) - jb;
  };
  auto branch_start = [&](int jl) { return (lds_bnd ? t_bnd[jl] : a.branch_qo_indptr[jb + jl]) - tok0; };
  auto branch_dstart = [&](int jl) {
    return lds_bnd ? t_dst[jl] : (a.draft_start ? a.draft_start[jb + jl] : 0);
  };
  if constexpr (kVerify) {
    if (builder) {
      if (lds_bnd) {
#pragma unroll
        for (int i = 0; i < TLD; ++i) {
          const int t = lane + i * 64;
          if (t <= nb) t_bnd[t] = tb_reg[i];
          if (t < nb) t_dst[t] = td_reg[i];
        }
      }
      wave_lds_sync();
      dlo = __builtin_amdgcn_readfirstlane(branch_start(branch_at(tok_first)));
      for (int t = lane; t <= tok_last - tok_first; t += 64) t_rbs[t] = branch_start(branch_at(tok_first + t));
      const int nk = min(dhi - dlo, KEYCAP);
      const int dstride = a.draft_page_table_stride;
      for (int t = lane; t < nk; t += 64) {
        const int x = dlo + t;
        const int jl = branch_at(x);
        const int slot = branch_dstart(jl) + (x - branch_start(jl));
        t_doff[t] = draft_slot_offset(kv, a.draft_page_table + (int64_t)(jb + jl) * dstride, dstride, slot);
      }
      wave_lds_sync();  // t_rbs and t_doff before this wave reads them
    }
  }
#pragma unroll
  for (int it = 0; it < QIT; ++it) {
    const int idx = (int)threadIdx.x + it * 256;
    if (idx < ROWS * CPR) *reinterpret_cast<u32x4*>(qs + (idx / CPR) * QSTR + (idx % CPR) * 8) = qtmp[it];
  }
  __syncthreads();

  auto qfrag = [&](int rb, int ks) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(qs + (rb * 16 + l16) * QSTR + ks * 32 + g4 * 8);
  };

  // ---- draft tiles (the draft wave of split 0) ------------------------------
  // off[kb]: element offset of key base + kb*16 + l16 (-2: no key, -1: bad
  // slot or page, flagged).  Loads are clamped into the pool; lanes without a
  // key hold zeros (their K is masked, their V zeroed when staged).
  const int64_t last_row = pool_last_row(kv, a.num_kv_heads);
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
          o = draft_offset(kv, a.branch_qo_indptr, a.draft_page_table, a.draft_page_table_stride, a.draft_start,
                           jb, je, key, g);
        }
        if (o == -1) atomicOr(&g_device_error, kErrPage);
      }
      off[kb] = o;
    }
  };
  auto load_draft = [&](const int64_t (&off)[2], Raw (&dst)[NL], const void* pool) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bool valid = off[kb] >= 0;
      const int64_t o2 = clamp_row(off[kb], last_row) + g4 * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) dst[kb * KS + ks] = valid ? load_key_chunk<Raw, EB>(pool, o2 + ks * 32) : Raw{};
    }
  };

  // ---- per-tile arithmetic ------------------------------------------------------
  uint16_t* st = reinterpret_cast<uint16_t*>(smem) + w * VSTAGE;
  // V into the stage: row-shaped loads (prefix tiles) or fragment-shaped
  // loads (draft tiles; bit kb of `ok` zeroes a half whose lanes hold no key).
  auto stage_v = [&](const Raw (&vr)[NL], bool rows, int ok) {
#pragma unroll
    for (int r = 0; r < NL; ++r) {
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
      *reinterpret_cast<u32x4*>(st + key * RS + ch * 8) = v;
    }
  };
  auto vt_frag = [&](int db) -> bf16x8 {
    const uint16_t* vb = st + (4 * g4 + (l16 >> 2)) * RS + db * 16 + 4 * (l16 & 3);
    const i16x4 lo = lds_read_tr16(vb);
    const i16x4 hi = lds_read_tr16(vb + 16 * RS);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // S^T of one tile: s[rb][kb] holds keys kb*16 + 4*g4 + i of row rb*16 + l16.
  auto scores = [&](const Raw (&kr)[NL], f32x4 (&s)[RB][2]) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) s[rb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 qf[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) qf[rb] = qfrag(rb, ks);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 kf = __builtin_bit_cast(bf16x8, widen_bf16(kr[kb * KS + ks]));
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) s[rb][kb] = mfma16(kf, qf[rb], s[rb][kb]);
      }
    }
    // Copy the scores out of the MFMA destinations in the block that issued
    // the MFMAs (every later read is then ordered behind the MFMA wait states).
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) asm volatile("" : "+v"(s[rb][kb]));
  };

  float m[RB], l[RB];
  f32x4 o[RB][DB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m[rb] = kNegInf;
    l[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // Online softmax of one tile's scores (masked already) and its P.V.
  auto accumulate = [&](f32x4 (&s)[RB][2]) {
    float lm[RB];
    bool raise = false;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      lm[rb] = fmaxf(fmaxf(fmaxf(s[rb][0][0], s[rb][0][1]), fmaxf(s[rb][0][2], s[rb][0][3])),
                     fmaxf(fmaxf(s[rb][1][0], s[rb][1][1]), fmaxf(s[rb][1][2], s[rb][1][3])));
      raise |= lm[rb] * c2 > m[rb] + kMaxSlack;
    }
    if (__any(raise)) {
      float alpha[RB];
      bool resc = false;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const float mx = rowgroup_max(lm[rb]) * c2;
        const float mold = m[rb];
        const float mnew = mx > mold + kMaxSlack ? mx : mold;
        const float ms = mnew == kNegInf ? 0.f : mnew;
        alpha[rb] = mnew == mold ? 1.f : fast_exp2(mold - ms);
        resc |= mnew != mold && mold != kNegInf;
        m[rb] = mnew;
        l[rb] *= alpha[rb];
      }
      if (__any(resc)) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int db = 0; db < DB; ++db) o[rb][db] *= alpha[rb];
      }
    }
    bf16x8 pf[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
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
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const bf16x8 vf = vt_frag(db);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) o[rb][db] = mfma16(vf, pf[rb], o[rb][db]);
    }
  };

  // ---- the key loop over this wave's prefix tiles ---------------------------------
  // pg holds the pages of the next tile to be requested.  Past the wave's last
  // tile the "next" tile is the current one again (L2-resident, unused), so
  // every iteration has the same loads and wait counts; the draft wave
  // requests its first draft tile there instead.
  const bool verify_drafts = kVerify && split == 0 && dlo < dhi && w == kDraftWave;
  int64_t doff[2] = {-2, -2};
  if (verify_drafts) draft_offsets(dlo, dhi, doff);
  auto pages_of = [&](int tau, int (&pgo)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int first = p0 + tau * 32 + kb * 16;
      pgo[kb] = page_id(first < p1 ? pt_row[first >> kv.log2_page] : -1);
    }
  };
  if (w < npt) pages_of(w + 4 < npt ? w + 4 : w, pg);
  if (verify_drafts && w >= npt) {
    load_draft(doff, vr, kv.v);
    load_draft(doff, kr, kv.k);
  }
  for (int tau = w; tau < npt; tau += 4) {
    const int base = p0 + tau * 32;
    const int nxt = tau + 4;
    const bool last = nxt >= npt;
    const int ld = last ? tau : nxt;
    stage_v(vr, true, 3);
    if (verify_drafts && last) {
      load_draft(doff, vr, kv.v);
    } else {
      spans(pg, p0 + ld * 32, p1, hs);
      load_v(hs, vr);
    }
    f32x4 s[RB][2];
    scores(kr, s);
    if (verify_drafts && last) {
      load_draft(doff, kr, kv.k);
    } else {
      load_k(hs, kr);
      pages_of(nxt + 4 < npt ? nxt + 4 : ld, pg);
    }
    if (base + 32 > p1) {
      // Key base + kb*16 + g4*4 + i is kept iff g4*4 < p1 - base - kb*16 - i.
      const int n = p1 - base;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) s[rb][kb][i] = g4 * 4 < n - (kb * 16 + i) ? s[rb][kb][i] : kNegInf;
    }
    accumulate(s);
  }

  // ---- pass B: the chunk's visible draft tiles, in the draft wave -------------
  if (verify_drafts) {
    int rtok[RB], rbs[RB];
    uint64_t ranc[RB] = {};
    const bool tree = a.draft_mask != nullptr;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      rtok[rb] = row_tok(rb);
      rbs[rb] = t_rbs[rtok[rb] - tok_first];
      if (tree) ranc[rb] = a.draft_mask[(int64_t)(tok0 + rtok[rb]) * a.draft_mask_words];
    }
    for (int base = dlo; base < dhi; base += 32) {
      if (base != dlo) {
        draft_offsets(base, dhi, doff);
        load_draft(doff, vr, kv.v);
        load_draft(doff, kr, kv.k);
      }
      const int ok = (doff[0] >= 0 ? 1 : 0) | (doff[1] >= 0 ? 2 : 0);
      stage_v(vr, false, ok);
      f32x4 s[RB][2];
      scores(kr, s);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        // The tree's window for this tile (see tree_window).
        uint64_t win = 0;
        int wbs = 0;
        if (tree) {
          const int ws = max(base - rbs[rb], 0);
          win = a.draft_mask_words == 1 ? tree_window1(ranc[rb], ws)
                                        : tree_window(a.draft_mask + (int64_t)(tok0 + rtok[rb]) * a.draft_mask_words,
                                                      a.draft_mask_words, ws);
          wbs = rbs[rb] + ws;
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = base + kb * 16 + g4 * 4 + i;
            const bool vis = (key < dhi) & (tree ? draft_visible_tree(win, wbs, key)
                                                 : draft_visible(rtok[rb], rbs[rb], key));
            s[rb][kb][i] = vis ? s[rb][kb][i] : kNegInf;
          }
      }
      accumulate(s);
    }
  }
  mfma_drain();

  // ---- merge the four waves' states (LSE identity) ------------------------------
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
  float lse2[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = rb * 16 + l16;
    float M = kNegInf;
#pragma unroll
    for (int w2 = 0; w2 < 4; ++w2) M = fmaxf(M, ml[(w2 * ROWS + r) * 2]);
    const float ms = M == kNegInf ? 0.f : M;
    float tot = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < 4; ++w2) tot += ml[(w2 * ROWS + r) * 2 + 1] * fast_exp2(ml[(w2 * ROWS + r) * 2] - ms);
    // FP8 pools: the V scale multiplies every normalised output once, here.
    const float f = tot > 0.f ? fast_exp2(m[rb] - ms) / tot * (KV8 ? a.v_scale : 1.f) : 0.f;
    lse2[rb] = tot > 0.f ? M + fast_log2(tot) : kNegInf;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[rb][db] *= f;
  }
  // Wave ow owns channel blocks [ow*DBW, ow*DBW + DBW).  Three rounds through
  // the (now free) V stages: in round r wave w sends its blocks of owner
  // (w + r) % 4 to that owner's slot, and every owner adds what it received.
  // Owner w sums its own blocks, then those of waves w-1, w-2, w-3 (mod 4).
  float* xbuf = reinterpret_cast<float*>(smem);
  f32x4 acc[RB][DBW];
#pragma unroll
  for (int ow = 0; ow < 4; ++ow)
    if (ow == w) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int dbl = 0; dbl < DBW; ++dbl) acc[rb][dbl] = o[rb][ow * DBW + dbl];
    }
#pragma unroll
  for (int r = 1; r < 4; ++r) {
    const int dst_owner = (w + r) & 3;
#pragma unroll
    for (int ow = 0; ow < 4; ++ow)
      if (ow == dst_owner) {
        float* dst = xbuf + ow * XSLOT;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int dbl = 0; dbl < DBW; ++dbl)
            *reinterpret_cast<f32x4*>(dst + ((rb * DBW + dbl) * 64 + lane) * 4) = o[rb][ow * DBW + dbl];
      }
    __syncthreads();
    const float* src = xbuf + w * XSLOT;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int dbl = 0; dbl < DBW; ++dbl)
        acc[rb][dbl] += *reinterpret_cast<const f32x4*>(src + ((rb * DBW + dbl) * 64 + lane) * 4);
    __syncthreads();
  }

  // ---- output ---------------------------------------------------------------------
  // A request whose keys all fall in split 0 writes its final output (the
  // split merge leaves its rows alone).
  const bool partial = a.n_splits > 1 && L > a.split_len;
  const int64_t plane = (int64_t)a.total_rows * a.num_qo_heads;
  if constexpr (KV8) {
    // Per-channel V scales multiply each normalised output channel.
    if (a.v_cs) {
#pragma unroll
      for (int dbl = 0; dbl < DBW; ++dbl) {
        const f32x4 vs = *reinterpret_cast<const f32x4*>(a.v_cs + (int64_t)g * D + (w * DBW + dbl) * 16 + g4 * 4);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) acc[rb][dbl] *= vs;
      }
    }
  }
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    if (!row_valid(rb)) continue;
    const int64_t orow = row_out(rb);
    if (partial) {
#pragma unroll
      for (int dbl = 0; dbl < DBW; ++dbl) {
        const int c = (w * DBW + dbl) * 16 + g4 * 4;
        *reinterpret_cast<f32x4*>(a.ws_o + (split * plane + orow) * D + c) = acc[rb][dbl];
      }
      if (w == 0 && g4 == 0) a.ws_lse[split * plane + orow] = lse2[rb];
      continue;
    }
#pragma unroll
    for (int dbl = 0; dbl < DBW; ++dbl) {
      const int c = (w * DBW + dbl) * 16 + g4 * 4;
      const f32x4 x = acc[rb][dbl];
      if (a.o_bf16) {
        *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a.o) + orow * D + c) =
            u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
      } else {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.o) + orow * D + c) = x;
      }
    }
    if (w == 0 && g4 == 0 && a.lse) a.lse[orow] = lse2[rb] * kLn2;
  }
}

template <bool KV8>
static hipError_t launch_pair(int mode, const AttnArgs& a, int grid, hipStream_t s, hipEvent_t e0,
                              hipEvent_t e1) {
  const dim3 g(grid), b(256);
  // Chunks of one 16-row block (few rows per kv head) run the one-block
  // instance: no MFMA work or state for the empty blocks.
  const bool one = a.chunk_rows <= 16;
  switch (mode) {
    case kModePrefix:
      if (one) go(pair_kernel<1, kModePrefix, KV8>, g, b, s, e0, e1, a);
      else go(pair_kernel<kPairRowBlocks, kModePrefix, KV8>, g, b, s, e0, e1, a);
      break;
    case kModeVerify:
      if (one) go(pair_kernel<1, kModeVerify, KV8>, g, b, s, e0, e1, a);
      else go(pair_kernel<kPairRowBlocks, kModeVerify, KV8>, g, b, s, e0, e1, a);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace casc
