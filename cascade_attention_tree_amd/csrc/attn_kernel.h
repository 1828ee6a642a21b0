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
//   * loads K straight from HBM into MFMA A-fragments (16 keys x 32 channels:
//     one 16-byte load per lane and k-step), gathered through the block table,
//   * computes S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (keys on M, rows on N),
//   * updates a base-2 online softmax per row (in-lane max over 8 keys, then
//     two cross-lane exchanges),
//   * stages V through its own LDS region and reads it back transposed as the
//     A-fragments of O^T += V^T P^T.  P^T is already in B-fragment layout in
//     the lanes that computed S^T, so P never moves between lanes.
// Loads of the wave's next tile are issued as soon as the registers they land
// in are free (V right after staging, K right after its MFMAs), so they run
// under the current tile's softmax and PV work.
//
// The four waves then merge their states with the LSE identity; each wave
// ends up owning a quarter of the head dimension.  Depending on the mode the
// merged state is written as a pass state, as a split partial, or merged once
// more with pass B (computed in the epilogue) into the final output.
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

template <int D, int RB, int MODE>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
attn_kernel(const AttnArgs a) {
  constexpr int KS = D / 32;        // k-steps of the Q K^T contraction
  constexpr int DB = D / 16;        // 16-channel blocks of the head dim
  constexpr int DBW = DB / 4;       // blocks each wave owns after the combine
  constexpr int ROWS = RB * 16;
  constexpr int VSTR = D + 4;       // LDS row stride of a staged V tile (bf16): the
                                    // transposed reads of keys 4 apart hit distinct banks
  constexpr int STAGE = 32 * VSTR;  // bf16 elements per staged tile
  constexpr int XSLOT = RB * DBW * 64 * 4;  // floats per (owner, source) exchange slot
  constexpr int STAGE_BYTES = 4 * 2 * STAGE * 2;
  constexpr int XBYTES = 12 * XSLOT * 4;
  constexpr int UNION_BYTES = STAGE_BYTES > XBYTES ? STAGE_BYTES : XBYTES;
  constexpr bool kMainLoop = MODE <= kModeNaive;
  constexpr bool kFinish = MODE == kModePrefixFinish || MODE == kModeVerifyFinish;
  constexpr bool kEpilogueDraft = MODE == kModeVerify || MODE == kModeVerifyFinish;
  constexpr bool kNeedQ = MODE != kModePrefixFinish;
  // Large row tiles keep Q in LDS (read per tile as B-fragments) so that the
  // architectural VGPRs stay free for K/V in flight and the softmax.
  constexpr bool kQInLds = kNeedQ && RB * KS >= 16;
  constexpr int QSTR = D + 8;  // padded LDS row stride of Q: rows land 4 banks apart
  constexpr int QBYTES = kQInLds ? ROWS * QSTR * 2 : 0;

  __shared__ __attribute__((aligned(16))) unsigned char smem[UNION_BYTES + QBYTES + 4 * ROWS * 2 * 4];
  uint16_t* qs = reinterpret_cast<uint16_t*>(smem + UNION_BYTES);               // [ROWS][QSTR]
  float* ml = reinterpret_cast<float*>(smem + UNION_BYTES + QBYTES);  // [4 waves][ROWS][m, l]

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15;
  const int g4 = lane >> 4;

  // ---- work item -------------------------------------------------------
  int item = blockIdx.x;
  const int split = item % a.grid_splits;
  item /= a.grid_splits;
  const int chunk = item % a.n_chunks;
  item /= a.n_chunks;
  const int g = item % a.num_kv_heads;
  const int seg = item / a.num_kv_heads;

  const int32_t* __restrict__ qo = a.branch_qo_indptr;
  int req, jb, je;
  if constexpr (MODE == kModeNaive) {
    jb = seg;
    je = seg + 1;
    req = request_of_branch(a.req_branch_indptr, a.batch_size, seg);
  } else {
    req = seg;
    jb = a.req_branch_indptr[seg];
    je = a.req_branch_indptr[seg + 1];
  }
  const int tok0 = qo[jb];
  const int tok1 = qo[je];
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

  int L = a.cache_seqlens[req];
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

  // ---- rows of this lane (column l16 of each 16-row block of S^T / O^T) --
  // Recomputed where needed rather than kept live across the key loop.
  auto row_valid = [&](int rb) { return row0 + rb * 16 + l16 < nrows; };
  auto row_tok = [&](int rb) {  // segment token of the row (0 for padding rows)
    const int rho = row0 + rb * 16 + l16;
    return rho < nrows ? rho / a.group : 0;
  };
  auto row_out = [&](int rb) -> int64_t {  // index of (row, head) in [total_rows, Hq]
    const int rho = row0 + rb * 16 + l16;
    const int t = rho / a.group;
    return (int64_t)(tok0 + t) * a.num_qo_heads + g * a.group + (rho - t * a.group);
  };
  // Segment token where the row's branch starts (draft masks only).
  auto row_branch_start = [&](int rb) {
    if constexpr (MODE == kModeNaive) return 0;
    return qo[branch_of_row(qo, jb, je, tok0 + row_tok(rb))] - tok0;
  };
  int rtok[RB] = {}, rbs[RB] = {};
  auto load_row_masks = [&]() {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      rtok[rb] = row_tok(rb);
      rbs[rb] = row_branch_start(rb);
    }
  };
  // Draft keys this chunk can see: [dlo, dhi) in segment tokens.
  const int tok_first = row0 / a.group;
  const int tok_last = (row_end - 1) / a.group;
  int dlo = 0;
  if constexpr (MODE != kModeNaive) dlo = qo[branch_of_row(qo, jb, je, tok0 + tok_first)] - tok0;
  const int dhi = tok_last + 1;

  // Q B-fragments: lane holds row rb*16 + l16, channels ks*32 + g4*8 .. +8.
  bf16x8 qf[kQInLds ? 1 : RB][KS];
  if constexpr (kQInLds) {
    // Cooperative copy of the chunk's rows into LDS; 16 bytes per thread step.
    constexpr int kChunks = D / 8;
    for (int idx = threadIdx.x; idx < ROWS * kChunks; idx += 256) {
      const int r = idx / kChunks, c = idx % kChunks;
      const int rho = row0 + r;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (rho < nrows) {
        const int t = rho / a.group;
        const int h = g * a.group + (rho - t * a.group);
        x = *reinterpret_cast<const u32x4*>(a.q + (int64_t)(tok0 + t) * a.q_row_stride +
                                            (int64_t)h * a.q_head_stride + c * 8);
      }
      *reinterpret_cast<u32x4*>(qs + r * QSTR + c * 8) = x;
    }
    __syncthreads();
  } else if constexpr (kNeedQ) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int rho = row0 + rb * 16 + l16;
      const int t = row_tok(rb);
      const uint16_t* qp = a.q + (int64_t)(tok0 + t) * a.q_row_stride +
                           (int64_t)(g * a.group + (rho - t * a.group)) * a.q_head_stride + g4 * 8;
      const bool ok = row_valid(rb);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qf[rb][ks] = ok ? *reinterpret_cast<const bf16x8*>(qp + ks * 32) : bf16x8{};
    }
  }
  auto qfrag = [&](int rb, int ks) -> bf16x8 {
    if constexpr (kQInLds) {
      return *reinterpret_cast<const bf16x8*>(qs + (rb * 16 + l16) * QSTR + ks * 32 + g4 * 8);
    } else {
      return qf[rb][ks];
    }
  };

  const KvView kv = a.kv;
  cint32* pt_row = as_const(a.page_table + (int64_t)req * a.page_table_stride);
  const float c2 = a.scale_log2;
  const int pmask = (1 << kv.log2_page) - 1;
  const int64_t head_off = (int64_t)g * kv.head_stride + g4 * 8;

  // ---- per-tile building blocks ----------------------------------------

  // Prefix tiles start at a multiple of 32 and pages hold >= 16 tokens, so
  // each 16-key half of a tile lies in one page whose id pg[kb] is
  // wave-uniform (-1: no key in that half, or an id outside the pool).
  auto load_prefix = [&](const uint16_t* pool, const int (&pg)[2], int base, int end,
                         bf16x8 (&r)[2][KS]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = base + kb * 16 + l16;
      const bool page_ok = pg[kb] >= 0;
      const __amdgpu_buffer_rsrc_t rs =
          page_rsrc(pool + (int64_t)(page_ok ? pg[kb] : 0) * kv.page_stride, page_ok ? kv.page_bytes : 0);
      const int off = key < end ? (int)(((int64_t)(key & pmask) * kv.token_stride + head_off) * 2)
                                : kOutOfRange;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) r[kb][ks] = __builtin_bit_cast(bf16x8, buf_load16(rs, off + ks * 64));
    }
  };
  auto load_k_prefix = [&](const int (&pg)[2], int base, int end, bf16x8 (&kr)[2][KS]) {
    load_prefix(kv.k, pg, base, end, kr);
  };
  auto load_v_prefix = [&](const int (&pg)[2], int base, int end, bf16x8 (&vr)[2][KS]) {
    load_prefix(kv.v, pg, base, end, vr);
  };
  auto prefix_pages = [&](int base, int end, int (&pg)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int first = base + kb * 16;
      int id = first < end ? pt_row[first >> kv.log2_page] : -1;
      if (id >= kv.num_pages) {
        if (lane == 0) atomicOr(&g_device_error, kErrPage);
      }
      if ((uint32_t)id >= (uint32_t)kv.num_pages) id = -1;
      pg[kb] = __builtin_amdgcn_readfirstlane(id);  // uniform by construction
    }
  };
  // Draft tiles: keys are segment tokens [base, base+32); each lane resolves
  // its own key's branch, slot and page (-2: no key, -1: bad page).
  auto draft_offsets = [&](int base, int end, int64_t (&off)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = base + kb * 16 + l16;
      off[kb] = -2;
      if (key < end) {
        off[kb] = draft_offset(kv, qo, a.draft_page_table, a.draft_page_table_stride, a.draft_start,
                               jb, je, key, g);
        if (off[kb] == -1) atomicOr(&g_device_error, kErrPage);
      }
    }
  };
  auto load_draft_at = [&](const int64_t (&off)[2], bf16x8 (&kr)[2][KS], bf16x8 (&vr)[2][KS]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bool ok = off[kb] >= 0;
      const int64_t o2 = ok ? off[kb] + g4 * 8 : (int64_t)(g4 * 8);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        kr[kb][ks] = *reinterpret_cast<const bf16x8*>(kv.k + o2 + ks * 32);
        const u32x4 x = *reinterpret_cast<const u32x4*>(kv.v + o2 + ks * 32);
        vr[kb][ks] = __builtin_bit_cast(bf16x8, ok ? x : u32x4{0u, 0u, 0u, 0u});
      }
    }
  };
  auto load_draft = [&](int base, int end, bf16x8 (&kr)[2][KS], bf16x8 (&vr)[2][KS]) {
    int64_t off[2];
    draft_offsets(base, end, off);
    load_draft_at(off, kr, vr);
  };

  // The fused verify epilogue starts with the first draft tile of the chunk;
  // its addresses are resolved now so that its loads can be issued as soon as
  // the prefix loop ends.
  int64_t doff0[2] = {-2, -2};
  if constexpr (kEpilogueDraft) {
    if (dlo < dhi) draft_offsets(dlo, dhi, doff0);
  }
  bf16x8 dkr[2][KS], dvr[2][KS];
  bool draft_loaded = false;

  // S^T for one tile: s[rb][kb] holds keys kb*16 + 4*g4 + i of row rb*16 + l16.
  auto scores = [&](const bf16x8 (&kr)[2][KS], f32x4 (&s)[RB][2]) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) acc = mfma16(kr[kb][ks], qfrag(rb, ks), acc);
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

  // Prefix keys: only the bound `end`.
  auto mask_prefix = [&](int base, int end, f32x4 (&s)[RB][2]) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (base + kb * 16 + g4 * 4 + i >= end) s[rb][kb][i] = kNegInf;
  };
  // Draft keys: the bound `end` and the in-branch ancestor rule (rtok / rbs
  // must have been loaded by load_row_masks).
  auto mask_draft = [&](int base, int end, f32x4 (&s)[RB][2]) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = base + kb * 16 + g4 * 4 + i;
          if (!(key < end && draft_visible(rtok[rb], rbs[rb], key))) s[rb][kb][i] = kNegInf;
        }
      }
    }
  };

  // Online softmax update in base 2.  m is the carried max (raised only past
  // the slack), alpha the factor the accumulator must be scaled by, pf the
  // weights as P^T B-fragments.  Returns whether this lane needs a rescale.
  auto softmax = [&](f32x4 (&s)[RB][2], float (&m)[RB], float (&l)[RB], float (&alpha)[RB],
                     bf16x8 (&pf)[RB]) -> bool {
    bool rescale = false;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float mx = fmaxf(fmaxf(fmaxf(s[rb][0][0], s[rb][0][1]), fmaxf(s[rb][0][2], s[rb][0][3])),
                       fmaxf(fmaxf(s[rb][1][0], s[rb][1][1]), fmaxf(s[rb][1][2], s[rb][1][3])));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      mx *= c2;
      const float mold = m[rb];
      const float mnew = mx > mold + kMaxSlack ? mx : mold;
      const float ms = mnew == kNegInf ? 0.f : mnew;
      alpha[rb] = mnew == mold ? 1.f : fast_exp2(mold - ms);
      rescale |= mnew != mold && mold != kNegInf;
      m[rb] = mnew;
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
    return rescale;
  };

  // Writes a tile's V rows to this wave's LDS stage: row = key, VSTR stride.
  auto stage_v = [&](const bf16x8 (&vr)[2][KS], uint16_t* vs) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 x = __builtin_bit_cast(u32x4, vr[kb][ks]);
        u32x2* dst = reinterpret_cast<u32x2*>(vs + (kb * 16 + l16) * VSTR + ks * 32 + g4 * 8);
        dst[0] = u32x2{x[0], x[1]};
        dst[1] = u32x2{x[2], x[3]};
      }
    }
  };

  // V^T A-fragment of channel block db: lane holds channel db*16 + l16 of keys
  // kb*16 + 4*g4 + i, the key order of P^T.
  auto vt_frag = [&](const uint16_t* vs, int db) -> bf16x8 {
    const uint16_t* vb = vs + (4 * g4) * VSTR + db * 16 + l16;
    uint32_t e[8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) e[kb * 4 + i] = vb[(kb * 16 + i) * VSTR];
    }
    const u32x4 pk = {e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16),
                      e[6] | (e[7] << 16)};
    return __builtin_bit_cast(bf16x8, pk);
  };

  // Merged pass state of this lane's rows for the channel blocks this wave
  // owns: acc[rb][dbl] normalised output, lse2[rb] base-2 LSE.
  f32x4 acc[RB][DBW];
  float lse2[RB];

  if constexpr (kMainLoop) {
    int p0 = 0, p1 = 0;
    if constexpr (MODE == kModePrefix || MODE == kModeVerify) {
      p0 = split * a.split_len;
      p1 = min(L, p0 + a.split_len);
      if (a.n_splits > 1 && p0 >= L) return;  // no keys in this split: no partial
      if (p1 < p0) p1 = p0;
    } else if constexpr (MODE == kModeNaive) {
      p1 = L;
    }
    int d0 = 0, d1 = 0;
    if constexpr (MODE == kModeDraft || MODE == kModeNaive) {
      d0 = dlo;
      d1 = dhi;
    }
    const int npt = (p1 - p0 + 31) >> 5;
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
    uint16_t* stage = reinterpret_cast<uint16_t*>(smem) + w * 2 * STAGE;

    // Tile tau covers prefix keys p0 + 32*tau .. for tau < npt, then draft
    // tokens d0 + 32*(tau - npt) .. .  Draft tiles load K and V together.
    auto pages_of = [&](int tau, int (&pg)[2]) {
      if (tau < npt) {
        prefix_pages(p0 + tau * 32, p1, pg);
      } else {
        pg[0] = -1;
        pg[1] = -1;
      }
    };

    bf16x8 kr[2][KS], vr[2][KS];
    int pg[2] = {-1, -1};
    // Prefix-only launches (pass A, verify) prefetch without branches: past the
    // wave's last tile the "next" tile is the current one again (L2-resident,
    // never used), so the load sequence and its wait counts are the same every
    // iteration.
    constexpr bool kPrefixOnly = MODE == kModePrefix || MODE == kModeVerify;
    if (w < nt) {
      pages_of(w, pg);
      if (w < npt) {
        load_v_prefix(pg, p0 + w * 32, p1, vr);
        load_k_prefix(pg, p0 + w * 32, p1, kr);
      } else {
        load_draft(d0 + (w - npt) * 32, d1, kr, vr);
      }
      pages_of(w + 4 < nt ? w + 4 : w, pg);
    }
    int buf = 0;
    for (int tau = w; tau < nt; tau += 4) {
      const int nxt = tau + 4;
      const bool is_prefix = tau < npt;
      const int base = is_prefix ? p0 + tau * 32 : d0 + (tau - npt) * 32;
      const int end = is_prefix ? p1 : d1;
      uint16_t* vs = stage + buf * STAGE;
      buf ^= 1;
      stage_v(vr, vs);
      f32x4 s[RB][2];
      if constexpr (kPrefixOnly) {
        const int ld = nxt < nt ? nxt : tau;
        load_v_prefix(pg, p0 + ld * 32, p1, vr);
        scores(kr, s);
        load_k_prefix(pg, p0 + ld * 32, p1, kr);
        pages_of(nxt + 4 < nt ? nxt + 4 : ld, pg);
      } else {
        if (nxt < npt) load_v_prefix(pg, p0 + nxt * 32, p1, vr);
        scores(kr, s);
        if (nxt < npt) {
          load_k_prefix(pg, p0 + nxt * 32, p1, kr);
        } else if (nxt < nt) {
          load_draft(d0 + (nxt - npt) * 32, d1, kr, vr);
        }
        if (nxt + 4 < nt) pages_of(nxt + 4, pg);
      }
      if (!is_prefix) {
        mask_draft(base, end, s);
      } else if (base + 32 > end) {
        mask_prefix(base, end, s);
      }
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
        const bf16x8 vf = vt_frag(vs, db);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) o[rb][db] = mfma16(vf, pf[rb], o[rb][db]);
      }
    }

    mfma_drain();
    if constexpr (MODE == kModeVerify) {
      if (a.n_splits == 1 && dlo < dhi) {
        load_draft_at(doff0, dkr, dvr);  // lands while the waves merge
        draft_loaded = true;
      }
    }

    // ---- merge the four waves' states (LSE identity) ----------------------
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      l[rb] += __shfl_xor(l[rb], 16);
      l[rb] += __shfl_xor(l[rb], 32);
    }
    if (g4 == 0) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        ml[(w * ROWS + rb * 16 + l16) * 2 + 0] = m[rb];
        ml[(w * ROWS + rb * 16 + l16) * 2 + 1] = l[rb];
      }
    }
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int r = rb * 16 + l16;
      float M = kNegInf;
#pragma unroll
      for (int w2 = 0; w2 < 4; ++w2) M = fmaxf(M, ml[(w2 * ROWS + r) * 2]);
      const float ms = M == kNegInf ? 0.f : M;
      float tot = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < 4; ++w2)
        tot += ml[(w2 * ROWS + r) * 2 + 1] * fast_exp2(ml[(w2 * ROWS + r) * 2] - ms);
      const float f = tot > 0.f ? fast_exp2(m[rb] - ms) / tot : 0.f;
      lse2[rb] = tot > 0.f ? M + fast_log2(tot) : kNegInf;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[rb][db] *= f;
    }
    // Owner ow of channel blocks [ow*DBW, ow*DBW + DBW) receives the other
    // waves' scaled blocks through LDS and sums all four in wave order.
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
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int dbl = 0; dbl < DBW; ++dbl) {
        f32x4 own = o[rb][dbl];
#pragma unroll
        for (int ow = 1; ow < 4; ++ow)
          if (ow == w) own = o[rb][ow * DBW + dbl];
        f32x4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) {
          const f32x4 x = w2 == w ? own
                                  : *reinterpret_cast<const f32x4*>(
                                        xbuf + slot(w, w2) * XSLOT + ((rb * DBW + dbl) * 64 + lane) * 4);
          sum += x;
        }
        acc[rb][dbl] = sum;
      }
    }
  }

  if constexpr (kFinish) {
    if constexpr (MODE == kModeVerifyFinish) {
      if (dlo < dhi) {
        load_draft_at(doff0, dkr, dvr);  // lands while the partials merge
        draft_loaded = true;
      }
    }
    // Merge the prefix split partials of these rows (fixed split order).
    const int nsp = (L + a.split_len - 1) / a.split_len;
    const int64_t plane = (int64_t)a.total_rows * a.num_qo_heads;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int dbl = 0; dbl < DBW; ++dbl) acc[rb][dbl] = f32x4{0.f, 0.f, 0.f, 0.f};
      lse2[rb] = kNegInf;
      if (!row_valid(rb)) continue;
      const int64_t orow = row_out(rb);
      float M = kNegInf;
      for (int sp = 0; sp < nsp; ++sp) M = fmaxf(M, a.ws_lse[sp * plane + orow]);
      const float ms = M == kNegInf ? 0.f : M;
      float tot = 0.f;
      for (int sp = 0; sp < nsp; ++sp) {
        const float wgt = fast_exp2(a.ws_lse[sp * plane + orow] - ms);
        tot += wgt;
#pragma unroll
        for (int dbl = 0; dbl < DBW; ++dbl) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(
              a.ws_o + (sp * plane + orow) * D + (w * DBW + dbl) * 16 + g4 * 4);
          if (wgt != 0.f) acc[rb][dbl] += wgt * x;
        }
      }
      const float inv = tot > 0.f ? 1.f / tot : 0.f;
#pragma unroll
      for (int dbl = 0; dbl < DBW; ++dbl) acc[rb][dbl] *= inv;
      lse2[rb] = tot > 0.f ? M + fast_log2(tot) : kNegInf;
    }
  }

  // Split prefix passes stop at a partial state; everything else is final.
  bool partial = false;
  if constexpr (MODE == kModePrefix || MODE == kModeVerify) partial = a.n_splits > 1;

  if constexpr (kEpilogueDraft) {
    if (!partial) {
      // Pass B for the rows of this chunk: every wave walks the request's
      // visible draft tiles (a handful of keys), keeping only its own channel
      // blocks of o_B, then merges with pass A by the LSE identity.
      __syncthreads();  // the exchange buffer is reused as staging below
      load_row_masks();
      uint16_t* vs = reinterpret_cast<uint16_t*>(smem) + w * STAGE;
      float mB[RB], lB[RB];
      f32x4 oB[RB][DBW];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        mB[rb] = kNegInf;
        lB[rb] = 0.f;
#pragma unroll
        for (int dbl = 0; dbl < DBW; ++dbl) oB[rb][dbl] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      for (int base = dlo; base < dhi; base += 32) {
        bf16x8 kr[2][KS], vr[2][KS];
        if (base == dlo && draft_loaded) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
              kr[kb][ks] = dkr[kb][ks];
              vr[kb][ks] = dvr[kb][ks];
            }
        } else {
          load_draft(base, dhi, kr, vr);
        }
        stage_v(vr, vs);
        f32x4 s[RB][2];
        scores(kr, s);
        mask_draft(base, dhi, s);
        float alpha[RB];
        bf16x8 pf[RB];
        softmax(s, mB, lB, alpha, pf);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int dbl = 0; dbl < DBW; ++dbl) oB[rb][dbl] *= alpha[rb];
#pragma unroll
        for (int dbl = 0; dbl < DBW; ++dbl) {
          const bf16x8 vf = vt_frag(vs, w * DBW + dbl);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) oB[rb][dbl] = mfma16(vf, pf[rb], oB[rb][dbl]);
        }
      }
      mfma_drain();
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        lB[rb] += __shfl_xor(lB[rb], 16);
        lB[rb] += __shfl_xor(lB[rb], 32);
        const float lseB = lB[rb] > 0.f ? mB[rb] + fast_log2(lB[rb]) : kNegInf;
        const float invB = lB[rb] > 0.f ? 1.f / lB[rb] : 0.f;
        float wa, wb, lt;
        merge_weights(lse2[rb], lseB, wa, wb, lt);
#pragma unroll
        for (int dbl = 0; dbl < DBW; ++dbl)
          acc[rb][dbl] = wsum(wa, acc[rb][dbl], wb, oB[rb][dbl] * invB);
        lse2[rb] = lt;
      }
    }
  }

  // ---- output ----------------------------------------------------------------
  const int64_t plane = (int64_t)a.total_rows * a.num_qo_heads;
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

}  // namespace casc
