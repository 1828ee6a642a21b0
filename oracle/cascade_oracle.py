"""CPU fp64 oracle for cascade verify attention (TEST INFRASTRUCTURE ONLY).

Only the tests, the package's smoke check and the bench's CPU-baseline leg may
import this module.  The product path never calls it; the GPU path and this
oracle share no code (the only common module is the seeded input generator,
which holds no attention arithmetic).

Sources (the three pages this work follows):

* Cascade attention page (zdszero.github.io, "cascade_attention"):
  - section "splittability of standard attention": softmax attention with the
    1/sqrt(d) scale, the per-part log-sum-exp LSE_A, and the merge of two
    disjoint key parts into one attention (the identity merge_state applies);
  - section "topk > 1": each draft token of a branch attends the request's
    prefix plus its own branch's ancestors, the prefix being shared by all
    branches; naive expansion into B*topk virtual requests and its KV read
    count B*topk*(L+S);
  - section "mathematical structure of the cascade scheme": pass A (prefix,
    per-request page table, all branches' queries), pass B (per-branch page
    table, own S draft tokens), merge; read count B*L + B*topk*S.
* KV-cache and speculative-decoding tutorial page:
  - section 5.2/5.3 (PagedAttention): fixed-size pages, per-request block table
    mapping logical to physical pages, gather inside the kernel;
  - section 6.3 (GQA): H % H_kv == 0, query head h uses kv head h // (H/H_kv);
  - section 8.2 (tree attention mask): a node attends exactly its ancestor set,
    itself included.
* Causal attention under a prefix-cache hit page (weigao.cc): sections 1-3,
  visible query-key pairs of a causal prompt and of a suffix after a hit of H
  tokens.

Readings taken where the pages leave a step open:

* Every score is scaled by sm_scale (1/sqrt(d) by default), in pass A, pass B
  and naive expansion alike; the cascade page writes o_A without the scale but
  its LSE_A with it, and the merge identity only holds with one scale.
* LSE is the natural logarithm of the sum of exponentials of the scaled scores.
* An empty key set has o = 0 and LSE = -inf; a merge with one empty side
  returns the other side; a merge of two empty sides is (0, -inf).
* A draft token sees itself (ancestor set includes the node).
* Branches share nothing but the prefix.  A branch is a chain unless the
  workload carries a draft tree; then each row's visible drafts are the nodes
  whose bits are set in its ancestor mask (tree attention mask, tutorial page
  section 8.2), and a request's tree is one branch holding all of its nodes.
* Draft token u of branch j lives at logical slot draft_start[j] + u of the
  block-table row draft_page_table[j].
* FP8 KV (tutorial page, section 4.5, per-tensor granularity): a pool element
  is an OCP E4M3 code c and stands for value(c) * scale, one scale for all of
  K and one for all of V; the attention is then the one over those values.

Parity pins: every function here is checked in tests/test_oracle_pins.py
against closed forms, library routines, brute force on tiny inputs, or the
numbers the pages print.  No function is parity-unpinned.
"""

from __future__ import annotations

import numpy as np


# ---------------------------------------------------------------------------
# FP8 KV (tutorial page, section 4.5: FP8 KV cache, per-tensor scale)
# ---------------------------------------------------------------------------

def e4m3_value(codes):
    """Values of OCP FP8 E4M3 codes (uint8), float64: sign bit 7, exponent bits
    6..3 with bias 7, mantissa bits 2..0.  Exponent field e > 0 gives
    (-1)^s 2^(e-7) (1 + m/8); e = 0 gives the subnormal (-1)^s 2^-6 (m/8).
    There are no infinities; e = 15 with m = 7 (0x7F, 0xFF) is NaN, so the
    largest finite magnitude is 2^8 * 1.75 = 448."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e > 0, np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int32)), np.ldexp(m / 8.0, -6))
    val = sign * mag
    return np.where((e == 15) & ((c & 0x7) == 7), np.nan, val)


def dequantize_kv(wl):
    """The workload with its K/V pools replaced by the values its FP8 codes
    stand for, float64: value(code) * scale, times the channel's scale when
    the workload has per-channel scales (tutorial page, section 4.5: per-tensor
    or per-channel scales; pools [pages, P, Hkv, d], channel scales [Hkv, d]).
    A workload without codes is returned unchanged."""
    import dataclasses
    if getattr(wl, "k_codes", None) is None:
        return wl
    k = e4m3_value(wl.k_codes) * float(wl.k_scale)
    v = e4m3_value(wl.v_codes) * float(wl.v_scale)
    if getattr(wl, "k_channel_scale", None) is not None:
        k = k * np.asarray(wl.k_channel_scale, np.float64)[None, None, :, :]
        v = v * np.asarray(wl.v_channel_scale, np.float64)[None, None, :, :]
    return dataclasses.replace(wl, k_pool=k, v_pool=v,
                               prefix_k=None, prefix_v=None, draft_k=None, draft_v=None)


# ---------------------------------------------------------------------------
# Paged gather (tutorial page, section 5.2: block table, logical -> physical)
# ---------------------------------------------------------------------------

def gather_slots(pool, table_row, first_slot, count, page_size):
    """Tokens at logical slots [first_slot, first_slot + count) of one block-table
    row.  Slot t lives in physical page table_row[t // P] at offset t % P.

    pool: [num_pages, P, Hkv, d].  Returns float64 [count, Hkv, d]."""
    t = int(first_slot) + np.arange(int(count))
    pages = np.asarray(table_row)[t // page_size]
    return np.asarray(pool[pages, t % page_size], dtype=np.float64)


def scatter_slots(pool, table_row, first_slot, values, page_size):
    """The inverse of gather_slots: a copy of ``pool`` with ``values`` [count,
    Hkv, d] written at logical slots [first_slot, first_slot + count) of one
    block-table row."""
    out = np.array(pool, copy=True)
    t = int(first_slot) + np.arange(values.shape[0])
    pages = np.asarray(table_row)[t // page_size]
    out[pages, t % page_size] = values
    return out


# ---------------------------------------------------------------------------
# The serving step around verification (tutorial page, section 5.2, pages
# through the block table; section 7, 7.1 and 7.6, the verify and rollback loop):
# the drafts' K/V are written into their pages before the verify pass, and
# after it the accepted path's K/V join the request's prefix.
# ---------------------------------------------------------------------------

def append_draft_kv(wl, k_new, v_new):
    """K and V of every query row's draft token, [total_rows, Hkv, d], written
    to its slot: row r = position u of branch j goes to logical slot
    draft_start[j] + u of draft block-table row j.  Returns (k_pool, v_pool)."""
    k_pool, v_pool = wl.k_pool, wl.v_pool
    qo = wl.branch_qo_indptr
    for j in range(wl.num_branches):
        r0, r1 = int(qo[j]), int(qo[j + 1])
        k_pool = scatter_slots(k_pool, wl.draft_page_table[j], int(wl.draft_start[j]),
                               np.asarray(k_new[r0:r1]), wl.page_size)
        v_pool = scatter_slots(v_pool, wl.draft_page_table[j], int(wl.draft_start[j]),
                               np.asarray(v_new[r0:r1]), wl.page_size)
    return k_pool, v_pool


def commit_accepted(wl, accepted_indptr, accepted_rows):
    """For request i, the accepted rows accepted_rows[accepted_indptr[i] ..
    accepted_indptr[i+1]) (global query rows, in path order) have their draft
    tokens' K and V appended to the prefix: slots L_i, L_i + 1, ... of block-table
    row i.  Returns (k_pool, v_pool, new cache_seqlens).  Nothing else changes,
    so rejected drafts cost nothing (their slots are rewritten next step)."""
    k_pool, v_pool = wl.k_pool, wl.v_pool
    br_of = _branch_of_row(wl.branch_qo_indptr)
    lens = np.array(wl.cache_seqlens, np.int64, copy=True)
    for i in range(wl.batch_size):
        rows = [int(r) for r in accepted_rows[int(accepted_indptr[i]):int(accepted_indptr[i + 1])]]
        if not rows:
            continue
        ks, vs = [], []
        for r in rows:
            j = int(br_of[r])
            slot = int(wl.draft_start[j]) + r - int(wl.branch_qo_indptr[j])
            ks.append(gather_slots(wl.k_pool, wl.draft_page_table[j], slot, 1, wl.page_size)[0])
            vs.append(gather_slots(wl.v_pool, wl.draft_page_table[j], slot, 1, wl.page_size)[0])
        L = int(wl.cache_seqlens[i])
        k_pool = scatter_slots(k_pool, wl.page_table[i], L, np.array(ks), wl.page_size)
        v_pool = scatter_slots(v_pool, wl.page_table[i], L, np.array(vs), wl.page_size)
        lens[i] = L + len(rows)
    return k_pool, v_pool, lens.astype(np.int32)


# ---------------------------------------------------------------------------
# One attention state (cascade page, "splittability of standard attention")
# ---------------------------------------------------------------------------

def attention_state(q, k, v, sm_scale):
    """Softmax attention of queries over one key set, with its LSE.

    q [n, d], k [m, d], v [m, dv] (float64).  Returns (o [n, dv], lse [n]) with
    o = softmax(sm_scale * q k^T) v and lse = ln sum_j exp(sm_scale * q . k_j).
    An empty key set gives o = 0 and lse = -inf."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    n = q.shape[0]
    if k.shape[0] == 0:
        return np.zeros((n, v.shape[1])), np.full(n, -np.inf)
    z = sm_scale * (q @ k.T)
    zmax = z.max(axis=1, keepdims=True)
    w = np.exp(z - zmax)
    tot = w.sum(axis=1, keepdims=True)
    lse = zmax[:, 0] + np.log(tot[:, 0])
    o = (w / tot) @ v
    return o, lse


def merge_state(o_a, lse_a, o_b, lse_b):
    """Merge two attention states over disjoint key sets A and B.

    LSE = ln(e^LSE_A + e^LSE_B), o = e^(LSE_A - LSE) o_A + e^(LSE_B - LSE) o_B,
    evaluated with the larger LSE factored out so that no exponential overflows.
    Shapes: o_* [..., d], lse_* [...].  A side with LSE = -inf contributes nothing;
    two such sides give (0, -inf)."""
    o_a = np.asarray(o_a, np.float64)
    o_b = np.asarray(o_b, np.float64)
    lse_a = np.asarray(lse_a, np.float64)
    lse_b = np.asarray(lse_b, np.float64)
    m = np.maximum(lse_a, lse_b)
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    tot = np.exp(lse_a - m_safe) + np.exp(lse_b - m_safe)
    lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, tot)))
    lse_safe = np.where(empty, 0.0, lse)
    wa = np.where(empty, 0.0, np.exp(lse_a - lse_safe))
    wb = np.where(empty, 0.0, np.exp(lse_b - lse_safe))
    o = wa[..., None] * o_a + wb[..., None] * o_b
    return o, lse


# ---------------------------------------------------------------------------
# Tree structure helpers (cascade page, "topk > 1")
# ---------------------------------------------------------------------------

def _request_of_branch(req_branch_indptr):
    rb = np.asarray(req_branch_indptr)
    out = np.empty(int(rb[-1]), np.int64)
    for i in range(rb.shape[0] - 1):
        out[rb[i]:rb[i + 1]] = i
    return out


def _branch_of_row(branch_qo_indptr):
    qo = np.asarray(branch_qo_indptr)
    out = np.empty(int(qo[-1]), np.int64)
    for j in range(qo.shape[0] - 1):
        out[qo[j]:qo[j + 1]] = j
    return out


def _kv_head(h, num_qo_heads, num_kv_heads):
    """GQA head sharing (tutorial page, section 6.3)."""
    if num_qo_heads % num_kv_heads:
        raise ValueError("query heads must be a multiple of kv heads")
    return h // (num_qo_heads // num_kv_heads)


def _prefix_kv(wl, i):
    L = int(wl.cache_seqlens[i])
    k = gather_slots(wl.k_pool, wl.page_table[i], 0, L, wl.page_size)
    v = gather_slots(wl.v_pool, wl.page_table[i], 0, L, wl.page_size)
    return k, v


def _draft_kv(wl, j):
    S = int(wl.branch_qo_indptr[j + 1] - wl.branch_qo_indptr[j])
    s0 = int(wl.draft_start[j])
    k = gather_slots(wl.k_pool, wl.draft_page_table[j], s0, S, wl.page_size)
    v = gather_slots(wl.v_pool, wl.draft_page_table[j], s0, S, wl.page_size)
    return k, v


# ---------------------------------------------------------------------------
# The two passes and their merge (cascade page, "mathematical structure")
# ---------------------------------------------------------------------------

def draft_visible(wl, j, s):
    """Draft positions of branch j that its position s attends: its ancestors
    and itself (tutorial page, section 8.2).  A chain is the tree in which node
    u's parent is u - 1, so it sees positions 0..s; a general tree gives each
    row its ancestor set as a bit mask over the branch's nodes."""
    if getattr(wl, "draft_mask", None) is None:
        return np.arange(s + 1)
    r0 = int(wl.branch_qo_indptr[j])
    S = int(wl.branch_qo_indptr[j + 1]) - r0
    # One 64-bit word per row, or W words (bit u % 64 of word u // 64: node u).
    words = np.atleast_1d(np.asarray(wl.draft_mask[r0 + s], np.uint64))
    m = sum(int(x) << (64 * w) for w, x in enumerate(words))
    return np.array([u for u in range(S) if (m >> u) & 1], np.int64)


def prefix_pass(wl, requests=None):
    """Pass A.  Request i's prefix (L_i tokens via its page-table row) is read
    once and attended by every query row of all of its branches.

    Returns (o_A [rows, Hq, d], lse_A [rows, Hq]); rows of requests not listed
    are left at (0, -inf)."""
    R, Hq, d = wl.q.shape
    o = np.zeros((R, Hq, d))
    lse = np.full((R, Hq), -np.inf)
    rb, qo = wl.req_branch_indptr, wl.branch_qo_indptr
    reqs = range(wl.batch_size) if requests is None else requests
    for i in reqs:
        r0, r1 = int(qo[rb[i]]), int(qo[rb[i + 1]])
        k, v = _prefix_kv(wl, i)
        for h in range(Hq):
            g = _kv_head(h, Hq, wl.num_kv_heads)
            o[r0:r1, h], lse[r0:r1, h] = attention_state(
                wl.q[r0:r1, h], k[:, g], v[:, g], wl.sm_scale)
    return o, lse


def draft_pass(wl, branches=None):
    """Pass B.  Branch j (one of the B*topk virtual requests) reads only its own
    S_j draft tokens via its draft page-table row; its token at position s
    attends its ancestors and itself (draft_visible: u <= s for a chain).

    Returns (o_B [rows, Hq, d], lse_B [rows, Hq])."""
    R, Hq, d = wl.q.shape
    o = np.zeros((R, Hq, d))
    lse = np.full((R, Hq), -np.inf)
    qo = wl.branch_qo_indptr
    brs = range(wl.num_branches) if branches is None else branches
    for j in brs:
        r0, r1 = int(qo[j]), int(qo[j + 1])
        k, v = _draft_kv(wl, j)
        for s in range(r1 - r0):
            vis = draft_visible(wl, j, s)
            for h in range(Hq):
                g = _kv_head(h, Hq, wl.num_kv_heads)
                oo, ll = attention_state(wl.q[r0 + s, h][None], k[vis, g],
                                         v[vis, g], wl.sm_scale)
                o[r0 + s, h], lse[r0 + s, h] = oo[0], ll[0]
    return o, lse


def cascade(wl):
    """Pass A, pass B, then merge_state: the cascade result for every row."""
    o_a, lse_a = prefix_pass(wl)
    o_b, lse_b = draft_pass(wl)
    return merge_state(o_a, lse_a, o_b, lse_b)


# ---------------------------------------------------------------------------
# Naive expansion: the plain definition of the result
# ---------------------------------------------------------------------------

def naive_expand(wl, rows=None):
    """One softmax per (row, head) over everything the row may see.

    Row r is position s of branch j of request i.  Its visible keys are the
    L_i prefix tokens of request i and the draft tokens of branch j that s
    attends (0..s for a chain), read through the two page tables (each virtual
    request re-reads the prefix).

    rows: optional iterable of global row ids; others stay (0, -inf).
    Returns (o [rows, Hq, d], lse [rows, Hq])."""
    R, Hq, d = wl.q.shape
    o = np.zeros((R, Hq, d))
    lse = np.full((R, Hq), -np.inf)
    req_of = _request_of_branch(wl.req_branch_indptr)
    br_of = _branch_of_row(wl.branch_qo_indptr)
    qo = wl.branch_qo_indptr
    want = np.arange(R) if rows is None else np.unique(np.asarray(list(rows), np.int64))
    by_branch = {}
    for r in want:
        by_branch.setdefault(int(br_of[r]), []).append(int(r))
    for j, rs in by_branch.items():
        i = int(req_of[j])
        kp, vp = _prefix_kv(wl, i)
        kd, vd = _draft_kv(wl, j)
        for r in rs:
            s = r - int(qo[j])
            vis = draft_visible(wl, j, s)
            k = np.concatenate([kp, kd[vis]], axis=0)
            v = np.concatenate([vp, vd[vis]], axis=0)
            for h in range(Hq):
                g = _kv_head(h, Hq, wl.num_kv_heads)
                oo, ll = attention_state(wl.q[r, h][None], k[:, g], v[:, g], wl.sm_scale)
                o[r, h], lse[r, h] = oo[0], ll[0]
    return o, lse


def cascade_rows(wl, rows):
    """Cascade result (pass A, pass B, merge) for selected global rows only.

    Rows are grouped by request and by kv head so that one prefix gather and
    one pass-A call serve all selected rows of a request; pass B runs per row
    over that row's visible drafts.  Returns (rows, o [n, Hq, d], lse [n, Hq])."""
    R, Hq, d = wl.q.shape
    Hkv = wl.num_kv_heads
    grp = Hq // Hkv
    rows = np.unique(np.asarray(list(rows), np.int64))
    req_of = _request_of_branch(wl.req_branch_indptr)
    br_of = _branch_of_row(wl.branch_qo_indptr)
    qo = wl.branch_qo_indptr
    n = rows.size
    o_a = np.zeros((n, Hq, d)); lse_a = np.full((n, Hq), -np.inf)
    o_b = np.zeros((n, Hq, d)); lse_b = np.full((n, Hq), -np.inf)
    by_req = {}
    for x, r in enumerate(rows):
        by_req.setdefault(int(req_of[br_of[r]]), []).append(x)
    for i, xs in by_req.items():
        xs = np.array(xs)
        kp, vp = _prefix_kv(wl, i)
        drafts = {}
        for g in range(Hkv):
            hs = [h for h in range(Hq) if _kv_head(h, Hq, Hkv) == g]
            q = wl.q[rows[xs]][:, hs].reshape(-1, d)
            oo, ll = attention_state(q, kp[:, g], vp[:, g], wl.sm_scale)
            o_a[np.ix_(xs, hs)] = oo.reshape(xs.size, len(hs), d)
            lse_a[np.ix_(xs, hs)] = ll.reshape(xs.size, len(hs))
        for x in xs:
            r = int(rows[x]); j = int(br_of[r]); s = r - int(qo[j])
            if j not in drafts:
                drafts[j] = _draft_kv(wl, j)
            kd, vd = drafts[j]
            vis = draft_visible(wl, j, s)
            for g in range(Hkv):
                hs = [h for h in range(Hq) if _kv_head(h, Hq, Hkv) == g]
                oo, ll = attention_state(wl.q[r, hs], kd[vis, g], vd[vis, g], wl.sm_scale)
                o_b[x, hs], lse_b[x, hs] = oo, ll
    o, lse = merge_state(o_a, lse_a, o_b, lse_b)
    return rows, o, lse


# ---------------------------------------------------------------------------
# Visibility and counters
# ---------------------------------------------------------------------------

def visibility_mask(wl, j):
    """Branch j's visibility over [its request's prefix ; its own drafts]:
    bool [S_j, L_i + S_j], True where row s may attend the key."""
    i = int(_request_of_branch(wl.req_branch_indptr)[j])
    L = int(wl.cache_seqlens[i])
    S = int(wl.branch_qo_indptr[j + 1] - wl.branch_qo_indptr[j])
    m = np.zeros((S, L + S), bool)
    for s in range(S):
        m[s, :L] = True
        m[s, L + draft_visible(wl, j, s)] = True
    return m


def kv_read_counts(cache_seqlens, req_branch_indptr, branch_qo_indptr):
    """KV tokens read by each scheme (cascade page).

    naive: every virtual request (branch) reads its request's prefix and its own
    drafts; cascade: each prefix once per request, each branch's drafts once."""
    L = np.asarray(cache_seqlens, np.int64)
    req_of = _request_of_branch(req_branch_indptr)
    S = np.diff(np.asarray(branch_qo_indptr, np.int64))
    naive = int(sum(L[req_of[j]] + S[j] for j in range(S.shape[0])))
    casc = int(L.sum() + S.sum())
    return naive, casc


def visible_pairs(wl):
    """Number of visible (query row, key) pairs per head, counted from the
    visibility of every row."""
    total = 0
    for j in range(wl.num_branches):
        total += int(visibility_mask(wl, j).sum())
    return total


def causal_pairs(n_tokens, n_hit):
    """Visible (query, key) pairs left to compute in a causal prompt of N tokens
    whose first H are a prefix-cache hit, counted by enumerating the grid:
    query p (1-based) sees keys 1..p; queries 1..H are already done."""
    count = 0
    for p in range(n_hit + 1, n_tokens + 1):
        for t in range(1, n_tokens + 1):
            if t <= p:
                count += 1
    return count
