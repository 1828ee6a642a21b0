"""Pins of the fp64 oracle to facts fixed outside of it (CPU only).

Each pin compares the oracle with something it does not share code with:
torch's scaled_dot_product_attention / logsumexp (library routines), a dense
brute force built from the tree-attention ancestor mask, closed forms, and the
numbers the pages print (tests/golden/).  ``test_planted_mistakes`` plants
plausible mistakes into a private copy of the oracle and checks that at least
one pin fails for each.
"""

import importlib.util
import json
import math
import os

import numpy as np
import pytest
import torch

from cascade_attention_tree_amd import workload as W

HERE = os.path.dirname(os.path.abspath(__file__))
ORACLE_PATH = os.path.join(os.path.dirname(HERE), "oracle", "cascade_oracle.py")


def load_oracle(mutation=None):
    """Fresh module object from the oracle source, optionally with one textual
    replacement applied (for planted-mistake checks)."""
    src = open(ORACLE_PATH, encoding="utf-8").read()
    if mutation is not None:
        old, new = mutation
        assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
        src = src.replace(old, new)
    spec = importlib.util.spec_from_loader("cascade_oracle_copy", loader=None)
    mod = importlib.util.module_from_spec(spec)
    exec(compile(src, ORACLE_PATH, "exec"), mod.__dict__)
    return mod


def golden(name):
    with open(os.path.join(HERE, "golden", name), encoding="utf-8") as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# Small workloads used by the pins
# ---------------------------------------------------------------------------

def wl_tiny():
    return W.tiny(values="fp32", keep_logical=True)


def wl_gqa_tree(seed=11):
    # GQA (group 3), ragged prefixes incl. an empty one, ragged branch counts/lengths.
    return W.build_workload("pin_gqa", [21, 0, 40], [[2, 4, 1], [3], [1, 5]], 6, 2, 16,
                            page_size=8, seed=seed, values="fp32", keep_logical=True)


def wl_topk1(seed=12):
    return W.build_workload("pin_topk1", [37, 5], [[6], [9]], 4, 2, 32, page_size=16,
                            seed=seed, values="fp32", keep_logical=True)


def wl_trees(seed=13):
    # One random draft tree per request (ragged prefixes incl. an empty one, a
    # 40-node tree), GQA group 3.
    wl = W.build_workload("pin_trees", [13, 0, 30], [[9], [5], [40]], 6, 2, 16, page_size=8,
                          seed=seed, values="fp32", keep_logical=True)
    return W.attach_random_trees(wl, seed + 1)


def wl_chain_masks(seed=14):
    # Chains written out as trees: node u's parent is u - 1.
    wl = W.build_workload("pin_chain_masks", [11, 3], [[4, 2], [6]], 4, 2, 16, page_size=8,
                          seed=seed, values="fp32", keep_logical=True)
    par = np.concatenate([np.arange(-1, s - 1) for s in np.diff(wl.branch_qo_indptr)]).astype(np.int32)
    wl.draft_parent = par
    wl.draft_mask = np.concatenate([(np.uint64(2) << np.arange(s, dtype=np.uint64)) - np.uint64(1)
                                    for s in np.diff(wl.branch_qo_indptr)]).astype(np.uint64)
    return wl


def wl_big_trees(seed=18):
    # Trees of more than 64 nodes (150 and 70: 3-word ancestor masks), and a
    # 130-node chain written out as a tree.
    wl = W.build_workload("pin_big_trees", [21, 0], [[150], [70]], 4, 2, 16, page_size=8,
                          seed=seed, values="fp32", keep_logical=True)
    return W.attach_random_trees(wl, seed + 1)


def wl_long_chain_masks(seed=20):
    wl = W.build_workload("pin_long_chain", [9], [[130]], 2, 1, 16, page_size=16,
                          seed=seed, values="fp32", keep_logical=True)
    S = 130
    wl.draft_parent = np.arange(-1, S - 1).astype(np.int32)
    m = [(1 << (u + 1)) - 1 for u in range(S)]
    wl.draft_mask = np.array([[(x >> (64 * w)) & 0xFFFFFFFFFFFFFFFF for w in range(3)] for x in m], np.uint64)
    return wl


def ancestors(wl, j, s):
    """Draft node s of branch j and its ancestors, by walking the parent array
    (chains: parent u - 1)."""
    out, u = [], s
    while u >= 0:
        out.append(u)
        u = int(wl.draft_parent[int(wl.branch_qo_indptr[j]) + u]) if wl.draft_parent is not None else u - 1
    return sorted(out)


# ---------------------------------------------------------------------------
# Independent formulations
# ---------------------------------------------------------------------------

def brute_force_tree(wl):
    """Dense attention per request over its BFS-flattened token tree.

    Nodes: the prefix chain, then the draft nodes level by level across the
    branches.  Each node's parent is the previous prefix token or its parent
    draft node (for a chain the previous draft token of its branch; roots hang
    off the last prefix token).  Mask[x, y] = y is an ancestor of x or x
    itself, found by walking parents.  Attention is
    torch's scaled_dot_product_attention (GQA by the library), the LSE is
    torch.logsumexp over the masked scores.  Uses the logical (unpaged) tensors
    only, never a page table."""
    R, Hq, d = wl.q.shape
    Hkv = wl.num_kv_heads
    o = np.zeros((R, Hq, d))
    lse = np.zeros((R, Hq))
    rb, qo = wl.req_branch_indptr, wl.branch_qo_indptr
    for i in range(wl.batch_size):
        L = int(wl.cache_seqlens[i])
        branches = list(range(int(rb[i]), int(rb[i + 1])))
        nodes = [("p", t) for t in range(L)]
        depth = max(int(qo[j + 1] - qo[j]) for j in branches)
        for u in range(depth):
            for j in branches:
                if u < qo[j + 1] - qo[j]:
                    nodes.append(("d", j, u))
        index = {n: x for x, n in enumerate(nodes)}

        def parent(n):
            if n[0] == "p":
                return ("p", n[1] - 1) if n[1] > 0 else None
            _, j, u = n
            pu = u - 1
            if wl.draft_parent is not None:
                pu = int(wl.draft_parent[int(qo[j]) + u])
            if pu >= 0:
                return ("d", j, pu)
            return ("p", L - 1) if L > 0 else None

        n_all = len(nodes)
        mask = np.zeros((n_all, n_all), bool)
        for x, n in enumerate(nodes):
            a = n
            while a is not None:
                mask[x, index[a]] = True
                a = parent(a)
        K = np.zeros((n_all, Hkv, d)); V = np.zeros((n_all, Hkv, d))
        qrows = []
        for x, n in enumerate(nodes):
            if n[0] == "p":
                K[x] = wl.prefix_k[i][n[1]]; V[x] = wl.prefix_v[i][n[1]]
            else:
                _, j, u = n
                K[x] = wl.draft_k[j][u]; V[x] = wl.draft_v[j][u]
                qrows.append((x, int(qo[j]) + u))
        xs = [x for x, _ in qrows]
        rows = [r for _, r in qrows]
        q_t = torch.from_numpy(wl.q[rows].astype(np.float64)).permute(1, 0, 2)[None]
        k_t = torch.from_numpy(K).permute(1, 0, 2)[None]
        v_t = torch.from_numpy(V).permute(1, 0, 2)[None]
        m_t = torch.from_numpy(mask[xs])
        out = torch.nn.functional.scaled_dot_product_attention(
            q_t, k_t, v_t, attn_mask=m_t, scale=wl.sm_scale, enable_gqa=True)
        o[rows] = out[0].permute(1, 0, 2).numpy()
        k_rep = k_t.repeat_interleave(Hq // Hkv, dim=1)
        sc = (q_t @ k_rep.transpose(-1, -2)) * wl.sm_scale
        sc = sc.masked_fill(~m_t, float("-inf"))
        lse[rows] = torch.logsumexp(sc, dim=-1)[0].permute(1, 0).numpy()
    return o, lse


# ---------------------------------------------------------------------------
# The pins.  Each takes the oracle module so planted mistakes can be checked.
# ---------------------------------------------------------------------------

def pin_gather(O):
    """Page gather reproduces the logical token order drawn before paging."""
    hit = W.prefix_hit(0.5, values="fp32", keep_logical=True, batch=2, n_tokens=45)
    for wl in (wl_tiny(), wl_gqa_tree(), hit):
        for i in range(wl.batch_size):
            L = int(wl.cache_seqlens[i])
            k = O.gather_slots(wl.k_pool, wl.page_table[i], 0, L, wl.page_size)
            assert np.array_equal(k, wl.prefix_k[i].astype(np.float64))
        for j in range(wl.num_branches):
            S = int(wl.branch_qo_indptr[j + 1] - wl.branch_qo_indptr[j])
            v = O.gather_slots(wl.v_pool, wl.draft_page_table[j], wl.draft_start[j], S,
                               wl.page_size)
            assert np.array_equal(v, wl.draft_v[j].astype(np.float64))


def pin_single_key(O):
    """One key: o is its value, LSE is its scaled score."""
    rng = np.random.default_rng(5)
    q, k, v = rng.standard_normal((3, 8)), rng.standard_normal((1, 8)), rng.standard_normal((1, 5))
    o, lse = O.attention_state(q, k, v, 0.3)
    assert np.allclose(o, np.repeat(v, 3, axis=0), rtol=0, atol=1e-14)
    assert np.allclose(lse, 0.3 * (q @ k.T)[:, 0], rtol=0, atol=1e-14)


def pin_attention_vs_library(O):
    """attention_state against torch SDPA and torch.logsumexp in float64."""
    rng = np.random.default_rng(6)
    for n, m, d, dv in ((1, 1, 4, 4), (5, 17, 16, 16), (7, 64, 64, 32)):
        q, k, v = (rng.standard_normal(s) * 2 for s in ((n, d), (m, d), (m, dv)))
        scale = 1.0 / math.sqrt(d)
        o, lse = O.attention_state(q, k, v, scale)
        qt, kt, vt = (torch.from_numpy(x) for x in (q, k, v))
        ref = torch.nn.functional.scaled_dot_product_attention(qt[None], kt[None], vt[None],
                                                               scale=scale)[0].numpy()
        ref_lse = torch.logsumexp(qt @ kt.T * scale, dim=-1).numpy()
        assert np.max(np.abs(o - ref)) < 1e-12
        assert np.max(np.abs(lse - ref_lse)) < 1e-12


def pin_merge_identity(O):
    """merge(state(A), state(B)) == state(A u B) for random splits, empty sides included."""
    rng = np.random.default_rng(7)
    for trial in range(40):
        m = int(rng.integers(1, 48))
        d = 16
        q = rng.standard_normal((4, d)) * 1.5
        k = rng.standard_normal((m, d)) * 1.5
        v = rng.standard_normal((m, d))
        sel = rng.random(m) < rng.random()
        if trial == 0:
            sel[:] = True          # B empty
        if trial == 1:
            sel[:] = False         # A empty
        full_o, full_l = O.attention_state(q, k, v, 0.25)
        oa, la = O.attention_state(q, k[sel], v[sel], 0.25)
        ob, lb = O.attention_state(q, k[~sel], v[~sel], 0.25)
        o, l = O.merge_state(oa, la, ob, lb)
        assert np.max(np.abs(o - full_o)) < 1e-12
        assert np.max(np.abs(l - full_l)) < 1e-12
        o2, l2 = O.merge_state(ob, lb, oa, la)   # order of the two parts is free
        assert np.max(np.abs(o2 - full_o)) < 1e-12 and np.max(np.abs(l2 - full_l)) < 1e-12


def pin_merge_closed_forms(O):
    """Equal LSEs: LSE + ln 2 and the mean of the two outputs.  One side empty:
    the other side unchanged.  Both empty: (0, -inf).  Huge LSEs: no overflow."""
    rng = np.random.default_rng(8)
    oa, ob = rng.standard_normal((3, 6)), rng.standard_normal((3, 6))
    la = np.array([0.5, -3.0, 700.0])
    o, l = O.merge_state(oa, la, ob, la)
    assert np.allclose(l, la + math.log(2.0), rtol=0, atol=1e-12)
    assert np.allclose(o, 0.5 * (oa + ob), rtol=0, atol=1e-12)
    ninf = np.full(3, -np.inf)
    o, l = O.merge_state(oa, la, ob, ninf)
    assert np.array_equal(l, la) and np.allclose(o, oa, rtol=0, atol=1e-15)
    o, l = O.merge_state(oa, ninf, ob, la)
    assert np.array_equal(l, la) and np.allclose(o, ob, rtol=0, atol=1e-15)
    o, l = O.merge_state(oa, ninf, ob, ninf)
    assert np.all(np.isneginf(l)) and np.all(o == 0)
    # weights e^(LSE_A - LSE) : e^(LSE_B - LSE) = e^1 : 1
    o, l = O.merge_state(oa, la + 1.0, ob, la)
    wa = math.e / (math.e + 1.0)
    assert np.allclose(o, wa * oa + (1 - wa) * ob, rtol=0, atol=1e-12)
    assert np.allclose(l, la + 1.0 + math.log1p(math.exp(-1.0)), rtol=0, atol=1e-12)


def pin_brute_force(O):
    """Oracle naive expansion and cascade == dense tree-mask brute force, also on
    a prefix-hit shape (one branch continuing the prefix inside its pages)."""
    hit = W.prefix_hit(0.5, values="fp32", keep_logical=True, batch=2, n_tokens=45)
    for wl in (wl_tiny(), wl_gqa_tree(), wl_topk1(), hit, wl_trees()):
        ref_o, ref_l = brute_force_tree(wl)
        for o, l in (O.naive_expand(wl), O.cascade(wl)):
            assert np.max(np.abs(o - ref_o)) < 1e-12
            assert np.max(np.abs(l - ref_l)) < 1e-12
        rows, o, l = O.cascade_rows(wl, [0, wl.total_rows - 1, wl.total_rows // 2])
        assert np.max(np.abs(o - ref_o[rows])) < 1e-12
        assert np.max(np.abs(l - ref_l[rows])) < 1e-12


def pin_topk1_is_causal(O):
    """With one branch, the cascade equals one causal pass over L + S keys whose
    queries are the last S positions (library SDPA, is_causal on the full
    sequence)."""
    wl = wl_topk1()
    o, l = O.cascade(wl)
    qo, Hq, Hkv = wl.branch_qo_indptr, wl.num_qo_heads, wl.num_kv_heads
    for i in range(wl.batch_size):
        j = int(wl.req_branch_indptr[i])
        L, S = int(wl.cache_seqlens[i]), int(qo[j + 1] - qo[j])
        K = np.concatenate([wl.prefix_k[i], wl.draft_k[j]]).astype(np.float64)
        V = np.concatenate([wl.prefix_v[i], wl.draft_v[j]]).astype(np.float64)
        Q = np.zeros((L + S, Hq, wl.head_dim))
        Q[L:] = wl.q[qo[j]:qo[j + 1]]
        t = lambda x: torch.from_numpy(x).permute(1, 0, 2)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            t(Q), t(K), t(V), is_causal=True, scale=wl.sm_scale, enable_gqa=True)
        ref = ref[0].permute(1, 0, 2).numpy()[L:]
        assert np.max(np.abs(o[qo[j]:qo[j + 1]] - ref)) < 1e-12
        kk = t(K).repeat_interleave(Hq // Hkv, dim=1)
        sc = (t(Q) @ kk.transpose(-1, -2)) * wl.sm_scale
        causal = torch.ones(L + S, L + S, dtype=torch.bool).tril()
        ref_l = torch.logsumexp(sc.masked_fill(~causal, float("-inf")), -1)[0].T.numpy()[L:]
        assert np.max(np.abs(l[qo[j]:qo[j + 1]] - ref_l)) < 1e-12


def pin_zero_query(O):
    """q = 0 makes every visible key weigh the same: LSE = ln(L_i + n) with n the
    row's node and its ancestors (s + 1 on a chain), and o is the plain mean of
    the visible values."""
    for wl in (wl_tiny(), wl_gqa_tree(), wl_trees()):
        wl.q[:] = 0.0
        qo, rb = wl.branch_qo_indptr, wl.req_branch_indptr
        g_of = np.arange(wl.num_qo_heads) // (wl.num_qo_heads // wl.num_kv_heads)
        for fn in (O.naive_expand, O.cascade):
            o, l = fn(wl)
            for i in range(wl.batch_size):
                L = int(wl.cache_seqlens[i])
                for j in range(int(rb[i]), int(rb[i + 1])):
                    for s in range(int(qo[j + 1] - qo[j])):
                        r = int(qo[j]) + s
                        anc = ancestors(wl, j, s)
                        assert np.allclose(l[r], math.log(L + len(anc)), rtol=0, atol=1e-13)
                        vis = np.concatenate([wl.prefix_v[i], wl.draft_v[j][anc]]).astype(np.float64)
                        assert np.allclose(o[r], vis.mean(axis=0)[g_of], rtol=0, atol=1e-13)


def pin_chain_as_tree(O):
    """Chains given as trees (parent u - 1, mask of bits 0..u) give the same bits
    as the same workload without a tree; the generator's tree masks are exactly
    the ancestor sets of its parent arrays."""
    wl = wl_chain_masks()
    o1, l1 = O.cascade(wl)
    n1, m1 = O.naive_expand(wl)
    wl.draft_parent, wl.draft_mask = None, None
    o0, l0 = O.cascade(wl)
    n0, m0 = O.naive_expand(wl)
    assert np.array_equal(o1, o0) and np.array_equal(l1, l0)
    assert np.array_equal(n1, n0) and np.array_equal(m1, m0)
    # Past 64 nodes the masks span several words: a long chain as a tree again
    # gives the chain's bits, and random trees' masks are their ancestor sets.
    wl = wl_long_chain_masks()
    assert wl.draft_mask.shape == (130, 3)
    o1, l1 = O.cascade(wl)
    wl.draft_parent, wl.draft_mask = None, None
    o0, l0 = O.cascade(wl)
    assert np.array_equal(o1, o0) and np.array_equal(l1, l0)
    for wl in (wl_trees(), wl_big_trees()):
        for j in range(wl.num_branches):
            S = int(wl.branch_qo_indptr[j + 1] - wl.branch_qo_indptr[j])
            vm = O.visibility_mask(wl, j)
            L = vm.shape[1] - S
            for s in range(S):
                assert list(O.draft_visible(wl, j, s)) == ancestors(wl, j, s)
                assert vm[s, L:].nonzero()[0].tolist() == ancestors(wl, j, s)


def pin_append_commit(O):
    """Appended drafts read back through the draft block tables as written, every
    other slot untouched; committed rows extend the prefix in path order and
    lengths grow by their count; committing nothing changes nothing."""
    import copy
    hit = W.prefix_hit(0.5, values="fp32", keep_logical=True, batch=2, n_tokens=45)
    for wl in (wl_tiny(), wl_gqa_tree(), hit):
        wl.k_pool = np.nan_to_num(wl.k_pool, nan=7.0)
        wl.v_pool = np.nan_to_num(wl.v_pool, nan=7.0)
        rng = np.random.default_rng(21)
        R = wl.total_rows
        k_new = rng.standard_normal((R, wl.num_kv_heads, wl.head_dim)).astype(np.float32)
        v_new = rng.standard_normal((R, wl.num_kv_heads, wl.head_dim)).astype(np.float32)
        k2, v2 = O.append_draft_kv(wl, k_new, v_new)
        qo, P = wl.branch_qo_indptr, wl.page_size
        written = np.zeros(wl.k_pool.shape[:2], bool)
        for j in range(wl.num_branches):
            r0, r1 = int(qo[j]), int(qo[j + 1])
            u = int(wl.draft_start[j]) + np.arange(r1 - r0)
            pages = wl.draft_page_table[j][u // P]
            assert np.array_equal(k2[pages, u % P], k_new[r0:r1])
            assert np.array_equal(v2[pages, u % P], v_new[r0:r1])
            written[pages, u % P] = True
        assert np.array_equal(k2[~written], wl.k_pool[~written])
        assert np.array_equal(v2[~written], wl.v_pool[~written])
        # room for the committed tokens: one fresh page per request, appended to
        # the pool and to the end of each block-table row
        B_, npg = wl.batch_size, wl.k_pool.shape[0]
        fresh = np.zeros((B_,) + wl.k_pool.shape[1:], np.float32)
        w2 = copy.copy(wl)
        w2.k_pool = np.concatenate([k2, fresh]); w2.v_pool = np.concatenate([v2, fresh])
        cols = -(-(wl.cache_seqlens.max() + 2) // P)
        pt = np.full((B_, max(cols, wl.page_table.shape[1])), -1, np.int32)
        pt[:, :wl.page_table.shape[1]] = wl.page_table
        for i in range(B_):
            pt[i, wl.page_table.shape[1]:] = npg + i
        w2.page_table = pt
        k2, v2 = w2.k_pool, w2.v_pool
        # accept a path per request: the first rows of its first branch
        rb = wl.req_branch_indptr
        acc, ind = [], [0]
        for i in range(wl.batch_size):
            j = int(rb[i])
            n = min(2, int(qo[j + 1] - qo[j]))
            acc += list(range(int(qo[j]), int(qo[j]) + n))
            ind.append(len(acc))
        k3, v3, lens = O.commit_accepted(w2, np.array(ind), np.array(acc))
        for i in range(wl.batch_size):
            L, n = int(wl.cache_seqlens[i]), ind[i + 1] - ind[i]
            assert lens[i] == L + n
            t = L + np.arange(n)
            pages = w2.page_table[i][t // P]
            assert np.array_equal(k3[pages, t % P], k_new[acc[ind[i]:ind[i + 1]]])
            assert np.array_equal(v3[pages, t % P], v_new[acc[ind[i]:ind[i + 1]]])
        k4, v4, lens4 = O.commit_accepted(w2, np.zeros(wl.batch_size + 1, int), np.zeros(0, int))
        assert np.array_equal(k4, k2) and np.array_equal(v4, v2)
        assert np.array_equal(lens4, wl.cache_seqlens)


def pin_read_counts(O):
    """The pages' worked example and formulas for KV tokens read."""
    g = golden("cascade_worked_example.json")
    B, topk, L, S = 32, g["topk"], g["prefix_len"], g["draft_len"]
    rb = np.arange(0, B * topk + 1, topk)
    qo = np.arange(0, B * topk * S + 1, S)
    naive, casc = O.kv_read_counts(np.full(B, L), rb, qo)
    assert naive == B * g["naive_kv_tokens_per_request"]
    assert casc == B * g["cascade_kv_tokens_per_request"]
    assert round(naive / casc) == g["saving_approx"]
    # the formulas: B*topk*(L+S) and B*L + B*topk*S, at the other configurations
    for (B, L, topk, S, per_naive, per_casc) in ((8, 1000, 4, 3, 4012, 1012), (2, 32, 2, 3, 70, 38)):
        rb = np.arange(0, B * topk + 1, topk)
        qo = np.arange(0, B * topk * S + 1, S)
        naive, casc = O.kv_read_counts(np.full(B, L), rb, qo)
        assert naive == B * topk * (L + S) == B * per_naive
        assert casc == B * L + B * topk * S == B * per_casc
    # ragged: per request sums
    wl = wl_gqa_tree()
    naive, casc = O.kv_read_counts(wl.cache_seqlens, wl.req_branch_indptr, wl.branch_qo_indptr)
    assert naive == (21 + 2) + (21 + 4) + (21 + 1) + (0 + 3) + (40 + 1) + (40 + 5)
    assert casc == (21 + 0 + 40) + (2 + 4 + 1 + 3 + 1 + 5)


def pin_prefix_hit_pairs(O):
    """Visible pairs after a prefix hit: the page's 8-token diagram, the closed form
    N(N+1)/2 - H(H+1)/2 = M*H + M(M+1)/2, and the oracle's own visibility sets on
    the prefix-hit workload shape."""
    g = golden("prefix_hit_diagram.json")
    N, H = g["n_tokens"], g["n_hit"]
    assert O.causal_pairs(N, 0) == g["pairs_full_triangle"]
    assert O.causal_pairs(N, H) == g["pairs_remaining_after_hit"]
    for (N, H) in ((8, 4), (50, 0), (50, 17), (64, 63), (64, 64)):
        M = N - H
        assert O.causal_pairs(N, H) == M * H + M * (M + 1) // 2 == (N * (N + 1) - H * (H + 1)) // 2
    # the prefix-hit workload expressed as a one-branch tree has exactly these pairs
    for h in (0.0, 0.5, 0.9):
        wl = W.prefix_hit(h, values="fp32", batch=2, n_tokens=40)
        H = int(math.floor(h * 40))
        assert O.visible_pairs(wl) == 2 * O.causal_pairs(40, H)
    ratio = lambda N, H: 1 - H * (H + 1) / (N * (N + 1))
    assert abs(ratio(8192, 4096) - 0.7499695) < 1e-7
    assert abs(ratio(8192, 7372) - 0.1901648) < 1e-7
    assert abs(ratio(8192, 4096) - g["half_hit_remaining_fraction_approx"]) < 1e-3


def pin_block_table_sharing(O):
    """Two block tables sharing their first two physical pages (tutorial page,
    section 5.3): the shared 32 tokens gather identically and give identical
    prefix states for identical queries."""
    g = golden("block_table_example.json")
    P = g["page_size"]
    rng = np.random.default_rng(9)
    num_pages = 40
    k_pool = rng.standard_normal((num_pages, P, 2, 8)).astype(np.float32)
    v_pool = rng.standard_normal((num_pages, P, 2, 8)).astype(np.float32)
    a, b = g["request_a_pages"], g["request_b_pages"]
    n = g["shared_tokens"]
    ka = O.gather_slots(k_pool, a, 0, n, P)
    kb = O.gather_slots(k_pool, b, 0, n, P)
    assert np.array_equal(ka, kb)
    assert not np.array_equal(O.gather_slots(k_pool, a, 0, n + P, P),
                              O.gather_slots(k_pool, b, 0, n + P, P))
    pt = np.array([a, b + [0]], np.int32)
    q = rng.standard_normal((2, 4, 8)).astype(np.float32)
    q[1] = q[0]
    wl = W.Workload(name="alias", num_qo_heads=4, num_kv_heads=2, head_dim=8, page_size=P,
                    sm_scale=8 ** -0.5, q=q, k_pool=k_pool, v_pool=v_pool, page_table=pt,
                    cache_seqlens=np.array([n, n], np.int32),
                    req_branch_indptr=np.array([0, 1, 2], np.int32),
                    branch_qo_indptr=np.array([0, 1, 2], np.int32),
                    draft_page_table=np.array([[30], [31]], np.int32),
                    draft_start=np.zeros(2, np.int32))
    o, l = O.prefix_pass(wl)
    assert np.array_equal(o[0], o[1]) and np.array_equal(l[0], l[1])


def pin_e4m3_values(O):
    """FP8 E4M3 decode: values fixed by the format's definition, then every
    code against torch's float8_e4m3fn conversion (a library routine)."""
    fixed = {0x00: 0.0, 0x80: -0.0, 0x38: 1.0, 0xB8: -1.0, 0x40: 2.0, 0x3C: 1.5,
             0x7E: 448.0, 0xFE: -448.0, 0x08: 2.0 ** -6, 0x07: 7 * 2.0 ** -9,
             0x01: 2.0 ** -9, 0x81: -(2.0 ** -9), 0x30: 0.5, 0x28: 0.25, 0x77: 240.0}
    codes = np.array(sorted(fixed), np.uint8)
    got = O.e4m3_value(codes)
    want = np.array([fixed[int(c)] for c in codes])
    assert np.array_equal(got, want) and np.array_equal(np.signbit(got), np.signbit(want))
    assert np.all(np.isnan(O.e4m3_value(np.array([0x7F, 0xFF], np.uint8))))
    allc = np.arange(256, dtype=np.uint8)
    lib = torch.from_numpy(allc.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = O.e4m3_value(allc)
    assert np.array_equal(np.isnan(ours), np.isnan(lib))
    fin = ~np.isnan(lib)
    assert np.array_equal(ours[fin], lib[fin])


def wl_fp8(seed=15):
    wl = W.build_workload("fp8", [37, 0, 70], [[3, 2], [4], [1, 5]], 4, 2, 16, 16, seed=seed,
                          values="fp32")
    wl.v_pool = wl.v_pool * np.float32(3.0)   # distinct K and V scales
    return W.with_fp8_kv(wl)


def pin_fp8_dequantize(O):
    """The dequantised pools are the codes' values times the per-tensor scales
    (torch's decode of the same codes), and lie within the format's rounding
    bound of the values that were quantised: half a unit in the last place,
    i.e. 2^-4 relative for normal codes, 2^-10 * scale for subnormal ones."""
    wl = wl_fp8()
    assert wl.k_scale != wl.v_scale
    dq = O.dequantize_kv(wl)
    for codes, scale, pool, ref in ((wl.k_codes, wl.k_scale, dq.k_pool, wl.k_pool),
                                    (wl.v_codes, wl.v_scale, dq.v_pool, wl.v_pool)):
        lib = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy() * scale
        assert np.array_equal(np.isnan(pool), np.isnan(lib))
        fin = ~np.isnan(lib)
        assert np.array_equal(pool[fin], lib[fin])
        assert np.array_equal(np.isnan(pool), np.isnan(ref))
        x = ref[fin].astype(np.float64)
        bound = np.maximum(np.abs(x) * 2.0 ** -4, scale * 2.0 ** -10) * (1 + 1e-12)
        assert np.all(np.abs(pool[fin] - x) <= bound)
    # A code of 1.0 stands for the scale itself.
    wl.v_codes[0, 0, 0, :2] = [0x38, 0xB8]
    dq = O.dequantize_kv(wl)
    assert dq.v_pool[0, 0, 0, 0] == wl.v_scale and dq.v_pool[0, 0, 0, 1] == -wl.v_scale


def pin_fp8_channel_dequantize(O):
    """Per-channel FP8 scales (tutorial page, section 4.5): element
    (page, slot, g, c) stands for value(code) * scale * channel_scale[g, c].
    Checked against torch's decode of the same codes times the channel scales,
    against the format's rounding bound of the quantised values (per channel:
    2^-4 relative for normal codes, 2^-10 * channel scale for subnormal ones),
    and in the special case of equal channel scales, which is the per-tensor
    case with that scale."""
    base = W.build_workload("fp8c", [37, 0, 70], [[3, 2], [4], [1, 5]], 4, 2, 16, 16, seed=16,
                            values="fp32")
    wl = W.with_fp8_kv(base, per_channel=True, channel_spread=3.0, seed=17)
    assert wl.k_channel_scale.shape == (2, 16) and np.ptp(wl.k_channel_scale) > 0
    assert not np.array_equal(wl.k_channel_scale, wl.v_channel_scale)
    dq = O.dequantize_kv(wl)
    for codes, cs, pool in ((wl.k_codes, wl.k_channel_scale, dq.k_pool), (wl.v_codes, wl.v_channel_scale, dq.v_pool)):
        lib = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        lib = lib * cs.astype(np.float64)[None, None, :, :]
        assert np.array_equal(np.isnan(pool), np.isnan(lib))
        fin = ~np.isnan(lib)
        assert np.array_equal(pool[fin], lib[fin])
    spread = W.with_fp8_kv(base, per_channel=False, channel_spread=3.0, seed=17)  # the same spread pools
    for ref, pool, cs in ((spread.k_pool, dq.k_pool, wl.k_channel_scale), (spread.v_pool, dq.v_pool, wl.v_channel_scale)):
        fin = np.isfinite(ref)
        x = ref.astype(np.float64)
        bound = np.maximum(np.abs(x) * 2.0 ** -4, cs.astype(np.float64)[None, None] * 2.0 ** -10) * (1 + 1e-12)
        assert np.all(np.abs(pool - x)[fin] <= bound[fin])
    # Equal channel scales s: the per-tensor dequantisation with scale s.
    import dataclasses
    s = np.float32(0.37)
    same = dataclasses.replace(wl, k_channel_scale=np.full_like(wl.k_channel_scale, s),
                               v_channel_scale=np.full_like(wl.v_channel_scale, s))
    tensor = dataclasses.replace(wl, k_channel_scale=None, v_channel_scale=None, k_scale=float(s), v_scale=float(s))
    a, b = O.dequantize_kv(same), O.dequantize_kv(tensor)
    assert np.array_equal(np.isnan(a.k_pool), np.isnan(b.k_pool))
    fin = ~np.isnan(a.k_pool)
    assert np.array_equal(a.k_pool[fin], b.k_pool[fin]) and np.array_equal(a.v_pool[fin], b.v_pool[fin])
    # A code of 1.0 in channel (g, c) stands for that channel's scale.
    wl.k_codes[0, 0, 1, 5] = 0x38
    assert O.dequantize_kv(wl).k_pool[0, 0, 1, 5] == float(wl.k_channel_scale[1, 5])


ALL_PINS = [pin_e4m3_values, pin_fp8_dequantize, pin_fp8_channel_dequantize, pin_gather, pin_single_key, pin_attention_vs_library, pin_merge_identity,
            pin_merge_closed_forms, pin_brute_force, pin_topk1_is_causal, pin_zero_query,
            pin_chain_as_tree, pin_append_commit, pin_read_counts, pin_prefix_hit_pairs,
            pin_block_table_sharing]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(load_oracle())


# Plausible mistakes, each a textual change of the oracle's source.
MUTATIONS = {
    "scale dropped": ("z = sm_scale * (q @ k.T)", "z = (q @ k.T)"),
    "log base 2": ("lse = zmax[:, 0] + np.log(tot[:, 0])", "lse = zmax[:, 0] + np.log2(tot[:, 0])"),
    "no max shift sign": ("w = np.exp(z - zmax)", "w = np.exp(z + zmax - 2 * zmax.max())"),
    "gqa modulo": ("return h // (num_qo_heads // num_kv_heads)", "return h % num_kv_heads"),
    "slot/page swapped": ("return np.asarray(pool[pages, t % page_size]", "return np.asarray(pool[pages, t // page_size % page_size]"),
    "draft excludes self (chains)": ("return np.arange(s + 1)", "return np.arange(s)"),
    "tree mask shifted": ("if (m >> u) & 1]", "if (m >> (u + 1)) & 1]"),
    "tree mask ignored": ("m = sum(int(x) << (64 * w) for w, x in enumerate(words))", "m = (2 << s) - 1"),
    "tree mask words reversed": ("m = sum(int(x) << (64 * w) for w, x in enumerate(words))",
                                 "m = sum(int(x) << (64 * w) for w, x in enumerate(words[::-1]))"),
    "naive drops the drafts": ("k = np.concatenate([kp, kd[vis]], axis=0)", "k = np.concatenate([kp, kd[vis[:1]]], axis=0)"),
    "merge weights swapped": ("o = wa[..., None] * o_a + wb[..., None] * o_b", "o = wb[..., None] * o_a + wa[..., None] * o_b"),
    "merge without log": ("lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, tot)))", "lse = np.where(empty, -np.inf, m_safe + np.where(empty, 1.0, tot) - 1)"),
    "prefix off by one": ("t = int(first_slot) + np.arange(int(count))", "t = int(first_slot) + 1 + np.arange(int(count))"),
    "naive reads prefix once": ("naive = int(sum(L[req_of[j]] + S[j] for j in range(S.shape[0])))", "naive = int(L.sum() + S.sum())"),
    "draft start ignored": ("s0 = int(wl.draft_start[j])", "s0 = 0"),
    "causal pairs strict": ("if t <= p:", "if t < p:"),
    "commit at the wrong slot": ("k_pool = scatter_slots(k_pool, wl.page_table[i], L, np.array(ks), wl.page_size)",
                                 "k_pool = scatter_slots(k_pool, wl.page_table[i], L + 1, np.array(ks), wl.page_size)"),
    "e4m3 exponent bias 8": ("np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int32))", "np.ldexp(1.0 + m / 8.0, (e - 8).astype(np.int32))"),
    "e4m3 subnormals as normals": ("np.ldexp(m / 8.0, -6)", "np.ldexp(1.0 + m / 8.0, -7)"),
    "e4m3 sign ignored": ("sign = np.where(c & 0x80, -1.0, 1.0)", "sign = np.where(c & 0x40, -1.0, 1.0)"),
    "fp8 scale dropped": ("k = e4m3_value(wl.k_codes) * float(wl.k_scale)", "k = e4m3_value(wl.k_codes)"),
    "fp8 V takes the K scale": ("v = e4m3_value(wl.v_codes) * float(wl.v_scale)", "v = e4m3_value(wl.v_codes) * float(wl.k_scale)"),
    "fp8 channel scale dropped": ("k = k * np.asarray(wl.k_channel_scale, np.float64)[None, None, :, :]", "k = k * 1.0"),
    "fp8 V takes the K channel scales": ("v = v * np.asarray(wl.v_channel_scale, np.float64)", "v = v * np.asarray(wl.k_channel_scale, np.float64)"),
    "append ignores draft_start": ("k_pool = scatter_slots(k_pool, wl.draft_page_table[j], int(wl.draft_start[j]),",
                                   "k_pool = scatter_slots(k_pool, wl.draft_page_table[j], 0,"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistakes(name):
    mutant = load_oracle(MUTATIONS[name])
    failed = []
    for pin in ALL_PINS:
        try:
            pin(mutant)
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"no pin catches the planted mistake '{name}'"


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(3).standard_normal(100000).astype(np.float32) * 7
    x[:4] = [0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8]   # ties to even
    ours = W.round_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours, ref)
