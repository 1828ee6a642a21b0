"""GPU: the writes of a serving step around verification, and a graph-captured
multi-layer verify step.

* cascade_append_draft_kv and cascade_commit_accepted against the oracle's
  append_draft_kv / commit_accepted, bit for bit on the whole pool (both page
  layouts), then a verify step over the committed prefix against the oracle.
* Several layers of (append, verify) captured in one HIP graph through torch,
  replayed several times with eager work in between; every replay equals the
  same sequence run eagerly, bit for bit.
"""

import copy
import sys

import numpy as np
import pytest
import torch

from cascade_attention_tree_amd import workload as W
from oracle import cascade_oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from cascade_attention_tree_amd import binding
    binding.lib()
    return binding


def note(msg):
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


def pool_bits_nhd(t, layout):
    """Device bf16 pool -> uint16 bits in the generator's [pages, P, Hkv, d] order."""
    if layout == "HND":
        t = t.permute(0, 2, 1, 3)
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def random_drafts(wl, seed):
    g = torch.Generator().manual_seed(seed)
    shape = (wl.total_rows, wl.num_kv_heads, wl.head_dim)
    k = torch.randn(shape, generator=g).to(torch.bfloat16)
    v = torch.randn(shape, generator=g).to(torch.bfloat16)
    return k, v


def with_room(wl, extra_tokens):
    """A copy of wl whose block-table rows map `extra_tokens` more slots past every
    prefix, in fresh pages appended to the pool (one run of pages per request)."""
    w = copy.copy(wl)
    P, npg = wl.page_size, wl.k_pool.shape[0]
    need = [-(-(int(L) + extra_tokens) // P) for L in wl.cache_seqlens]
    width = max(max(need), wl.page_table.shape[1])
    extra = width - wl.page_table.shape[1]
    pt = np.full((wl.batch_size, width), 0, np.int32)
    pt[:, :wl.page_table.shape[1]] = wl.page_table
    for i in range(wl.batch_size):
        pt[i, wl.page_table.shape[1]:] = npg + i * extra + np.arange(extra)
    fresh = np.zeros((wl.batch_size * extra,) + wl.k_pool.shape[1:], np.float32)
    w.k_pool = np.concatenate([wl.k_pool, fresh])
    w.v_pool = np.concatenate([wl.v_pool, fresh])
    w.page_table = pt
    return w


@pytest.mark.parametrize("layout", ["NHD", "HND"])
def test_append_and_commit_bit_exact(B, layout):
    base = W.build_workload("step", [40, 0, 75], [[3, 5], [2], [4, 1, 6]], 8, 2, 128, 16, seed=61)
    wl = with_room(base, 4)
    x = B.to_device(wl, layout=layout)
    k_new, v_new = random_drafts(wl, 7)
    note(f"append {layout}")
    B.cascade_append_draft_kv(x, k_new.cuda(), v_new.cuda())
    kn, vn = k_new.float().numpy(), v_new.float().numpy()
    ko, vo = O.append_draft_kv(wl, kn, vn)
    torch.cuda.synchronize()
    assert np.array_equal(pool_bits_nhd(x.k_pool, layout), W.bf16_bits(ko))
    assert np.array_equal(pool_bits_nhd(x.v_pool, layout), W.bf16_bits(vo))
    assert B.cascade_device_error(clear=True) == 0

    # accept, per request, a path of up to 3 rows of its first branch
    qo, rb = wl.branch_qo_indptr, wl.req_branch_indptr
    acc, ind = [], [0]
    for i in range(wl.batch_size):
        j = int(rb[i])
        n = min(3, int(qo[j + 1] - qo[j]))
        acc += list(range(int(qo[j]), int(qo[j]) + n))
        ind.append(len(acc))
    wa = copy.copy(wl)
    wa.k_pool, wa.v_pool = ko, vo
    kc, vc, lens = O.commit_accepted(wa, np.array(ind), np.array(acc))
    note(f"commit {layout}")
    B.cascade_commit_accepted(x, torch.tensor(ind, dtype=torch.int32, device="cuda"),
                              torch.tensor(acc, dtype=torch.int32, device="cuda"), 3)
    torch.cuda.synchronize()
    assert np.array_equal(x.cache_seqlens.cpu().numpy(), lens)
    assert np.array_equal(pool_bits_nhd(x.k_pool, layout), W.bf16_bits(kc))
    assert np.array_equal(pool_bits_nhd(x.v_pool, layout), W.bf16_bits(vc))
    assert B.cascade_device_error(clear=True) == 0

    # next step: the same rows verify over the committed prefix
    wn = copy.copy(wa)
    wn.k_pool, wn.v_pool, wn.cache_seqlens = kc, vc, lens
    x2 = B.to_device(wn, layout=layout)
    o, l = B.cascade_verify_attn(x2)
    ro, rl = O.cascade(wn)
    torch.cuda.synchronize()
    o = o.cpu().numpy().astype(np.float64)
    l = l.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(o - ro)) <= 1e-2
    fin = np.isfinite(rl)
    assert np.max(np.abs(l[fin] - rl[fin])) <= 1e-3 and np.array_equal(np.isneginf(l), np.isneginf(rl))


@pytest.mark.parametrize("layout", ["NHD", "HND"])
def test_commit_tree_path_skipping_nodes_in_prefix_pages(B, layout):
    """Drafts continue the prefix pages (draft_start = L_i) and each request
    accepts a root-to-leaf path of its draft tree that skips nodes, so the k-th
    destination L_i + k is the draft slot of an earlier accepted node: every
    copy must still move the value its source held before the commit."""
    wl = W.build_workload("treecommit", [37, 64, 5, 90], [[12], [20], [9], [16]], 8, 2, 128, 16,
                          seed=64, suffix_in_prefix_pages=True)
    wl = W.attach_random_trees(wl, seed=65, max_children=2)
    qo = wl.branch_qo_indptr
    acc, ind = [], [0]
    for i in range(wl.batch_size):
        r0, S = int(qo[i]), int(qo[i + 1] - qo[i])
        leaf = S - 1                        # deepest-numbered node; walk up to the root
        path = []
        u = leaf
        while u >= 0:
            path.append(u)
            u = int(wl.draft_parent[r0 + u])
        path = path[::-1]
        acc += [r0 + u for u in path]
        ind.append(len(acc))
    skipping = sum(1 for i in range(wl.batch_size)
                   for k, r in enumerate(acc[ind[i]:ind[i + 1]]) if r - int(qo[i]) != k)
    assert skipping > 0                     # some destination is an earlier node's draft slot
    x = B.to_device(wl, layout=layout)
    kc, vc, lens = O.commit_accepted(wl, np.array(ind), np.array(acc))
    note(f"commit tree path {layout}")
    B.cascade_commit_accepted(x, torch.tensor(ind, dtype=torch.int32, device="cuda"),
                              torch.tensor(acc, dtype=torch.int32, device="cuda"),
                              max(np.diff(ind)))
    torch.cuda.synchronize()
    assert np.array_equal(x.cache_seqlens.cpu().numpy(), lens)
    assert np.array_equal(pool_bits_nhd(x.k_pool, layout), W.bf16_bits(kc))
    assert np.array_equal(pool_bits_nhd(x.v_pool, layout), W.bf16_bits(vc))
    assert B.cascade_device_error(clear=True) == 0


def test_append_empty_commit_changes_nothing(B):
    wl = W.build_workload("step0", [33, 17], [[2, 2], [3]], 4, 2, 64, 16, seed=63)
    x = B.to_device(wl)
    before_k = x.k_pool.clone()
    lens = x.cache_seqlens.clone()
    note("empty commit")
    B.cascade_commit_accepted(x, torch.zeros(wl.batch_size + 1, dtype=torch.int32, device="cuda"),
                              torch.zeros(1, dtype=torch.int32, device="cuda"), 0)
    torch.cuda.synchronize()
    # bit patterns: unused slots hold NaN
    assert torch.equal(x.k_pool.view(torch.int16), before_k.view(torch.int16))
    assert torch.equal(x.cache_seqlens, lens)


def test_graph_captured_multi_layer_step(B):
    """Three layers of (append drafts, fused verify) in one captured graph."""
    wl = W.build_workload("graph", [300, 120, 0, 64], [[3] * 4, [5, 2], [4], [2, 2, 2]], 16, 4, 128, 16,
                          seed=62)
    n_layers = 3
    xs = [B.to_device(wl, layout="HND") for _ in range(n_layers)]
    wss = [B.workspace_for(x) for x in xs]
    drafts = [tuple(t.cuda() for t in random_drafts(wl, 100 + l)) for l in range(n_layers)]
    shape_o, shape_l = (wl.total_rows, wl.num_qo_heads, wl.head_dim), (wl.total_rows, wl.num_qo_heads)
    o_e = [torch.empty(shape_o, dtype=torch.bfloat16, device="cuda") for _ in range(n_layers)]
    l_e = [torch.empty(shape_l, dtype=torch.float32, device="cuda") for _ in range(n_layers)]
    o_g = [torch.empty_like(t) for t in o_e]
    l_g = [torch.empty_like(t) for t in l_e]

    def step(outs, lses):
        for l in range(n_layers):
            B.cascade_append_draft_kv(xs[l], drafts[l][0], drafts[l][1])
            B.cascade_verify_attn(xs[l], o=outs[l], lse=lses[l], workspace=wss[l])

    note("graph: eager warm-up")
    step(o_e, l_e)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    note("graph: capture")
    with torch.cuda.graph(g):
        step(o_g, l_g)
    torch.cuda.synchronize()
    for rep in range(3):
        note(f"graph: replay {rep}")
        gen = torch.Generator(device="cuda").manual_seed(200 + rep)
        for k, v in drafts:            # eager work between replays: new draft values
            k.copy_(torch.randn(k.shape, generator=gen, device="cuda").to(torch.bfloat16))
            v.copy_(torch.randn(v.shape, generator=gen, device="cuda").to(torch.bfloat16))
        g.replay()
        torch.cuda.synchronize()
        step(o_e, l_e)
        torch.cuda.synchronize()
        for l in range(n_layers):
            assert torch.equal(o_g[l], o_e[l]) and torch.equal(l_g[l], l_e[l])
    # the last eager step also matches the oracle for layer 0's inputs
    ko, vo = O.append_draft_kv(wl, drafts[0][0].float().cpu().numpy(), drafts[0][1].float().cpu().numpy())
    w0 = copy.copy(wl)
    w0.k_pool, w0.v_pool = ko, vo
    ro, rl = O.cascade(w0)
    o = o_e[0].float().cpu().numpy().astype(np.float64)
    assert np.max(np.abs(o - ro)) <= 1e-2


def _move_page_on_device(x, i, p, old, new_page):
    """Moves logical page p of request i from physical page `old` to
    `new_page` in place: the page's K/V are copied, then the block-table entry
    is rewritten (the device buffers keep their addresses)."""
    for pool in (x.k_pool, x.v_pool):
        pool[new_page].copy_(pool[old])
    x.page_table[i, p] = new_page


def test_graph_replay_after_in_place_table_updates(B):
    """One serving step -- draft-KV append, fused verify, commit of the accepted
    rows with in-place lengths -- captured once in a HIP graph and replayed
    while, between replays, block-table entries are rewritten in place (pages
    moved to fresh physical pages), the committed lengths grow on the device,
    and new draft values and acceptance lists are written into the captured
    buffers (the KV-cache tutorial's CUDA-Graph note: update the block-table
    contents, replay without re-capture).  Every replay must equal the same
    step run eagerly on a second copy of the state, bit for bit (outputs,
    pools, lengths), and the final step must match the oracle."""
    n_steps = 4
    base = W.build_workload("replay", [300, 120, 64], [[3, 3, 2], [4], [2, 5]], 8, 2, 128, 16, seed=66)
    w = with_room(base, 3 * n_steps + 4)
    # fresh pages at the end of the pool, targets of the in-place remaps
    extra = 2 * n_steps
    fresh = np.full((extra,) + w.k_pool.shape[1:], np.nan, np.float32)
    first_fresh = w.k_pool.shape[0]
    w.k_pool = np.concatenate([w.k_pool, fresh])
    w.v_pool = np.concatenate([w.v_pool, fresh.copy()])
    bound = int(w.cache_seqlens.max()) + 3 * n_steps
    xs = {}
    for name in ("graph", "eager"):
        x = B.to_device(w, layout="HND")
        x.tree.max_prefix_len = bound       # the lengths grow by up to 3 per step
        xs[name] = x
    ws = {k: B.workspace_for(x) for k, x in xs.items()}
    shape = (w.total_rows, w.num_kv_heads, w.head_dim)
    R, Hq, d = w.total_rows, w.num_qo_heads, w.head_dim
    bufs = {}
    for name in xs:
        bufs[name] = dict(k=torch.zeros(shape, dtype=torch.bfloat16, device="cuda"),
                          v=torch.zeros(shape, dtype=torch.bfloat16, device="cuda"),
                          ind=torch.zeros(w.batch_size + 1, dtype=torch.int32, device="cuda"),
                          rows=torch.zeros(3 * w.batch_size, dtype=torch.int32, device="cuda"),
                          o=torch.empty((R, Hq, d), dtype=torch.bfloat16, device="cuda"),
                          lse=torch.empty((R, Hq), dtype=torch.float32, device="cuda"))

    def step(name):
        x, b = xs[name], bufs[name]
        B.cascade_append_draft_kv(x, b["k"], b["v"])
        B.cascade_verify_attn(x, o=b["o"], lse=b["lse"], workspace=ws[name])
        B.cascade_commit_accepted(x, b["ind"], b["rows"], 3)

    # capture the step once (its inputs are the buffers above); capturing
    # runs nothing, so both copies still hold the same state
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    note("graph replay: capture")
    with torch.cuda.graph(g):
        step("graph")
    torch.cuda.synchronize()
    qo, rbi = w.branch_qo_indptr, w.req_branch_indptr
    rng = np.random.default_rng(67)
    for it in range(n_steps):
        # in place, on both copies: draft values, acceptance, a page move
        gen = torch.Generator().manual_seed(300 + it)
        kn = torch.randn(shape, generator=gen).to(torch.bfloat16)
        vn = torch.randn(shape, generator=gen).to(torch.bfloat16)
        acc, ind = [], [0]
        for i in range(w.batch_size):
            j = int(rbi[i] + rng.integers(int(rbi[i + 1] - rbi[i])))
            n = int(rng.integers(0, min(3, int(qo[j + 1] - qo[j])) + 1))
            acc += list(range(int(qo[j]), int(qo[j]) + n))
            ind.append(len(acc))
        i_move = it % w.batch_size
        p_move = int(rng.integers(max(1, -(-int(w.cache_seqlens[i_move]) // w.page_size))))
        for name in xs:
            b = bufs[name]
            b["k"].copy_(kn)
            b["v"].copy_(vn)
            b["ind"].copy_(torch.tensor(ind, dtype=torch.int32))
            b["rows"].zero_()
            if acc:
                b["rows"][:len(acc)].copy_(torch.tensor(acc, dtype=torch.int32))
        old, new_page = int(w.page_table[i_move, p_move]), first_fresh + it
        for x in xs.values():
            _move_page_on_device(x, i_move, p_move, old, new_page)
        w.k_pool[new_page] = w.k_pool[old]
        w.v_pool[new_page] = w.v_pool[old]
        w.page_table[i_move, p_move] = new_page
        torch.cuda.synchronize()
        note(f"graph replay {it}: move request {i_move} page {p_move}, accept {len(acc)} rows")
        g.replay()
        torch.cuda.synchronize()
        step("eager")
        torch.cuda.synchronize()
        xg, xe, bg, be = xs["graph"], xs["eager"], bufs["graph"], bufs["eager"]
        assert torch.equal(bg["o"], be["o"]) and torch.equal(bg["lse"], be["lse"])
        assert torch.equal(xg.cache_seqlens, xe.cache_seqlens)
        assert torch.equal(xg.k_pool.view(torch.int16), xe.k_pool.view(torch.int16))
        assert torch.equal(xg.v_pool.view(torch.int16), xe.v_pool.view(torch.int16))
        # the oracle follows the same step on the host copy
        ko, vo = O.append_draft_kv(w, kn.float().numpy(), vn.float().numpy())
        w.k_pool, w.v_pool = ko, vo
        ro, rl = O.cascade(w)
        o = be["o"].float().cpu().numpy().astype(np.float64)
        l = be["lse"].cpu().numpy().astype(np.float64)
        assert np.max(np.abs(o - ro)) <= 1e-2
        fin = np.isfinite(rl)
        assert np.max(np.abs(l[fin] - rl[fin])) <= 1e-3
        kc, vc, lens = O.commit_accepted(w, np.array(ind), np.array(acc, dtype=np.int64))
        w.k_pool, w.v_pool, w.cache_seqlens = kc, vc, lens
        assert np.array_equal(xe.cache_seqlens.cpu().numpy(), lens)
        assert np.array_equal(pool_bits_nhd(xe.k_pool, "HND"), W.bf16_bits(kc))
    assert B.cascade_device_error(clear=True) == 0


def test_stream_read_reference(B):
    buf = torch.arange(1 << 20, dtype=torch.int32, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    note("stream read")
    B.cascade_stream_read(buf, sink)
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0
