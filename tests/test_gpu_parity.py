"""GPU parity: every entry point of the C ABI against the fp64 oracle.

Bounds (bf16 inputs, fp32 accumulation): max |o - o_ref| <= 1e-2 and
max |LSE - LSE_ref| <= 1e-3 where LSE_ref is finite; LSE_ref = -inf must be
-inf exactly.  Gather and mask hooks are compared bit for bit.
"""

import dataclasses
import math
import sys

import numpy as np
import pytest
import torch

from cascade_attention_tree_amd import workload as W
from oracle import cascade_oracle as O

pytestmark = pytest.mark.gpu

O_TOL = 1e-2
LSE_TOL = 1e-3


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from cascade_attention_tree_amd import binding
    binding.lib()
    return binding


def note(msg):
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


def cmp(o_gpu, lse_gpu, o_ref, lse_ref, rows=None, o_tol=O_TOL, lse_tol=LSE_TOL):
    o = o_gpu.float().cpu().numpy().astype(np.float64)
    l = lse_gpu.float().cpu().numpy().astype(np.float64)
    if rows is not None:
        o, l = o[rows], l[rows]
    assert np.all(np.isfinite(o)), "non-finite output"
    ninf = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(l), ninf), "LSE = -inf pattern differs"
    err_o = float(np.max(np.abs(o - o_ref))) if o.size else 0.0
    fin = ~ninf
    err_l = float(np.max(np.abs(l[fin] - lse_ref[fin]))) if fin.any() else 0.0
    assert err_o <= o_tol, f"max |o - ref| = {err_o}"
    assert err_l <= lse_tol, f"max |lse - ref| = {err_l}"
    return err_o, err_l


# 28 requests of 5 query tokens (one to three branches), prefixes 0 to 1300.
PAIR16_LENS = [1300, 77, 0, 512, 33, 900, 260, 1, 640, 100, 1024, 7, 450, 300,
               64, 1111, 16, 800, 5, 230, 999, 48, 700, 129, 31, 600, 2, 1200]
PAIR16_BRANCHES = [[5], [4, 1], [2, 3], [1, 2, 2]] * 7


def small_cases():
    """Shapes chosen to span several tiles, ragged tails, splits and chunks."""
    return {
        "tiny": lambda: W.tiny(values="bf16"),
        "gqa_ragged": lambda: W.build_workload("gqa_ragged", [75, 0, 300, 33], [[2, 4, 1], [3], [1, 5, 2, 2], [6]],
                                               8, 2, 128, 16, seed=21),
        "page64_d64": lambda: W.build_workload("page64_d64", [700, 129, 1], [[3, 3], [7], [1, 1, 1]],
                                               4, 4, 64, 64, seed=22),
        "rows_chunked": lambda: W.build_workload("rows_chunked", [400, 1200], [[8] * 8, [5] * 3],
                                                 16, 2, 128, 16, seed=23),
        "long_split": lambda: W.build_workload("long_split", [5000, 2500], [[4, 4], [2]], 8, 8, 128, 32,
                                               seed=24),
        "topk1": lambda: W.build_workload("topk1", [90, 17], [[6], [9]], 4, 2, 128, 16, seed=25),
        # Few (request, kv head) pairs with few rows: 16-row chunks of the
        # key-split kernel, the longest prefix split in three.
        "thin_split": lambda: W.build_workload("thin_split", [2500, 300, 0], [[3, 2], [5], [1, 1, 1]],
                                               8, 2, 128, 16, seed=51),
        # 80 rows per (request, kv head) over 56 pairs, too few to fill the
        # device: five 16-row chunks each on the pair kernel's one-block
        # instance.
        "pair_16row": lambda: W.build_workload("pair_16row", PAIR16_LENS, PAIR16_BRANCHES, 32, 2, 128, 16,
                                               seed=52),
        # 96 rows per (request, kv head) over 4 pairs: one row-split item each
        # (three of its four waves hold rows), a 1300-key prefix split.
        "rows_small": lambda: W.build_workload("rows_small", [1300, 77], [[4, 4, 4], [6, 6]], 16, 2, 128, 16,
                                               seed=69),
        # More branches per request than one wave has lanes (70), and more than
        # the per-workgroup branch window holds (130): the tree tables' slow paths.
        "wide_tree": lambda: W.build_workload("wide_tree", [300, 50], [[1] * 70, [2] * 130], 4, 2, 64, 16,
                                              seed=26),
        # General draft trees (ancestor masks): one tree per request, incl. an
        # empty prefix; 64- and 33-node trees over several row chunks at d = 64.
        "draft_tree": lambda: W.attach_random_trees(
            W.build_workload("draft_tree", [75, 0, 300], [[12], [7], [20]], 8, 2, 128, 16, seed=27), 28),
        "draft_tree_big": lambda: W.attach_random_trees(
            W.build_workload("draft_tree_big", [200, 40], [[64], [33]], 16, 2, 64, 16, seed=29), 30),
        # Trees of more than 64 nodes (3-word ancestor masks): 150- and
        # 70-node trees on the row-split kernel (600 rows per kv head) and in pass B
        # and naive expansion on the key-split kernel; at d = 64 on the
        # key-split kernel throughout.
        "wide_tree_masks": lambda: W.attach_random_trees(
            W.build_workload("wide_tree_masks", [300, 0], [[150], [70]], 8, 2, 128, 16, seed=63), 64),
        "wide_tree_masks_d64": lambda: W.attach_random_trees(
            W.build_workload("wide_tree_masks_d64", [130, 77], [[100], [129]], 4, 2, 64, 16, seed=65), 66),
        # At least 1024 query rows per (request, kv head) at d = 128: pass A
        # and the fused verify pass run the row-split kernel.  Chains whose
        # 40-token branches span several draft tiles of a 128-row chunk, an
        # empty prefix, a one-token request among large ones; a 64-node tree
        # with 16 query heads per kv head; a long prefix split over workgroups
        # (partials merged by the split-merge pass).
        "rows_chains": lambda: W.build_workload("rows_chains", [700, 0, 45], [[40] * 4, [30] * 5, [1]],
                                                16, 2, 128, 16, seed=31),
        "rows_tree": lambda: W.attach_random_trees(
            W.build_workload("rows_tree", [300, 90], [[64], [50]], 32, 2, 128, 16, seed=32), 33),
        "rows_split": lambda: W.build_workload("rows_split", [9000], [[64, 64]], 16, 2, 128, 16, seed=34),
        # The row-split kernel over 64-token pages: several branches per
        # request; one long branch whose tokens continue its prefix pages from
        # slot 600 (not a multiple of 32), read like a prefix in pass B.
        "rows_page64": lambda: W.build_workload("rows_page64", [1500, 333], [[48, 48, 48], [20] * 5],
                                                16, 2, 128, 64, seed=35),
        "rows_suffix_p64": lambda: W.build_workload("rows_suffix_p64", [600], [[200]], 16, 2, 128, 64,
                                                    seed=36, suffix_in_prefix_pages=True),
        # One branch per request behind a long, key-split prefix: split 0 of
        # the fused verify launch streams the branch after its prefix keys
        # while the other splits hold prefix keys only; a chain and a tree.
        "rows_split_slot": lambda: W.build_workload("rows_split_slot", [9000], [[130]], 16, 2, 128, 16,
                                                    seed=37),
        "rows_split_slot_tree": lambda: W.attach_random_trees(
            W.build_workload("rows_split_slot_tree", [5000, 2100], [[64], [40]], 32, 2, 128, 16, seed=38), 39),
        # A 300-node tree streamed through the row-split kernel's ring loop
        # (1200 rows per kv head; 5-word masks), with a split prefix.
        "rows_wide_tree": lambda: W.attach_random_trees(
            W.build_workload("rows_wide_tree", [4500], [[300]], 8, 2, 128, 16, seed=67), 68),
        # Row-split launches whose chunks see more draft keys than the LDS
        # table of draft-key offsets holds (256 at three workgroups per CU,
        # 512 at two): two branches per request, so no chunk streams its
        # drafts; the keys past the table resolve through the block table.
        "rows_long_branch": lambda: W.build_workload("rows_long_branch", [700], [[300, 10]], 16, 2, 128, 16,
                                                     seed=72),
        "rows_long_branch_g1": lambda: W.build_workload("rows_long_branch_g1", [300], [[600, 10]], 2, 2, 128, 16,
                                                        seed=73),
        # A 600-token suffix (one branch continuing its prefix pages) at d = 64,
        # which the key-split kernel runs: row chunks near the end of the
        # suffix see more than 512 draft keys, past the LDS table of draft-key
        # offsets, so those keys resolve through the block table one by one.
        "suffix600_d64": lambda: W.build_workload("suffix600_d64", [100, 37], [[600], [530]], 8, 2, 64, 16,
                                                  seed=40, suffix_in_prefix_pages=True),
        # The same past-the-table draft keys in draft pages of their own, a
        # short branch in front of a 560-token one.
        "long_branch_d64": lambda: W.build_workload("long_branch_d64", [64], [[40, 560]], 4, 2, 64, 16,
                                                    seed=42),
    }


CASES = sorted(small_cases())


@pytest.mark.parametrize("case", CASES)
def test_prefix_pass(B, case):
    wl = small_cases()[case]()
    note(f"prefix_attn {case} rows={wl.total_rows}")
    x = B.to_device(wl)
    o, l = B.cascade_prefix_attn(x)
    torch.cuda.synchronize()
    ro, rl = O.prefix_pass(wl)
    cmp(o, l, ro, rl)


@pytest.mark.parametrize("case", CASES)
def test_draft_pass(B, case):
    wl = small_cases()[case]()
    note(f"draft_attn {case}")
    x = B.to_device(wl)
    o, l = B.cascade_draft_attn(x)
    torch.cuda.synchronize()
    ro, rl = O.draft_pass(wl)
    cmp(o, l, ro, rl)


@pytest.mark.parametrize("layout", ["NHD", "HND"])
@pytest.mark.parametrize("case", CASES)
def test_verify_and_three_call_path(B, case, layout):
    wl = small_cases()[case]()
    note(f"verify {case} {layout}")
    x = B.to_device(wl, layout=layout)
    ro, rl = O.cascade(wl)
    o, l = B.cascade_verify_attn(x)
    oa, la = B.cascade_prefix_attn(x)
    ob, lb = B.cascade_draft_attn(x)
    o3, l3 = B.merge_state(oa, la, ob, lb)
    torch.cuda.synchronize()
    cmp(o, l, ro, rl)
    cmp(o3, l3, ro, rl)


@pytest.mark.parametrize("layout", ["NHD", "HND"])
def test_rows_kernel_fixed_order(B, layout):
    """The row-split kernel without room for its work list (no workspace, an
    unsplit prefix): its items in the fixed grid order give results equal,
    bit for bit, to the work-list order, and match the oracle."""
    wl = W.build_workload("rows_short", [500, 0, 300, 45], [[40] * 4, [30] * 5, [12, 9], [1]], 16, 2, 128, 16,
                          seed=70)
    note(f"rows fixed order {layout}")
    x = B.to_device(wl, layout=layout)
    ws = B.workspace_for(x)
    assert ws is not None and ws.numel() > 0, "the row-split launch has a work list"
    none = torch.empty(0, dtype=torch.uint8, device="cuda")
    o1, l1 = B.cascade_verify_attn(x, workspace=ws)
    o0, l0 = B.cascade_verify_attn(x, workspace=none)
    a1, la1 = B.cascade_prefix_attn(x, workspace=ws)
    a0, la0 = B.cascade_prefix_attn(x, workspace=none)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    assert torch.equal(a0, a1) and torch.equal(la0, la1)
    ro, rl = O.cascade(wl)
    cmp(o0, l0, ro, rl)
    ra, rla = O.prefix_pass(wl)
    cmp(a0, la0, ra, rla)


@pytest.mark.parametrize("layout", ["NHD", "HND"])
@pytest.mark.parametrize("case", CASES)
def test_naive_expand(B, case, layout):
    wl = small_cases()[case]()
    note(f"naive_expand {case} {layout}")
    x = B.to_device(wl, layout=layout)
    o, l = B.naive_expand(x)
    torch.cuda.synchronize()
    ro, rl = O.naive_expand(wl)
    cmp(o, l, ro, rl)


def test_merge_state_kernel(B):
    note("merge_state")
    rng = np.random.default_rng(31)
    R, H, d = 37, 6, 128
    oa = rng.standard_normal((R, H, d)).astype(np.float32)
    ob = rng.standard_normal((R, H, d)).astype(np.float32)
    la = (rng.standard_normal((R, H)) * 5).astype(np.float32)
    lb = (rng.standard_normal((R, H)) * 5).astype(np.float32)
    la[0, :] = -np.inf
    lb[1, :] = -np.inf
    la[2, :] = -np.inf
    lb[2, :] = -np.inf
    la[3, :] = lb[3, :] = 80.0   # large equal LSEs: + ln 2, mean of outputs
    ro, rl = O.merge_state(oa, la, ob, lb)
    t = lambda a: torch.from_numpy(a).cuda()
    o, l = B.merge_state(t(oa), t(la), t(ob), t(lb))
    ob16, _ = B.merge_state(t(oa), t(la), t(ob), t(lb), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    cmp(o, l, ro, rl, o_tol=1e-5, lse_tol=2e-5)
    assert np.allclose(l.cpu().numpy()[3], 80.0 + math.log(2.0), atol=1e-5)
    ref16 = torch.from_numpy(ro.astype(np.float32)).to(torch.bfloat16).float().numpy()
    assert np.max(np.abs(ob16.float().cpu().numpy() - ref16)) <= 2 ** -7


@pytest.mark.parametrize("layout", ["NHD", "HND"])
def test_verify_headline_all_rows(B, layout):
    """The headline launch the benchmark times (bf16 output), naive expansion,
    and the three-call form (pass A, pass B, merge_state), all rows."""
    wl = W.headline()
    note(f"verify headline rows={wl.total_rows} {layout}")
    x = B.to_device(wl, layout=layout)
    o, l = B.cascade_verify_attn(x, out_dtype=torch.bfloat16)
    on, ln = B.naive_expand(x)
    oa, la = B.cascade_prefix_attn(x, workspace=B.workspace_for(x))
    ob, lb = B.cascade_draft_attn(x)
    o3, l3 = B.merge_state(oa, la, ob, lb, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ro, rl = O.cascade(wl)
    cmp(o, l, ro, rl)
    cmp(on, ln, ro, rl)
    cmp(o3, l3, ro, rl)


def test_verify_gqa_config(B):
    """The GQA verify configuration (B=8, Hq=32, Hkv=8, d=128, L=1000, topk=4,
    S=3), all rows: fused verify and pass A."""
    wl = W.gqa()
    x = B.to_device(wl)
    note("verify gqa")
    o, l = B.cascade_verify_attn(x)
    oa, la = B.cascade_prefix_attn(x)
    torch.cuda.synchronize()
    ro, rl = O.cascade(wl)
    cmp(o, l, ro, rl)
    rao, ral = O.prefix_pass(wl)
    cmp(oa, la, rao, ral)


def test_verify_ragged_sampled(B):
    wl = W.ragged()
    rb, qo = wl.req_branch_indptr, wl.branch_qo_indptr
    # 8 whole requests: the longest and shortest prefixes, the largest and
    # smallest row counts, and four more spread over the batch.
    L = wl.cache_seqlens
    rows_per = np.array([qo[rb[i + 1]] - qo[rb[i]] for i in range(wl.batch_size)])
    pick = {int(np.argmax(L)), int(np.argmin(L)), int(np.argmax(rows_per)), int(np.argmin(rows_per))}
    for i in np.linspace(0, wl.batch_size - 1, 8).astype(int):
        if len(pick) >= 8:
            break
        pick.add(int(i))
    rows = np.concatenate([np.arange(qo[rb[i]], qo[rb[i + 1]]) for i in sorted(pick)])
    note(f"verify ragged: {len(pick)} requests, {rows.size} sampled rows")
    x = B.to_device(wl)
    o, l = B.cascade_verify_attn(x)
    torch.cuda.synchronize()
    r, ro, rl = O.cascade_rows(wl, rows)
    cmp(o, l, ro, rl, rows=r)


@pytest.mark.parametrize("h", [0.0, 0.5, 0.9])
def test_prefix_hit_small_all_rows(B, h):
    wl = W.prefix_hit(h, batch=2, n_tokens=300, seed=41)
    note(f"prefix-hit small h={h}")
    x = B.to_device(wl)
    ro, rl = O.naive_expand(wl)
    o, l = B.cascade_verify_attn(x)
    oa, la = B.cascade_prefix_attn(x)
    ob, lb = B.cascade_draft_attn(x)
    o3, l3 = B.merge_state(oa, la, ob, lb)
    torch.cuda.synchronize()
    cmp(o, l, ro, rl)
    cmp(o3, l3, ro, rl)


@pytest.mark.parametrize("n_tokens", [300, 600])
@pytest.mark.parametrize("h", [0.5, 0.9])
def test_draft_pass_ignores_slots_in_front_of_the_branch(B, h, n_tokens):
    """The prefix slots just in front of a prefix-hit suffix are set to NaN:
    pass B must not let them into its result.  At 600 tokens (1200 query rows
    per kv head) pass B streams the suffix like a prefix from tiles that start
    at a multiple of 32 slots, so its first tile covers those slots (H is not
    such a multiple here)."""
    wl = W.prefix_hit(h, batch=2, n_tokens=n_tokens, seed=43)
    P = wl.page_size
    k, v = wl.k_pool.copy(), wl.v_pool.copy()
    for j in range(wl.num_branches):
        hs = int(wl.draft_start[j])
        assert hs % 32 != 0
        for t in range(hs - hs % 32, hs):
            pg = wl.draft_page_table[j][t // P]
            k[pg, t % P] = np.nan
            v[pg, t % P] = np.nan
    wl = dataclasses.replace(wl, k_pool=k, v_pool=v)
    note(f"draft_attn prefix-hit h={h} N={n_tokens}, NaN in front of the suffix")
    x = B.to_device(wl)
    o, l = B.cascade_draft_attn(x)
    torch.cuda.synchronize()
    ro, rl = O.draft_pass(wl)
    cmp(o, l, ro, rl)


@pytest.mark.parametrize("h", [0.0, 0.5, 0.9])
def test_prefix_hit_full_sampled(B, h):
    wl = W.prefix_hit(h)
    M = wl.total_rows // wl.batch_size
    rng = np.random.default_rng(5)
    rows = []
    for i in range(wl.batch_size):
        base = i * M
        rows += [base, base + M - 1] + list(base + rng.choice(M, 126, replace=False))
    rows = np.unique(np.array(rows))
    note(f"prefix-hit full h={h} sampled rows={rows.size}")
    x = B.to_device(wl)
    oa, la = B.cascade_prefix_attn(x)
    ob, lb = B.cascade_draft_attn(x)
    o, l = B.merge_state(oa, la, ob, lb)
    of, lf = B.cascade_verify_attn(x)  # the same split and merge in one launch
    torch.cuda.synchronize()
    r, ro, rl = O.cascade_rows(wl, rows)
    cmp(o, l, ro, rl, rows=r)
    cmp(of, lf, ro, rl, rows=r)


def _gather_ref_bits(wl, pool_name, table_row, first_slot, count, g):
    """CPU gather of `count` logical slots from `first_slot` of one block-table
    row (kv head g), as bf16 bits: bf16 pools directly, FP8 pools as the value
    of each E4M3 code (exact in bf16; scales not applied)."""
    t = first_slot + np.arange(count)
    P = wl.page_size
    if getattr(wl, "k_codes", None) is not None:
        codes = (wl.k_codes if pool_name == "k" else wl.v_codes)[table_row[t // P], t % P, g]
        return W.bf16_bits(O.e4m3_value(codes).astype(np.float32))
    pool = wl.k_pool if pool_name == "k" else wl.v_pool
    return W.bf16_bits(pool[table_row[t // P], t % P, g])


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("page", [16, 64])
@pytest.mark.parametrize("layout", ["NHD", "HND"])
def test_gather_hook_bit_exact(B, layout, page, kv):
    """The gather hook runs the attention kernels' own gather functions (page
    id of each 16-key half, its buffer descriptor, the lane offset; the
    draft-slot resolution and the clamped draft-key load) and must reproduce
    the CPU gather through the block tables bit for bit, for prefixes (tails
    that end inside a half and inside a page, an empty one) and for draft
    branches, one of which continues its request's prefix pages."""
    wls = [W.build_workload("gather", [75, 0, 300, 31], [[2, 4, 1], [3], [1, 5], [9]], 8, 2, 128, page,
                            seed=51),
           # one branch per request continuing its prefix pages from slot L_i
           # (31: inside a 16-key half; 100: inside a page)
           W.build_workload("gather_suffix", [31, 100, 0], [[9], [40], [3]], 8, 2, 128, page, seed=54,
                            suffix_in_prefix_pages=True)]
    for wl in wls:
        if kv == "fp8":
            wl = W.with_fp8_kv(wl)
        _check_gather(B, wl, layout, f"{wl.name} {layout} page {page}")


def _check_gather(B, wl, layout, label):
    x = B.to_device(wl, layout=layout)
    note(f"debug gather {label}")
    for i in range(wl.batch_size):
        L = int(wl.cache_seqlens[i])
        for g in range(wl.num_kv_heads):
            k, v = B.cascade_debug_gather(x, 0, i, g, L)
            assert np.array_equal(_bits(k), _gather_ref_bits(wl, "k", wl.page_table[i], 0, L, g))
            assert np.array_equal(_bits(v), _gather_ref_bits(wl, "v", wl.page_table[i], 0, L, g))
    for j in range(wl.num_branches):
        S = int(wl.branch_qo_indptr[j + 1] - wl.branch_qo_indptr[j])
        for g in range(wl.num_kv_heads):
            k, v = B.cascade_debug_gather(x, 1, j, g, S)
            ds = int(wl.draft_start[j])
            assert np.array_equal(_bits(k), _gather_ref_bits(wl, "k", wl.draft_page_table[j], ds, S, g))
            assert np.array_equal(_bits(v), _gather_ref_bits(wl, "v", wl.draft_page_table[j], ds, S, g))
    assert B.cascade_device_error(clear=True) == 0


@pytest.mark.parametrize("tree", ["chains", "tree", "wide_tree"])
def test_mask_hook_bit_exact(B, tree):
    wl = W.build_workload("gm", [75, 0, 300], [[2, 4, 1], [3], [1, 5]], 8, 2, 128, 16, seed=51)
    if tree == "tree":
        wl = W.build_workload("gm_tree", [75, 0, 300], [[13], [3], [40]], 8, 2, 128, 16, seed=52)
        W.attach_random_trees(wl, 53)
    elif tree == "wide_tree":   # 2- and 3-word ancestor masks
        wl = W.build_workload("gm_wide_tree", [75, 0, 30], [[130], [3], [90]], 8, 2, 128, 16, seed=54)
        W.attach_random_trees(wl, 55)
    x = B.to_device(wl)
    note("debug mask")
    for j in range(wl.num_branches):
        S = int(wl.branch_qo_indptr[j + 1] - wl.branch_qo_indptr[j])
        i = int(np.searchsorted(wl.req_branch_indptr, j, side="right") - 1)
        L = int(wl.cache_seqlens[i])
        m = B.cascade_debug_mask(x, j, S, L + S + 3).cpu().numpy().astype(bool)
        ref_m = np.zeros((S, L + S + 3), bool)
        ref_m[:, :L + S] = O.visibility_mask(wl, j)
        assert np.array_equal(m, ref_m)


def test_page_permutation_bit_identical(B):
    wl = W.build_workload("perm", [300, 77], [[3, 5], [4]], 8, 4, 128, 16, seed=61)
    x1 = B.to_device(wl)
    o1, l1 = B.cascade_verify_attn(x1)
    n1, nl1 = B.naive_expand(x1)
    perm = np.random.default_rng(7).permutation(wl.k_pool.shape[0]).astype(np.int32)
    wl2 = W.build_workload("perm", [300, 77], [[3, 5], [4]], 8, 4, 128, 16, seed=61)
    k2 = np.empty_like(wl.k_pool)
    v2 = np.empty_like(wl.v_pool)
    k2[perm] = wl.k_pool
    v2[perm] = wl.v_pool
    wl2.k_pool, wl2.v_pool = k2, v2
    wl2.page_table = perm[wl.page_table]
    wl2.draft_page_table = perm[wl.draft_page_table]
    note("page permutation")
    x2 = B.to_device(wl2)
    o2, l2 = B.cascade_verify_attn(x2)
    n2, nl2 = B.naive_expand(x2)
    o3, l3 = B.cascade_verify_attn(x1)   # same inputs again: deterministic
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(n1, n2) and torch.equal(nl1, nl2)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)


def test_shared_prefix_pages(B):
    """Two requests whose block tables share their first two pages (aliasing)."""
    wl = W.build_workload("alias", [64, 48], [[2, 2], [3]], 4, 2, 128, 16, seed=71)
    wl.page_table[1, :2] = wl.page_table[0, :2]
    note("shared prefix pages")
    x = B.to_device(wl)
    o, l = B.cascade_verify_attn(x)
    torch.cuda.synchronize()
    ro, rl = O.cascade(wl)
    cmp(o, l, ro, rl)


def test_bf16_output(B):
    wl = W.build_workload("bf16out", [500, 64], [[4, 4], [2]], 8, 2, 128, 16, seed=81)
    x = B.to_device(wl)
    note("bf16 output")
    o32, l32 = B.cascade_verify_attn(x)
    o16, l16 = B.cascade_verify_attn(x, out_dtype=torch.bfloat16)
    n16, _ = B.naive_expand(x, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(l32, l16)
    assert torch.equal(o32.to(torch.bfloat16), o16)
    ro, rl = O.cascade(wl)
    cmp(o16, l16, ro, rl)
    cmp(n16, l16, ro, rl)


@pytest.mark.parametrize("case", ["tiny", "long_split"])
def test_kernel_timing_events(B, case):
    """Timed launches (events around the kernels, split and unsplit plans)
    give the same bits as plain launches and a positive kernel time."""
    wl = small_cases()[case]()
    x = B.to_device(wl, layout="HND")
    ws = B.workspace_for(x)
    note(f"kernel timing {case}")
    o0, l0 = B.cascade_verify_attn(x, workspace=ws)
    B.cascade_kernel_timing(True)
    try:
        o1, l1 = B.cascade_verify_attn(x, workspace=ws)
        ms = B.cascade_last_verify_ms()
    finally:
        B.cascade_kernel_timing(False)
    torch.cuda.synchronize()
    assert 0.0 < ms < 1000.0
    assert torch.equal(o0, o1) and torch.equal(l0, l1)


def test_no_device_error_raised(B):
    note("device error word")
    assert B.cascade_device_error(clear=True) == 0
