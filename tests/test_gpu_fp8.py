"""GPU parity of the FP8 KV read path (KV-cache tutorial page, section 4.5:
FP8 KV with a per-tensor scale) against the fp64 oracle.

The pools hold E4M3 codes; the oracle attends over value(code) * scale.  The
kernels widen the codes to bf16 exactly and apply the scales in fp32, so the
bounds are those of the bf16 path: max |o - o_ref| <= 1e-2, max |LSE -
LSE_ref| <= 1e-3 (LSE_ref = -inf exactly).  The widening itself, and the
append / commit copies of codes, are compared bit for bit.
"""

import copy
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


def cmp(o_gpu, lse_gpu, o_ref, lse_ref):
    o = o_gpu.float().cpu().numpy().astype(np.float64)
    l = lse_gpu.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(o)), "non-finite output"
    ninf = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(l), ninf), "LSE = -inf pattern differs"
    err_o = float(np.max(np.abs(o - o_ref))) if o.size else 0.0
    fin = ~ninf
    err_l = float(np.max(np.abs(l[fin] - lse_ref[fin]))) if fin.any() else 0.0
    assert err_o <= O_TOL, f"max |o - ref| = {err_o}"
    assert err_l <= LSE_TOL, f"max |lse - ref| = {err_l}"


# 28 requests of 5 query tokens, 80 rows per (request, kv head) over 56
# pairs: the pair kernel's one-block instance (16-row chunks).
PAIR16_LENS = [1300, 77, 0, 512, 33, 900, 260, 1, 640, 100, 1024, 7, 450, 300,
               64, 1111, 16, 800, 5, 230, 999, 48, 700, 129, 31, 600, 2, 1200]
PAIR16_BRANCHES = [[5], [4, 1], [2, 3], [1, 2, 2]] * 7


def cases():
    """Several tiles and ragged tails, both head dims, page sizes 16/32/64, a
    split prefix, more branches than a wave has lanes, and draft trees."""
    return {
        "gqa_ragged": lambda: W.build_workload("gqa_ragged", [75, 0, 300, 33], [[2, 4, 1], [3], [1, 5, 2, 2], [6]],
                                               8, 2, 128, 16, seed=41),
        "page64_d64": lambda: W.build_workload("page64_d64", [700, 129, 1], [[3, 3], [7], [1, 1, 1]],
                                               4, 4, 64, 64, seed=42),
        "rows_chunked": lambda: W.build_workload("rows_chunked", [400, 1200], [[8] * 8, [5] * 3],
                                                 16, 2, 128, 16, seed=43),
        "long_split": lambda: W.build_workload("long_split", [5000, 2500], [[4, 4], [2]], 8, 8, 128, 32,
                                               seed=44),
        "wide_tree": lambda: W.build_workload("wide_tree", [300, 50], [[1] * 70, [2] * 130], 4, 2, 64, 16,
                                              seed=45),
        "draft_tree": lambda: W.attach_random_trees(
            W.build_workload("draft_tree", [75, 0, 300], [[12], [7], [20]], 8, 2, 128, 16, seed=46), 47),
        # A 600-token suffix continuing its prefix pages (one branch): the row
        # chunks near its end see more than 512 draft keys, past the kernel's
        # LDS table of draft-key offsets, so those keys resolve through the
        # block table one by one.
        "suffix600": lambda: W.build_workload("suffix600", [100, 37], [[600], [530]], 8, 2, 128, 16, seed=49,
                                              suffix_in_prefix_pages=True),
        # Few pairs: 16-row chunks of the key-split kernel with a split
        # prefix, and the pair kernel's one-block instance.
        "thin_split": lambda: W.build_workload("thin_split", [2500, 300, 0], [[3, 2], [5], [1, 1, 1]],
                                               8, 2, 128, 16, seed=53),
        "pair_16row": lambda: W.build_workload("pair_16row", PAIR16_LENS, PAIR16_BRANCHES, 32, 2, 128, 16,
                                               seed=54),
        # 96 rows per (request, kv head): one row-split item each.
        "rows_small": lambda: W.build_workload("rows_small", [1300, 77], [[4, 4, 4], [6, 6]], 16, 2, 128, 16,
                                               seed=71),
        # At least 1024 query rows per (request, kv head): the row-split
        # kernel over FP8 pools -- chains over several draft tiles, a split
        # prefix, a suffix streamed from its prefix pages (64-token pages),
        # and draft trees.
        "rows_chains": lambda: W.build_workload("rows_chains", [700, 0, 45], [[40] * 4, [30] * 5, [1]],
                                                16, 2, 128, 16, seed=55),
        "rows_split": lambda: W.build_workload("rows_split", [9000], [[64, 64]], 16, 2, 128, 16, seed=56),
        "rows_suffix_p64": lambda: W.build_workload("rows_suffix_p64", [600], [[200]], 16, 2, 128, 64,
                                                    seed=57, suffix_in_prefix_pages=True),
        "rows_tree": lambda: W.attach_random_trees(
            W.build_workload("rows_tree", [300, 90], [[64], [50]], 32, 2, 128, 16, seed=58), 59),
    }


CASES = sorted(cases())


def fp8_case(name):
    return W.with_fp8_kv(cases()[name]())


@pytest.mark.parametrize("layout", ["NHD", "HND"])
@pytest.mark.parametrize("case", CASES)
def test_fp8_verify_and_three_call_path(B, case, layout):
    wl = fp8_case(case)
    note(f"fp8 verify {case} {layout}")
    x = B.to_device(wl, layout=layout)
    ref = O.dequantize_kv(wl)
    ro, rl = O.cascade(ref)
    o, l = B.cascade_verify_attn(x)
    oa, la = B.cascade_prefix_attn(x)
    ob, lb = B.cascade_draft_attn(x)
    o3, l3 = B.merge_state(oa, la, ob, lb)
    torch.cuda.synchronize()
    cmp(o, l, ro, rl)
    cmp(o3, l3, ro, rl)
    ra, rla = O.prefix_pass(ref)
    cmp(oa, la, ra, rla)
    assert B.cascade_device_error(clear=True) == 0


@pytest.mark.parametrize("layout", ["NHD", "HND"])
def test_fp8_headline_all_rows(B, layout):
    """The headline shapes (B=32, Hq=32, Hkv=8, d=128, L=2000, topk=4 chains of
    S=5, page 16) over FP8 E4M3 KV: the fused verify launch the benchmark
    times, all 640 x 32 rows, and naive expansion, against the oracle over the
    dequantised pools."""
    wl = W.with_fp8_kv(W.headline())
    note(f"fp8 headline all rows {layout}")
    x = B.to_device(wl, layout=layout)
    o, l = B.cascade_verify_attn(x, out_dtype=torch.bfloat16)
    on, ln = B.naive_expand(x)
    torch.cuda.synchronize()
    ro, rl = O.cascade(O.dequantize_kv(wl))
    cmp(o, l, ro, rl)
    cmp(on, ln, ro, rl)
    assert B.cascade_device_error(clear=True) == 0


@pytest.mark.parametrize("values", ["bf16", "fp8"])
def test_full_pairs_split_prefix_sampled(B, values):
    """32 requests x 8 kv heads (one key-split workgroup per pair holds all 80
    rows) with 4500-key prefixes, past the 4096 keys one split may hold: the
    fused verify launch splits every prefix in two and merges the partial
    states.  The first, the last and four random rows of every request
    against the oracle (over the dequantised pools for FP8)."""
    wl = W.build_workload("split_full_pairs", [4500] * 32, [[5] * 4] * 32, 32, 8, 128, 16, seed=81)
    if values == "fp8":
        wl = W.with_fp8_kv(wl)
    note(f"full pairs, split prefix, {values}")
    x = B.to_device(wl, layout="HND")
    assert B.workspace_for(x) is not None
    o, l = B.cascade_verify_attn(x, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    per = wl.total_rows // wl.batch_size
    rows = []
    for i in range(wl.batch_size):
        rows += [i * per, i * per + per - 1] + list(i * per + rng.choice(per, 4, replace=False))
    r, ro, rl = O.cascade_rows(O.dequantize_kv(wl) if values == "fp8" else wl, rows)
    idx = torch.as_tensor(r, device=o.device)
    cmp(o[idx], l[idx], ro, rl)
    assert B.cascade_device_error(clear=True) == 0


# Per-channel scales through each kernel: key-split (16-row chunks, d 128 and
# d 64, split prefixes, trees), pair (one-block chunks), row-split.
CHANNEL_CASES = ["gqa_ragged", "page64_d64", "long_split", "draft_tree", "pair_16row", "rows_split"]


@pytest.mark.parametrize("case", CHANNEL_CASES)
def test_fp8_channel_scales(B, case):
    """FP8 pools with per-channel scales (tutorial page, section 4.5), one
    power of two per (kv head, channel), over pools whose channels span a
    16x range: the fused verify, the three calls and naive expansion against
    the oracle over the dequantised pools."""
    wl = W.with_fp8_kv(cases()[case](), per_channel=True, channel_spread=4.0, seed=61)
    note(f"fp8 channel scales {case}")
    x = B.to_device(wl, layout="HND")
    ref = O.dequantize_kv(wl)
    ro, rl = O.cascade(ref)
    o, l = B.cascade_verify_attn(x)
    oa, la = B.cascade_prefix_attn(x)
    ob, lb = B.cascade_draft_attn(x)
    o3, l3 = B.merge_state(oa, la, ob, lb)
    on, ln = B.naive_expand(x)
    torch.cuda.synchronize()
    cmp(o, l, ro, rl)
    cmp(o3, l3, ro, rl)
    cmp(on, ln, ro, rl)
    assert B.cascade_device_error(clear=True) == 0


def test_fp8_channel_scales_headline(B):
    """The headline shapes over FP8 pools with per-channel scales: the fused
    verify launch (pair kernel, 40-row chunks), all rows."""
    wl = W.with_fp8_kv(W.headline(), per_channel=True, channel_spread=4.0, seed=62)
    note("fp8 channel scales headline")
    x = B.to_device(wl, layout="HND")
    o, l = B.cascade_verify_attn(x, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ro, rl = O.cascade(O.dequantize_kv(wl))
    cmp(o, l, ro, rl)
    assert B.cascade_device_error(clear=True) == 0


@pytest.mark.parametrize("case", CASES)
def test_fp8_naive_expand(B, case):
    wl = fp8_case(case)
    note(f"fp8 naive_expand {case}")
    x = B.to_device(wl)
    o, l = B.naive_expand(x)
    torch.cuda.synchronize()
    ro, rl = O.naive_expand(O.dequantize_kv(wl))
    cmp(o, l, ro, rl)


def test_fp8_widening_is_exact_for_every_code(B):
    """The prefix of request 0 holds all 256 codes (each channel sees many of
    them); the gather hook widens them with the kernels' conversion and must
    give the bf16 bits of each code's value (exact: E4M3 embeds in bf16)."""
    wl = W.build_workload("codes", [64, 16], [[2], [3]], 4, 2, 128, 16, seed=48)
    wl = W.with_fp8_kv(wl)
    L = int(wl.cache_seqlens[0])
    t = np.arange(L)
    pages = wl.page_table[0][t // wl.page_size]
    cell = np.arange(L * wl.head_dim).reshape(L, 1, wl.head_dim)
    heads = np.arange(wl.num_kv_heads).reshape(1, -1, 1)
    ramp = ((cell * 7 + heads * 5) % 256).astype(np.uint8)   # 7 is odd: every code per head
    wl.k_codes[pages, t % wl.page_size] = ramp
    wl.v_codes[pages, t % wl.page_size] = 255 - ramp
    assert all(len(np.unique(ramp[:, g])) == 256 for g in range(wl.num_kv_heads))
    x = B.to_device(wl)
    for g in range(wl.num_kv_heads):
        note(f"fp8 gather kv head {g}")
        k, v = B.cascade_debug_gather(x, 0, 0, g, L)
        torch.cuda.synchronize()
        for got, codes in ((k, ramp[:, g]), (v, 255 - ramp[:, g])):
            bits = got.view(torch.int16).cpu().numpy().view(np.uint16)
            val = O.e4m3_value(codes)
            nan = np.isnan(val)
            f32 = bits.astype(np.uint32) << np.uint32(16)
            assert np.array_equal(np.isnan(f32.view(np.float32)), nan)
            want = W.bf16_bits(np.where(nan, 0.0, val).astype(np.float32))
            assert np.array_equal(bits[~nan], want[~nan])
    assert B.cascade_device_error(clear=True) == 0


def with_room_codes(wl, extra_tokens):
    """A copy of an FP8 workload whose block-table rows map `extra_tokens` more
    slots past every prefix, in fresh zero-coded pages appended to the pool."""
    w = copy.copy(wl)
    P, npg = wl.page_size, wl.k_codes.shape[0]
    need = [-(-(int(L) + extra_tokens) // P) for L in wl.cache_seqlens]
    width = max(max(need), wl.page_table.shape[1])
    extra = width - wl.page_table.shape[1]
    pt = np.zeros((wl.batch_size, width), np.int32)
    pt[:, :wl.page_table.shape[1]] = wl.page_table
    for i in range(wl.batch_size):
        pt[i, wl.page_table.shape[1]:] = npg + i * extra + np.arange(extra)
    fresh = np.zeros((wl.batch_size * extra,) + wl.k_codes.shape[1:], np.uint8)
    w.k_codes = np.concatenate([wl.k_codes, fresh])
    w.v_codes = np.concatenate([wl.v_codes, fresh])
    w.k_pool = np.concatenate([wl.k_pool, fresh.astype(np.float32)])
    w.v_pool = np.concatenate([wl.v_pool, fresh.astype(np.float32)])
    w.page_table = pt
    return w


def codes_nhd(t, layout):
    if layout == "HND":
        t = t.permute(0, 2, 1, 3)
    return t.contiguous().cpu().numpy()


@pytest.mark.parametrize("layout", ["NHD", "HND"])
def test_fp8_append_commit_and_verify(B, layout):
    """Append of E4M3 codes, commit of an accepted path (byte copies, compared
    bit for bit with the oracle's append / commit on the code arrays), then a
    verify step over the committed FP8 prefix."""
    base = W.with_fp8_kv(W.build_workload("step8", [40, 0, 75], [[3, 5], [2], [4, 1, 6]], 8, 2, 128, 16,
                                          seed=62))
    wl = with_room_codes(base, 4)
    x = B.to_device(wl, layout=layout)
    rng = np.random.default_rng(63)
    shape = (wl.total_rows, wl.num_kv_heads, wl.head_dim)
    kn = rng.integers(0, 256, shape, dtype=np.uint8)
    vn = rng.integers(0, 256, shape, dtype=np.uint8)
    kn[(kn & 0x7F) == 0x7F] = 0   # no NaN codes in the appended drafts
    vn[(vn & 0x7F) == 0x7F] = 0
    note(f"fp8 append {layout}")
    B.cascade_append_draft_kv(x, torch.from_numpy(kn).cuda(), torch.from_numpy(vn).cuda())
    wc = copy.copy(wl)
    wc.k_pool, wc.v_pool = wl.k_codes, wl.v_codes
    ko, vo = O.append_draft_kv(wc, kn, vn)
    torch.cuda.synchronize()
    assert np.array_equal(codes_nhd(x.k_pool, layout), ko)
    assert np.array_equal(codes_nhd(x.v_pool, layout), vo)
    assert B.cascade_device_error(clear=True) == 0

    qo, rb = wl.branch_qo_indptr, wl.req_branch_indptr
    acc, ind = [], [0]
    for i in range(wl.batch_size):
        j = int(rb[i])
        n = min(3, int(qo[j + 1] - qo[j]))
        acc += list(range(int(qo[j]), int(qo[j]) + n))
        ind.append(len(acc))
    wa = copy.copy(wc)
    wa.k_pool, wa.v_pool = ko, vo
    kc, vc, lens = O.commit_accepted(wa, np.array(ind), np.array(acc))
    note(f"fp8 commit {layout}")
    B.cascade_commit_accepted(x, torch.tensor(ind, dtype=torch.int32, device="cuda"),
                              torch.tensor(acc, dtype=torch.int32, device="cuda"), 3)
    torch.cuda.synchronize()
    assert np.array_equal(x.cache_seqlens.cpu().numpy(), lens)
    assert np.array_equal(codes_nhd(x.k_pool, layout), kc)
    assert np.array_equal(codes_nhd(x.v_pool, layout), vc)
    assert B.cascade_device_error(clear=True) == 0

    wn = copy.copy(wl)
    wn.k_codes, wn.v_codes, wn.cache_seqlens = kc, vc, lens
    x2 = B.to_device(wn, layout=layout)
    note(f"fp8 verify after commit {layout}")
    o, l = B.cascade_verify_attn(x2)
    ro, rl = O.cascade(O.dequantize_kv(wn))
    torch.cuda.synchronize()
    cmp(o, l, ro, rl)
