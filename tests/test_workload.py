"""Host-side checks of the seeded input generator (CPU only)."""

import math

import numpy as np

from cascade_attention_tree_amd import workload as W


def test_deterministic_and_seed_sensitive():
    a = W.tiny(values="bf16")
    b = W.tiny(values="bf16")
    c = W.tiny(values="bf16", seed=5)
    for f in ("q", "k_pool", "v_pool", "page_table", "draft_page_table"):
        assert np.array_equal(getattr(a, f), getattr(b, f), equal_nan=True)
    assert not np.array_equal(a.q, c.q)


def test_bf16_values_are_exact():
    wl = W.tiny(values="bf16")
    assert np.array_equal(W.round_to_bf16(wl.q), wl.q)
    finite = wl.k_pool[np.isfinite(wl.k_pool)]
    assert np.array_equal(W.round_to_bf16(finite), finite)
    bits = W.bf16_bits(wl.q)
    assert np.array_equal((bits.astype(np.uint32) << 16).view(np.float32), wl.q)


def test_unused_slots_are_nan_and_pages_permuted():
    wl = W.build_workload("t", [20, 7], [[3, 2], [17]], 4, 2, 8, page_size=16, seed=1)
    used = np.zeros(wl.k_pool.shape[:2], bool)
    for i in range(wl.batch_size):
        L = wl.cache_seqlens[i]
        for t in range(L):
            used[wl.page_table[i, t // 16], t % 16] = True
    for j in range(wl.num_branches):
        S = wl.branch_qo_indptr[j + 1] - wl.branch_qo_indptr[j]
        for u in range(S):
            used[wl.draft_page_table[j, u // 16], u % 16] = True
    assert np.all(np.isfinite(wl.k_pool[used])) and np.all(np.isnan(wl.k_pool[~used]))
    assert used.sum() == 20 + 7 + 3 + 2 + 17
    # spare pages exist and padding entries of the tables point at one
    spare = wl.meta["spare_page"]
    assert wl.page_table[1, 1] == spare and np.all(np.isnan(wl.k_pool[spare]))


def test_config_shapes():
    wl = W.headline()
    assert wl.batch_size == 32 and wl.num_branches == 128 and wl.total_rows == 640
    assert wl.q.shape == (640, 32, 128) and wl.k_pool.shape[1:] == (16, 8, 128)
    assert wl.max_rows_per_request() == 20 and wl.max_prefix_len() == 2000
    g = W.gqa()
    assert g.total_rows == 96 and g.page_table.shape == (8, math.ceil(1000 / 16))
    r = W.ragged(batch=8)
    L = r.cache_seqlens
    assert np.all((L >= 512) & (L <= 32768))
    topk = np.diff(r.req_branch_indptr)
    assert set(topk.tolist()) <= {2, 4, 8}
    assert set(r.draft_lens.tolist()) <= set(range(3, 9))
    for h, H in ((0.0, 0), (0.5, 4096), (0.9, 7372)):
        p = W.prefix_hit(h, batch=1)
        assert p.meta["H"] == H and p.total_rows == 8192 - H
        assert p.draft_start[0] == H
        assert np.array_equal(p.draft_page_table[0, :p.page_table.shape[1]], p.page_table[0])
