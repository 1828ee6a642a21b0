"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any HIP call."""

import ctypes
import os
import re

import pytest

from cascade_attention_tree_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cascade_attn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH), reason="library not built")

FAKE = 0x10000  # a 16-byte aligned non-null address; never dereferenced on the host


def header_functions():
    src = open(HEADER, encoding="utf-8").read()
    return set(re.findall(r"CASCADE_API\s+[\w\s\*]+?\b(\w+)\s*\(", src))


def test_exports_every_declared_symbol():
    declared = header_functions()
    assert declared == set(B.EXPORTED)
    lib = B.lib()
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings():
    lib = B.lib()
    for s in range(6):
        assert lib.cascade_status_string(s)
    assert lib.cascade_status_string(99) == b"unknown status"


def make(B_=2, Hq=8, Hkv=4, d=128, P=16, L=100, rows=6, npages=64, branches=4, dmax=3):
    q = B.Query(FAKE, Hq * d, d, Hq, B_ * rows, d ** -0.5)
    kv = B.PagedKV(FAKE, FAKE, npages, P, Hkv, d, P * Hkv * d, Hkv * d, d)
    stride = -(-L // P)
    t = B.Tree(B_, branches, FAKE, stride, FAKE, FAKE, FAKE, FAKE, 1, None, L, rows, dmax)
    return q, kv, t


def call_verify(q, kv, t, o=FAKE, ws=None, nbytes=0):
    lib = B.lib()
    return lib.cascade_verify_attn(ctypes.byref(q), ctypes.byref(kv), ctypes.byref(t), o,
                                   B.CASCADE_F32, None, ws, nbytes, None)


def test_rejects_before_launch():
    lib = B.lib()
    q, kv, t = make(Hq=6, Hkv=4)
    assert call_verify(q, kv, t) == B.CASCADE_ERR_SHAPE
    assert b"multiple" in lib.cascade_last_error()
    q, kv, t = make(d=96)
    assert call_verify(q, kv, t) == B.CASCADE_ERR_UNSUPPORTED
    q, kv, t = make(P=8)
    assert call_verify(q, kv, t) == B.CASCADE_ERR_UNSUPPORTED
    q, kv, t = make(P=24)
    assert call_verify(q, kv, t) == B.CASCADE_ERR_UNSUPPORTED
    q, kv, t = make()
    kv.k = None
    assert call_verify(q, kv, t) == B.CASCADE_ERR_NULL
    q, kv, t = make()
    t.cache_seqlens = None
    assert call_verify(q, kv, t) == B.CASCADE_ERR_NULL
    q, kv, t = make()
    assert call_verify(q, kv, t, o=None) == B.CASCADE_ERR_NULL
    q, kv, t = make()
    assert call_verify(q, kv, t, o=FAKE + 4) == B.CASCADE_ERR_UNSUPPORTED
    q, kv, t = make()
    kv.token_stride = 1020
    assert call_verify(q, kv, t) == B.CASCADE_ERR_UNSUPPORTED
    q, kv, t = make()
    kv.token_stride = kv.head_dim - 8   # rows of one kv head would overlap
    assert call_verify(q, kv, t) == B.CASCADE_ERR_UNSUPPORTED
    assert b"token_stride" in lib.cascade_last_error()
    q, kv, t = make()
    t.page_table_stride = 3          # 3 pages of 16 cannot hold L = 100
    assert call_verify(q, kv, t) == B.CASCADE_ERR_SHAPE
    q, kv, t = make()
    q.sm_scale = float("nan")
    assert call_verify(q, kv, t) == B.CASCADE_ERR_SHAPE
    # The running max is taken over raw scores and then scaled: only a
    # positive scale keeps it the max of the scaled scores.
    for bad in (-0.125, 0.0):
        q, kv, t = make()
        q.sm_scale = bad
        assert call_verify(q, kv, t) == B.CASCADE_ERR_SHAPE
        assert b"sm_scale" in lib.cascade_last_error()
    q, kv, t = make()
    assert lib.naive_expand(ctypes.byref(q), ctypes.byref(kv), ctypes.byref(t), FAKE, 7, None,
                            None) == B.CASCADE_ERR_UNSUPPORTED


def test_empty_batch_with_long_prefix_bound():
    # No requests but a long max_prefix_len: the split planner must not divide
    # by the (zero) item count, and the calls succeed without launching.
    lib = B.lib()
    q, kv, t = make(B_=0, L=1000, rows=0, branches=0)
    t.page_table_stride = 63
    assert lib.cascade_workspace_size(ctypes.byref(q), ctypes.byref(kv), ctypes.byref(t)) == 0
    assert call_verify(q, kv, t, o=None) == B.CASCADE_OK
    assert lib.cascade_prefix_attn(ctypes.byref(q), ctypes.byref(kv), ctypes.byref(t), None, None,
                                   None, 0, None) == B.CASCADE_OK


def test_workspace_rules():
    lib = B.lib()
    # Headline shape: 32 requests x 8 kv heads fill the GPU, the prefix is not split.
    q, kv, t = make(B_=32, Hq=32, Hkv=8, L=2000, rows=20, branches=128, dmax=5)
    assert lib.cascade_workspace_size(ctypes.byref(q), ctypes.byref(kv), ctypes.byref(t)) == 0
    # Few requests with a long prefix: split, so a workspace is required.
    q, kv, t = make(B_=2, Hq=8, Hkv=4, L=5000, rows=6)
    need = lib.cascade_workspace_size(ctypes.byref(q), ctypes.byref(kv), ctypes.byref(t))
    assert need > 0
    assert call_verify(q, kv, t) == B.CASCADE_ERR_WORKSPACE
    assert call_verify(q, kv, t, ws=FAKE, nbytes=need - 1) == B.CASCADE_ERR_WORKSPACE
    # (o, lse) of every split: splits * rows * Hq * (d + 1) floats, lse block 256-aligned.
    nsplit = need // (12 * 8 * 129 * 4)
    assert nsplit >= 2
    # Invalid arguments give 0.
    q.num_qo_heads = 7
    assert lib.cascade_workspace_size(ctypes.byref(q), ctypes.byref(kv), ctypes.byref(t)) == 0


def test_work_list_workspace():
    lib = B.lib()
    size = lambda q, kv, t: lib.cascade_workspace_size(ctypes.byref(q), ctypes.byref(kv), ctypes.byref(t))
    # 40 query tokens x 8 query heads per kv head = 320 rows per (request, kv
    # head) at head_dim 128, a 400-key prefix (unsplit): the workspace is only
    # the row-split kernel's work list, a 256-byte count block and one int32
    # per (request, split, 128-row chunk).
    q, kv, t = make(B_=4, Hq=16, Hkv=2, L=400, rows=40, branches=8, dmax=10)
    assert size(q, kv, t) == 256 + 4 * (4 * 1 * 3)
    # 80 rows: the key-split or pair kernel, no work list.
    q, kv, t = make(B_=4, Hq=16, Hkv=2, L=400, rows=10, branches=8, dmax=5)
    assert size(q, kv, t) == 0
    # d = 64 has no row-split kernel.
    q, kv, t = make(B_=4, Hq=16, Hkv=2, d=64, L=400, rows=40, branches=8, dmax=10)
    assert size(q, kv, t) == 0
    # A split prefix: the partial states of at least two splits (rows x Hq x
    # (d + 1) floats each), then the list.
    q, kv, t = make(B_=1, Hq=16, Hkv=2, L=9000, rows=40, branches=4, dmax=10, npages=600)
    assert size(q, kv, t) > 2 * 40 * 16 * 129 * 4 + 256


def test_merge_state_validation():
    lib = B.lib()
    assert lib.merge_state(FAKE, FAKE, FAKE, FAKE, 4, 2, 6, FAKE, 0, None, None) == B.CASCADE_ERR_UNSUPPORTED
    assert lib.merge_state(None, FAKE, FAKE, FAKE, 4, 2, 8, FAKE, 0, None, None) == B.CASCADE_ERR_NULL
    assert lib.merge_state(FAKE, FAKE, FAKE, FAKE, -1, 2, 8, FAKE, 0, None, None) == B.CASCADE_ERR_SHAPE
    # nothing to do: OK without touching the GPU
    assert lib.merge_state(None, None, None, None, 0, 2, 8, None, 0, None, None) == B.CASCADE_OK


def test_debug_hook_validation():
    lib = B.lib()
    q, kv, t = make()
    assert lib.cascade_debug_gather(ctypes.byref(kv), ctypes.byref(t), 2, 0, 0, FAKE, FAKE,
                                    None) == B.CASCADE_ERR_SHAPE
    assert lib.cascade_debug_gather(ctypes.byref(kv), ctypes.byref(t), 0, 5, 0, FAKE, FAKE,
                                    None) == B.CASCADE_ERR_SHAPE
    assert lib.cascade_debug_gather(ctypes.byref(kv), ctypes.byref(t), 0, 0, 9, FAKE, FAKE,
                                    None) == B.CASCADE_ERR_SHAPE
    assert lib.cascade_debug_mask(ctypes.byref(t), -1, FAKE, 4, None) == B.CASCADE_ERR_SHAPE


def test_kernel_timing_without_a_timed_call():
    lib = B.lib()
    assert lib.cascade_last_verify_ms(None) == B.CASCADE_ERR_NULL
    assert lib.cascade_kernel_timing(0) == 0
    v = ctypes.c_float(0.0)
    assert lib.cascade_last_verify_ms(ctypes.byref(v)) == B.CASCADE_ERR_SHAPE
    assert b"timed" in lib.cascade_last_error()


def test_draft_tree_limits():
    """A tree of S nodes needs ceil(S / 64) mask words per row (0 words is
    one), at most 64 words; masks are 8-byte aligned."""
    q, kv, t = make(dmax=65)
    t.draft_page_table_stride = 8
    mask = (ctypes.c_uint64 * 64)()
    t.draft_mask = ctypes.addressof(mask)
    for words in (0, 1):
        t.draft_mask_words = words
        assert call_verify(q, kv, t) == B.CASCADE_ERR_UNSUPPORTED
        assert b"64 * draft_mask_words = 64 nodes" in B.lib().cascade_last_error()
    for words in (-1, 65):
        t.draft_mask_words = words
        assert call_verify(q, kv, t) == B.CASCADE_ERR_UNSUPPORTED
        assert b"draft_mask_words" in B.lib().cascade_last_error()
    q, kv, t = make(dmax=129)
    t.draft_page_table_stride = 16
    t.draft_mask = ctypes.addressof(mask)
    t.draft_mask_words = 2
    assert call_verify(q, kv, t) == B.CASCADE_ERR_UNSUPPORTED
    assert b"= 128 nodes" in B.lib().cascade_last_error()
    q, kv, t = make(dmax=64)
    t.draft_page_table_stride = 8
    t.draft_mask = ctypes.addressof(mask) + 4
    assert call_verify(q, kv, t) == B.CASCADE_ERR_UNSUPPORTED
    assert b"8-byte aligned" in B.lib().cascade_last_error()


def test_stream_read_checks():
    lib = B.lib()
    assert lib.cascade_stream_read(None, 0, None, None) == 0
    assert lib.cascade_stream_read(None, 64, None, None) == B.CASCADE_ERR_NULL
    buf = (ctypes.c_uint8 * 128)()
    base = ctypes.addressof(buf)
    aligned = base + (-base) % 16
    sink = (ctypes.c_uint32 * 4)()
    assert lib.cascade_stream_read(aligned + 4, 64, ctypes.addressof(sink), None) == B.CASCADE_ERR_UNSUPPORTED
    assert lib.cascade_stream_read(aligned, 60, ctypes.addressof(sink), None) == B.CASCADE_ERR_UNSUPPORTED


def test_fp8_kv_checks():
    """FP8 pools: the element type must be known and both scales finite and
    positive; bf16 pools ignore the scales (zero is fine there)."""
    q, kv, t = make()
    kv.dtype = 7
    assert call_verify(q, kv, t) == B.CASCADE_ERR_UNSUPPORTED
    assert b"dtype" in B.lib().cascade_last_error()
    for ks, vs in ((0.0, 1.0), (1.0, -2.0), (float("inf"), 1.0), (1.0, float("nan"))):
        q, kv, t = make()
        kv.dtype, kv.k_scale, kv.v_scale = B.KV_FP8_E4M3, ks, vs
        assert call_verify(q, kv, t) == B.CASCADE_ERR_SHAPE
        assert b"k_scale" in B.lib().cascade_last_error()
    # Per-channel scales must be 16-byte aligned (FP8 only; bf16 ignores them).
    for kcs, vcs in ((FAKE + 4, 0), (0, FAKE + 8), (FAKE + 4, FAKE + 4)):
        q, kv, t = make()
        kv.dtype, kv.k_scale, kv.v_scale = B.KV_FP8_E4M3, 1.0, 1.0
        kv.k_channel_scale, kv.v_channel_scale = kcs, vcs
        assert call_verify(q, kv, t) == B.CASCADE_ERR_UNSUPPORTED
        assert b"channel scales" in B.lib().cascade_last_error()
    q, kv, t = make()
    kv.k_channel_scale = FAKE + 4
    assert kv.dtype == B.KV_BF16 and kv.k_scale == 0.0
    kv.head_dim = 96   # a later check still runs: the scales were not the problem
    assert call_verify(q, kv, t) == B.CASCADE_ERR_UNSUPPORTED
    assert b"head_dim" in B.lib().cascade_last_error()


def test_binding_rejects_wrong_output_buffers():
    """A caller's output buffer of the wrong shape, element type or layout is
    refused before any library call (the C ABI cannot check its extent)."""
    import torch
    from cascade_attention_tree_amd import binding as B
    from cascade_attention_tree_amd import workload as W
    wl = W.tiny(values="bf16")
    x = B.to_device(wl, "cpu")
    R, Hq, d = x.q.shape
    bad = [torch.empty((R, Hq, d - 1)), torch.empty((R, Hq, d), dtype=torch.float16),
           torch.empty((R, d, Hq)).transpose(1, 2)]
    for o in bad:
        with pytest.raises(ValueError):
            B.cascade_verify_attn(x, o=o)
        with pytest.raises(ValueError):
            B.cascade_prefix_attn(x, o_a=o)
        with pytest.raises(ValueError):
            B.cascade_draft_attn(x, o_b=o)
        with pytest.raises(ValueError):
            B.naive_expand(x, o=o)
    with pytest.raises(ValueError):
        B.cascade_verify_attn(x, lse=torch.empty((R, Hq + 1)))
