"""ctypes binding of libcascade_attn.so.

Argument marshalling only: every step of the attention path runs in the
library's HIP kernels.  torch tensors serve as device memory and streams.
Functions carry the names of the C entry points they call.  The library is
loaded on first use; if it is missing every call raises.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from . import workload as _wl

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcascade_attn.so")

CASCADE_OK = 0
CASCADE_ERR_NULL = 1
CASCADE_ERR_SHAPE = 2
CASCADE_ERR_UNSUPPORTED = 3
CASCADE_ERR_WORKSPACE = 4
CASCADE_ERR_HIP = 5
CASCADE_F32 = 0
CASCADE_BF16 = 1

EXPORTED = (
    "cascade_workspace_size", "cascade_prefix_attn", "cascade_draft_attn", "merge_state",
    "cascade_verify_attn", "naive_expand", "cascade_status_string", "cascade_last_error",
    "cascade_debug_gather", "cascade_debug_mask", "cascade_device_error",
    "cascade_kernel_timing", "cascade_last_verify_ms", "cascade_append_draft_kv",
    "cascade_commit_accepted", "cascade_stream_read", "cascade_verify_attn_noalloc",
)


class PagedKV(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("num_pages", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("page_stride", ctypes.c_int64), ("token_stride", ctypes.c_int64),
                ("head_stride", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
                ("k_channel_scale", ctypes.c_void_p), ("v_channel_scale", ctypes.c_void_p)]


KV_BF16 = 0
KV_FP8_E4M3 = 1


class Query(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("row_stride", ctypes.c_int64),
                ("head_stride", ctypes.c_int64), ("num_qo_heads", ctypes.c_int32),
                ("total_rows", ctypes.c_int32), ("sm_scale", ctypes.c_float)]


class Tree(ctypes.Structure):
    _fields_ = [("batch_size", ctypes.c_int32), ("num_branches", ctypes.c_int32),
                ("page_table", ctypes.c_void_p), ("page_table_stride", ctypes.c_int32),
                ("cache_seqlens", ctypes.c_void_p), ("req_branch_indptr", ctypes.c_void_p),
                ("branch_qo_indptr", ctypes.c_void_p), ("draft_page_table", ctypes.c_void_p),
                ("draft_page_table_stride", ctypes.c_int32), ("draft_start", ctypes.c_void_p),
                ("max_prefix_len", ctypes.c_int32), ("max_request_rows", ctypes.c_int32),
                ("max_draft_len", ctypes.c_int32), ("draft_mask", ctypes.c_void_p),
                ("draft_mask_words", ctypes.c_int32)]


class CascadeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"status {status}: {message}")
        self.status = status


_LIB = None


def lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built (run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        st = ctypes.c_int
        vp = ctypes.c_void_p
        L.cascade_workspace_size.argtypes = [P(Query), P(PagedKV), P(Tree)]
        L.cascade_workspace_size.restype = ctypes.c_size_t
        L.cascade_prefix_attn.argtypes = [P(Query), P(PagedKV), P(Tree), vp, vp, vp, ctypes.c_size_t, vp]
        L.cascade_prefix_attn.restype = st
        L.cascade_draft_attn.argtypes = [P(Query), P(PagedKV), P(Tree), vp, vp, vp]
        L.cascade_draft_attn.restype = st
        L.merge_state.argtypes = [vp, vp, vp, vp, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                  vp, ctypes.c_int, vp, vp]
        L.merge_state.restype = st
        L.cascade_verify_attn.argtypes = [P(Query), P(PagedKV), P(Tree), vp, ctypes.c_int, vp, vp,
                                          ctypes.c_size_t, vp]
        L.cascade_verify_attn.restype = st
        L.cascade_verify_attn_noalloc.argtypes = [P(Query), P(PagedKV), P(Tree), vp, ctypes.c_int, vp, vp]
        L.cascade_verify_attn_noalloc.restype = st
        L.naive_expand.argtypes = [P(Query), P(PagedKV), P(Tree), vp, ctypes.c_int, vp, vp]
        L.naive_expand.restype = st
        L.cascade_status_string.argtypes = [ctypes.c_int]
        L.cascade_status_string.restype = ctypes.c_char_p
        L.cascade_last_error.argtypes = []
        L.cascade_last_error.restype = ctypes.c_char_p
        L.cascade_debug_gather.argtypes = [P(PagedKV), P(Tree), ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_int32, vp, vp, vp]
        L.cascade_debug_gather.restype = st
        L.cascade_debug_mask.argtypes = [P(Tree), ctypes.c_int32, vp, ctypes.c_int32, vp]
        L.cascade_debug_mask.restype = st
        L.cascade_device_error.argtypes = [P(ctypes.c_int32), ctypes.c_int32]
        L.cascade_device_error.restype = st
        L.cascade_append_draft_kv.argtypes = [P(PagedKV), P(Tree), ctypes.c_int32, vp, vp,
                                              ctypes.c_int64, ctypes.c_int64, vp]
        L.cascade_append_draft_kv.restype = st
        L.cascade_commit_accepted.argtypes = [P(PagedKV), P(Tree), ctypes.c_int32, vp, vp,
                                              ctypes.c_int32, vp, vp]
        L.cascade_commit_accepted.restype = st
        L.cascade_stream_read.argtypes = [vp, ctypes.c_size_t, vp, vp]
        L.cascade_stream_read.restype = st
        L.cascade_kernel_timing.argtypes = [ctypes.c_int32]
        L.cascade_kernel_timing.restype = st
        L.cascade_last_verify_ms.argtypes = [P(ctypes.c_float)]
        L.cascade_last_verify_ms.restype = st
        _LIB = L
    return _LIB


def _check(status: int) -> None:
    if status != CASCADE_OK:
        raise CascadeError(status, lib().cascade_last_error().decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


# ---------------------------------------------------------------------------
# Device-side inputs
# ---------------------------------------------------------------------------

@dataclass
class DeviceInputs:
    """A workload's arrays on the GPU, plus the C structs that point at them."""
    q: torch.Tensor            # bf16 [R, Hq, d]
    k_pool: torch.Tensor       # bf16 (or uint8 E4M3 codes) [pages, P, Hkv, d]
    v_pool: torch.Tensor
    page_table: torch.Tensor   # int32
    cache_seqlens: torch.Tensor
    req_branch_indptr: torch.Tensor
    branch_qo_indptr: torch.Tensor
    draft_page_table: torch.Tensor
    draft_start: torch.Tensor
    query: Query
    kv: PagedKV
    tree: Tree
    draft_mask: Optional[torch.Tensor] = None   # int64 view of the uint64 ancestor masks
    k_channel_scale: Optional[torch.Tensor] = None  # fp32 [Hkv, d] (FP8 per-channel scales)
    v_channel_scale: Optional[torch.Tensor] = None

    @property
    def total_rows(self) -> int:
        return int(self.query.total_rows)


def _bf16_tensor(x: np.ndarray, device) -> torch.Tensor:
    bits = _wl.bf16_bits(x).view(np.int16)
    return torch.from_numpy(bits).to(device).view(torch.bfloat16)


def make_structs(q, k_pool, v_pool, page_table, cache_seqlens, req_branch_indptr,
                 branch_qo_indptr, draft_page_table, draft_start, sm_scale,
                 max_prefix_len, max_request_rows, max_draft_len, layout="NHD",
                 draft_mask=None, k_scale=1.0, v_scale=1.0, k_channel_scale=None,
                 v_channel_scale=None):
    """layout "NHD": pools are [pages, P, Hkv, d]; "HND": [pages, Hkv, P, d].
    Pools are bf16, or uint8 / float8_e4m3fn E4M3 codes with the per-tensor
    scales k_scale, v_scale and optional per-channel scales (fp32 device
    tensors [Hkv, d]).  draft_mask: optional ancestor masks (draft trees), one
    64-bit word per row ([rows]) or W words per row ([rows, W])."""
    R, Hq, d = q.shape
    assert k_pool.stride() == v_pool.stride()
    if layout == "NHD":
        num_pages, P, Hkv, _ = k_pool.shape
        ps, ts, hs = k_pool.stride(0), k_pool.stride(1), k_pool.stride(2)
    elif layout == "HND":
        num_pages, Hkv, P, _ = k_pool.shape
        ps, ts, hs = k_pool.stride(0), k_pool.stride(2), k_pool.stride(1)
    else:
        raise ValueError(layout)
    query = Query(q.data_ptr(), q.stride(0), q.stride(1), Hq, R, float(sm_scale))
    fp8 = k_pool.dtype in (torch.uint8, torch.float8_e4m3fn)
    assert k_pool.dtype == v_pool.dtype and (fp8 or k_pool.dtype == torch.bfloat16)
    kv = PagedKV(k_pool.data_ptr(), v_pool.data_ptr(), num_pages, P, Hkv, d, ps, ts, hs,
                 KV_FP8_E4M3 if fp8 else KV_BF16, float(k_scale) if fp8 else 0.0,
                 float(v_scale) if fp8 else 0.0, _ptr(k_channel_scale) if fp8 else None,
                 _ptr(v_channel_scale) if fp8 else None)
    tree = Tree(int(cache_seqlens.shape[0]), int(branch_qo_indptr.shape[0] - 1),
                page_table.data_ptr(), page_table.stride(0), cache_seqlens.data_ptr(),
                req_branch_indptr.data_ptr(), branch_qo_indptr.data_ptr(),
                draft_page_table.data_ptr(), draft_page_table.stride(0),
                _ptr(draft_start), int(max_prefix_len), int(max_request_rows), int(max_draft_len),
                _ptr(draft_mask), 1 if draft_mask is None or draft_mask.dim() == 1 else int(draft_mask.shape[1]))
    return query, kv, tree


def to_device(wl: "_wl.Workload", device="cuda", layout="NHD") -> DeviceInputs:
    """Uploads a workload (bf16 values, or its E4M3 codes when it has FP8 KV;
    int32 tables) and builds its C structs.

    layout "NHD" keeps the generator's token-major pages [pages, P, Hkv, d];
    "HND" stores each page head-major, [pages, Hkv, P, d], so that one kv head's
    tokens of a page are one contiguous run (same logical content)."""
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(device)
    q = _bf16_tensor(wl.q, device)
    fp8 = getattr(wl, "k_codes", None) is not None
    if fp8:
        k = torch.from_numpy(np.ascontiguousarray(wl.k_codes, np.uint8)).to(device)
        v = torch.from_numpy(np.ascontiguousarray(wl.v_codes, np.uint8)).to(device)
    else:
        k = _bf16_tensor(wl.k_pool, device)
        v = _bf16_tensor(wl.v_pool, device)
    if layout == "HND":
        k = k.permute(0, 2, 1, 3).contiguous()
        v = v.permute(0, 2, 1, 3).contiguous()
    pt, cs, rb = i32(wl.page_table), i32(wl.cache_seqlens), i32(wl.req_branch_indptr)
    qo, dpt, ds = i32(wl.branch_qo_indptr), i32(wl.draft_page_table), i32(wl.draft_start)
    dm = None
    if getattr(wl, "draft_mask", None) is not None:
        dm = torch.from_numpy(np.ascontiguousarray(wl.draft_mask, np.uint64).view(np.int64)).to(device)
    kcs = vcs = None
    if fp8 and getattr(wl, "k_channel_scale", None) is not None:
        f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device)
        kcs, vcs = f32(wl.k_channel_scale), f32(wl.v_channel_scale)
    query, kv, tree = make_structs(q, k, v, pt, cs, rb, qo, dpt, ds, wl.sm_scale,
                                   wl.max_prefix_len(), wl.max_rows_per_request(),
                                   wl.max_draft_len(), layout, draft_mask=dm,
                                   k_scale=wl.k_scale if fp8 else 1.0, v_scale=wl.v_scale if fp8 else 1.0,
                                   k_channel_scale=kcs, v_channel_scale=vcs)
    return DeviceInputs(q, k, v, pt, cs, rb, qo, dpt, ds, query, kv, tree, dm, kcs, vcs)


# ---------------------------------------------------------------------------
# Entry points
# ---------------------------------------------------------------------------

def cascade_workspace_size(x: DeviceInputs) -> int:
    return int(lib().cascade_workspace_size(ctypes.byref(x.query), ctypes.byref(x.kv),
                                            ctypes.byref(x.tree)))


def workspace_for(x: DeviceInputs) -> Optional[torch.Tensor]:
    n = cascade_workspace_size(x)
    return torch.empty(n, dtype=torch.uint8, device=x.q.device) if n else None


def _out_shape(x: DeviceInputs):
    R, Hq, d = x.q.shape
    return (R, Hq, d), (R, Hq)


def _out(t, shape, dtypes, like):
    """An output buffer: a new one of dtypes[0], or the caller's, which must have
    the shape, one of the element types, contiguity and device the kernels write
    (the C ABI cannot check a buffer's extent)."""
    if t is None:
        return torch.empty(shape, dtype=dtypes[0], device=like.device)
    if tuple(t.shape) != tuple(shape) or t.dtype not in dtypes or not t.is_contiguous() or t.device != like.device:
        raise ValueError(f"output buffer {tuple(t.shape)} {t.dtype} on {t.device}: expected a contiguous "
                         f"{tuple(shape)} tensor of {[str(d) for d in dtypes]} on {like.device}")
    return t


def cascade_prefix_attn(x: DeviceInputs, o_a=None, lse_a=None, workspace=None, stream=None):
    """Pass A.  Returns (o_A float32 [R, Hq, d], LSE_A float32 [R, Hq])."""
    so, sl = _out_shape(x)
    o_a = _out(o_a, so, (torch.float32,), x.q)
    lse_a = _out(lse_a, sl, (torch.float32,), x.q)
    if workspace is None:
        workspace = workspace_for(x)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().cascade_prefix_attn(ctypes.byref(x.query), ctypes.byref(x.kv), ctypes.byref(x.tree),
                                     o_a.data_ptr(), lse_a.data_ptr(), _ptr(workspace), nbytes,
                                     _stream(stream)))
    return o_a, lse_a


def cascade_draft_attn(x: DeviceInputs, o_b=None, lse_b=None, stream=None):
    """Pass B.  Returns (o_B float32 [R, Hq, d], LSE_B float32 [R, Hq])."""
    so, sl = _out_shape(x)
    o_b = _out(o_b, so, (torch.float32,), x.q)
    lse_b = _out(lse_b, sl, (torch.float32,), x.q)
    _check(lib().cascade_draft_attn(ctypes.byref(x.query), ctypes.byref(x.kv), ctypes.byref(x.tree),
                                    o_b.data_ptr(), lse_b.data_ptr(), _stream(stream)))
    return o_b, lse_b


def merge_state(o_a, lse_a, o_b, lse_b, out_dtype=torch.float32, o=None, lse=None, stream=None):
    """LSE merge of two states; o_* float32 [..., H, d], lse_* float32 [..., H]."""
    assert o_a.shape == o_b.shape and lse_a.shape == lse_b.shape
    assert o_a.dtype == torch.float32 and lse_a.dtype == torch.float32
    for t in (o_a, lse_a, o_b, lse_b):
        assert t.is_contiguous()
    H, d = o_a.shape[-2], o_a.shape[-1]
    rows = o_a.numel() // (H * d)
    o = torch.empty(o_a.shape, dtype=out_dtype, device=o_a.device) if o is None else o
    lse = torch.empty(lse_a.shape, dtype=torch.float32, device=o_a.device) if lse is None else lse
    # The element type written is the one of `o` (a given `o` overrides out_dtype).
    assert o.dtype in (torch.float32, torch.bfloat16) and o.is_contiguous() and o.numel() == o_a.numel()
    assert lse.dtype == torch.float32 and lse.is_contiguous() and lse.numel() == lse_a.numel()
    _check(lib().merge_state(o_a.data_ptr(), lse_a.data_ptr(), o_b.data_ptr(), lse_b.data_ptr(),
                             rows, H, d, o.data_ptr(),
                             CASCADE_BF16 if o.dtype == torch.bfloat16 else CASCADE_F32,
                             _ptr(lse), _stream(stream)))
    return o, lse


def cascade_verify_attn(x: DeviceInputs, out_dtype=torch.float32, o=None, lse=None, workspace=None,
                        stream=None, want_lse=True):
    """Pass A + pass B + merge.  Returns (o [R, Hq, d], LSE float32 [R, Hq] or None)."""
    so, sl = _out_shape(x)
    o = _out(o, so, (out_dtype, torch.bfloat16 if out_dtype == torch.float32 else torch.float32), x.q)
    if lse is not None or want_lse:
        lse = _out(lse, sl, (torch.float32,), x.q)
    if workspace is None:
        workspace = workspace_for(x)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().cascade_verify_attn(ctypes.byref(x.query), ctypes.byref(x.kv), ctypes.byref(x.tree),
                                     o.data_ptr(),
                                     CASCADE_BF16 if o.dtype == torch.bfloat16 else CASCADE_F32,
                                     _ptr(lse), _ptr(workspace), nbytes, _stream(stream)))
    return o, lse


def cascade_verify_attn_noalloc(x: DeviceInputs, out_dtype=torch.float32, o=None, lse=None, stream=None,
                                want_lse=True):
    """cascade_verify_attn with the library's built-in workspace (no device
    allocation by the library)."""
    so, sl = _out_shape(x)
    o = _out(o, so, (out_dtype, torch.bfloat16 if out_dtype == torch.float32 else torch.float32), x.q)
    if lse is not None or want_lse:
        lse = _out(lse, sl, (torch.float32,), x.q)
    _check(lib().cascade_verify_attn_noalloc(ctypes.byref(x.query), ctypes.byref(x.kv), ctypes.byref(x.tree),
                                             o.data_ptr(),
                                             CASCADE_BF16 if o.dtype == torch.bfloat16 else CASCADE_F32,
                                             _ptr(lse), _stream(stream)))
    return o, lse


def naive_expand(x: DeviceInputs, out_dtype=torch.float32, o=None, lse=None, stream=None,
                 want_lse=True):
    """Baseline: one softmax per branch over prefix + own drafts."""
    so, sl = _out_shape(x)
    o = _out(o, so, (out_dtype, torch.bfloat16 if out_dtype == torch.float32 else torch.float32), x.q)
    if lse is not None or want_lse:
        lse = _out(lse, sl, (torch.float32,), x.q)
    _check(lib().naive_expand(ctypes.byref(x.query), ctypes.byref(x.kv), ctypes.byref(x.tree),
                              o.data_ptr(), CASCADE_BF16 if o.dtype == torch.bfloat16 else CASCADE_F32,
                              _ptr(lse), _stream(stream)))
    return o, lse


def cascade_debug_gather(x: DeviceInputs, which: int, index: int, kv_head: int, count: int):
    d = x.q.shape[2]
    k = torch.empty((max(count, 1), d), dtype=torch.bfloat16, device=x.q.device)
    v = torch.empty_like(k)
    _check(lib().cascade_debug_gather(ctypes.byref(x.kv), ctypes.byref(x.tree), which, index,
                                      kv_head, k.data_ptr(), v.data_ptr(), _stream(None)))
    return k[:count], v[:count]


def cascade_debug_mask(x: DeviceInputs, branch: int, rows: int, cols: int):
    m = torch.zeros((max(rows, 1), max(cols, 1)), dtype=torch.uint8, device=x.q.device)
    _check(lib().cascade_debug_mask(ctypes.byref(x.tree), branch, m.data_ptr(), cols, _stream(None)))
    return m[:rows, :cols]


def cascade_device_error(clear: bool = True) -> int:
    v = ctypes.c_int32(0)
    _check(lib().cascade_device_error(ctypes.byref(v), 1 if clear else 0))
    return int(v.value)


def cascade_kernel_timing(enable: bool) -> None:
    _check(lib().cascade_kernel_timing(1 if enable else 0))


def cascade_last_verify_ms() -> float:
    v = ctypes.c_float(0.0)
    _check(lib().cascade_last_verify_ms(ctypes.byref(v)))
    return float(v.value)


def cascade_append_draft_kv(x: DeviceInputs, k_new: torch.Tensor, v_new: torch.Tensor, stream=None) -> None:
    """Writes every query row's draft K/V ([total_rows, Hkv, d] in the pool's
    element type: bf16, or E4M3 codes for an FP8 pool) into its slot of the
    paged pool of ``x`` (in place)."""
    assert k_new.dtype == x.k_pool.dtype and v_new.dtype == x.k_pool.dtype
    assert k_new.stride() == v_new.stride() and k_new.shape == v_new.shape
    _check(lib().cascade_append_draft_kv(ctypes.byref(x.kv), ctypes.byref(x.tree), x.total_rows,
                                         k_new.data_ptr(), v_new.data_ptr(), k_new.stride(0),
                                         k_new.stride(1), _stream(stream)))


def cascade_commit_accepted(x: DeviceInputs, accepted_indptr: torch.Tensor, accepted_rows: torch.Tensor,
                            max_accepted: int, cache_seqlens_out: Optional[torch.Tensor] = None,
                            stream=None) -> None:
    """Appends each request's accepted draft rows (int32 device tensors) to its
    prefix in the pool of ``x``; lengths go to ``cache_seqlens_out`` (default:
    ``x.cache_seqlens`` in place)."""
    out = x.cache_seqlens if cache_seqlens_out is None else cache_seqlens_out
    _check(lib().cascade_commit_accepted(ctypes.byref(x.kv), ctypes.byref(x.tree), x.total_rows,
                                         accepted_indptr.data_ptr(), _ptr(accepted_rows),
                                         int(max_accepted), out.data_ptr(), _stream(stream)))


def cascade_stream_read(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Plain streaming read of ``buf`` (a measurement reference)."""
    _check(lib().cascade_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(),
                                     _stream(stream)))
