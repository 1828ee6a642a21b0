"""Seeded synthetic inputs for verify attention over a paged KV cache.

This module only draws random values and lays them out (page pool, block
tables, row order).  It holds none of the attention arithmetic, so the CPU
oracle and the GPU path can both consume what it produces.

Layout (all host numpy arrays; the GPU side uploads them unchanged):

* ``q``            float32 ``[total_rows, Hq, d]``; rows are request-major, then
                   branch, then draft position.
* ``k_pool/v_pool`` float32 ``[num_pages, page_size, Hkv, d]`` (one layer's K or
                   V, token-major "NHD" pages).  Values are exact bf16 numbers
                   when ``values == "bf16"``.  Slots that hold no token, and the
                   spare pages, are NaN so that a stray read shows up.
* ``page_table``   int32 ``[B, max_pages]``: logical prefix page -> physical page
                   (the per-request block table).  Entries past a request's last
                   page point at a spare NaN page.
* ``cache_seqlens`` int32 ``[B]``: prefix length L_i.
* ``req_branch_indptr`` int32 ``[B+1]``: branches of request i are
                   ``[indptr[i], indptr[i+1])``.
* ``branch_qo_indptr`` int32 ``[NV+1]``: query rows of branch j; the branch has
                   S_j = diff draft tokens, which are both its queries and its
                   draft keys.
* ``draft_page_table`` int32 ``[NV, max_draft_pages]`` and ``draft_start`` int32
                   ``[NV]``: draft token u of branch j sits at logical slot
                   ``draft_start[j] + u`` of the pages listed in row j.

Draw order for a given seed (numpy PCG64 ``default_rng``): shape draws (ragged
configurations only), then Q, then K of every token in logical order, then V,
then the physical page permutation.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even).

    Returns float32 holding the rounded values exactly.  Non-finite inputs are
    passed through unchanged.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    r = ((u + bias) & np.uint32(0xFFFF0000)).view(np.float32)
    return np.where(np.isfinite(x), r, x).astype(np.float32, copy=False)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already exact bf16 numbers."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


@dataclass
class Workload:
    name: str
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    sm_scale: float
    q: np.ndarray
    k_pool: np.ndarray
    v_pool: np.ndarray
    page_table: np.ndarray
    cache_seqlens: np.ndarray
    req_branch_indptr: np.ndarray
    branch_qo_indptr: np.ndarray
    draft_page_table: np.ndarray
    draft_start: np.ndarray
    # General draft trees (None: every branch is a chain).  Per query row, the
    # parent of its node within its branch (-1: the node hangs off the prefix)
    # and the node's ancestor set as a bit mask over the branch's nodes (bit u:
    # node u is the row's node or one of its ancestors).  Nodes are numbered in
    # breadth-first order, so a parent always precedes its children.
    draft_parent: Optional[np.ndarray] = None
    draft_mask: Optional[np.ndarray] = None
    # FP8 KV (None: the pools are bf16).  E4M3 codes (uint8, same shape as
    # k_pool / v_pool) and the per-tensor scales: element x of the pool is held
    # as code(x / scale).  k_pool / v_pool keep the unquantised values.
    k_codes: Optional[np.ndarray] = None
    v_codes: Optional[np.ndarray] = None
    k_scale: float = 1.0
    v_scale: float = 1.0
    # Optional per-channel scales [Hkv, d] (float32): element (page, slot, g, c)
    # is held as code(x / (scale * channel_scale[g, c])).
    k_channel_scale: Optional[np.ndarray] = None
    v_channel_scale: Optional[np.ndarray] = None
    # Logical (unpaged) copies, kept only when asked for: per request the prefix
    # tokens [L_i, Hkv, d], per branch its draft tokens [S_j, Hkv, d].
    prefix_k: Optional[List[np.ndarray]] = None
    prefix_v: Optional[List[np.ndarray]] = None
    draft_k: Optional[List[np.ndarray]] = None
    draft_v: Optional[List[np.ndarray]] = None
    meta: dict = field(default_factory=dict)

    @property
    def batch_size(self) -> int:
        return int(self.cache_seqlens.shape[0])

    @property
    def num_branches(self) -> int:
        return int(self.branch_qo_indptr.shape[0] - 1)

    @property
    def total_rows(self) -> int:
        return int(self.branch_qo_indptr[-1])

    @property
    def draft_lens(self) -> np.ndarray:
        return np.diff(self.branch_qo_indptr).astype(np.int32)

    def request_of_branch(self) -> np.ndarray:
        out = np.empty(self.num_branches, np.int32)
        for i in range(self.batch_size):
            out[self.req_branch_indptr[i]:self.req_branch_indptr[i + 1]] = i
        return out

    def max_rows_per_request(self) -> int:
        rb = self.req_branch_indptr
        qo = self.branch_qo_indptr
        return int(max(qo[rb[i + 1]] - qo[rb[i]] for i in range(self.batch_size)))

    def max_draft_len(self) -> int:
        return int(self.draft_lens.max()) if self.num_branches else 0

    def max_prefix_len(self) -> int:
        return int(self.cache_seqlens.max()) if self.batch_size else 0


def build_workload(name: str,
                   prefix_lens: Sequence[int],
                   branch_lens: Sequence[Sequence[int]],
                   num_qo_heads: int,
                   num_kv_heads: int,
                   head_dim: int,
                   page_size: int = 16,
                   seed: int = 0,
                   values: str = "bf16",
                   spare_frac: float = 0.1,
                   suffix_in_prefix_pages: bool = False,
                   keep_logical: bool = False,
                   rng: Optional[np.random.Generator] = None) -> Workload:
    """Draw Q/K/V ~ N(0,1) and scatter K/V into randomly permuted pages.

    ``branch_lens[i]`` lists S_j for the branches of request i.  With
    ``suffix_in_prefix_pages`` each request has exactly one branch whose tokens
    continue the prefix inside the same pages (a prefix-cache hit followed by a
    suffix), so that branch's draft page row is the request's page row and its
    ``draft_start`` is L_i.
    """
    if values not in ("bf16", "fp32"):
        raise ValueError("values must be 'bf16' or 'fp32'")
    if num_qo_heads % num_kv_heads:
        raise ValueError("num_qo_heads must be a multiple of num_kv_heads")
    rng = rng if rng is not None else np.random.default_rng(seed)
    B = len(prefix_lens)
    P = int(page_size)
    Hq, Hkv, d = int(num_qo_heads), int(num_kv_heads), int(head_dim)
    prefix_lens = np.asarray(prefix_lens, np.int64)
    if suffix_in_prefix_pages and any(len(b) != 1 for b in branch_lens):
        raise ValueError("suffix_in_prefix_pages needs exactly one branch per request")

    req_branch_indptr = np.zeros(B + 1, np.int32)
    sj: List[int] = []
    for i in range(B):
        req_branch_indptr[i + 1] = req_branch_indptr[i] + len(branch_lens[i])
        sj.extend(int(s) for s in branch_lens[i])
    NV = len(sj)
    branch_qo_indptr = np.zeros(NV + 1, np.int32)
    branch_qo_indptr[1:] = np.cumsum(sj) if NV else []
    R = int(branch_qo_indptr[-1])

    def draw(shape):
        a = rng.standard_normal(shape, dtype=np.float32)
        return round_to_bf16(a) if values == "bf16" else a

    q = draw((R, Hq, d))
    n_prefix_tok = int(prefix_lens.sum())
    n_tok = n_prefix_tok + R
    k_tok = draw((n_tok, Hkv, d))
    v_tok = draw((n_tok, Hkv, d))

    # Logical page demand: request prefixes first, then branch drafts.
    if suffix_in_prefix_pages:
        req_pages = [-(-int(prefix_lens[i] + sj[i]) // P) for i in range(B)]
        draft_pages = [0] * NV
    else:
        req_pages = [-(-int(prefix_lens[i]) // P) for i in range(B)]
        draft_pages = [-(-s // P) for s in sj]
    n_need = sum(req_pages) + sum(draft_pages)
    n_spare = max(1, int(math.ceil(spare_frac * n_need)))
    num_pages = n_need + n_spare
    perm = rng.permutation(num_pages).astype(np.int32)
    spare_page = int(perm[n_need])

    max_pages = max([1] + req_pages)
    page_table = np.full((B, max_pages), spare_page, np.int32)
    cur = 0
    for i in range(B):
        page_table[i, :req_pages[i]] = perm[cur:cur + req_pages[i]]
        cur += req_pages[i]
    max_dpages = max([1] + draft_pages + (req_pages if suffix_in_prefix_pages else []))
    draft_page_table = np.full((NV, max_dpages), spare_page, np.int32)
    draft_start = np.zeros(NV, np.int32)
    if suffix_in_prefix_pages:
        for i in range(B):
            j = int(req_branch_indptr[i])
            draft_page_table[j, :req_pages[i]] = page_table[i, :req_pages[i]]
            draft_start[j] = int(prefix_lens[i])
    else:
        for j in range(NV):
            draft_page_table[j, :draft_pages[j]] = perm[cur:cur + draft_pages[j]]
            cur += draft_pages[j]

    # Physical slot of every token, then scatter.
    phys = np.empty(n_tok, np.int64)
    tok = 0
    for i in range(B):
        L = int(prefix_lens[i])
        t = np.arange(L)
        phys[tok:tok + L] = page_table[i, t // P].astype(np.int64) * P + t % P
        tok += L
    for j in range(NV):
        S = sj[j]
        u = draft_start[j] + np.arange(S)
        phys[tok:tok + S] = draft_page_table[j, u // P].astype(np.int64) * P + u % P
        tok += S
    assert tok == n_tok
    assert np.unique(phys).size == n_tok, "two tokens mapped to one slot"

    k_pool = np.full((num_pages * P, Hkv, d), np.nan, np.float32)
    v_pool = np.full((num_pages * P, Hkv, d), np.nan, np.float32)
    k_pool[phys] = k_tok
    v_pool[phys] = v_tok
    k_pool = k_pool.reshape(num_pages, P, Hkv, d)
    v_pool = v_pool.reshape(num_pages, P, Hkv, d)

    wl = Workload(name=name, num_qo_heads=Hq, num_kv_heads=Hkv, head_dim=d,
                  page_size=P, sm_scale=1.0 / math.sqrt(d), q=q,
                  k_pool=k_pool, v_pool=v_pool, page_table=page_table,
                  cache_seqlens=prefix_lens.astype(np.int32),
                  req_branch_indptr=req_branch_indptr,
                  branch_qo_indptr=branch_qo_indptr,
                  draft_page_table=draft_page_table, draft_start=draft_start,
                  meta={"seed": seed, "values": values, "num_pages": num_pages,
                        "spare_page": spare_page})
    if keep_logical:
        offs = np.concatenate([[0], np.cumsum(prefix_lens)]).astype(np.int64)
        wl.prefix_k = [k_tok[offs[i]:offs[i + 1]] for i in range(B)]
        wl.prefix_v = [v_tok[offs[i]:offs[i + 1]] for i in range(B)]
        base = n_prefix_tok
        wl.draft_k = [k_tok[base + branch_qo_indptr[j]: base + branch_qo_indptr[j + 1]] for j in range(NV)]
        wl.draft_v = [v_tok[base + branch_qo_indptr[j]: base + branch_qo_indptr[j + 1]] for j in range(NV)]
    return wl


def attach_random_trees(wl: Workload, seed: int, max_children: int = 4) -> Workload:
    """Turn every branch of ``wl`` into a random draft tree over its S_j nodes:
    nodes are created level by level, each node of a level picking its parent
    uniformly among the previous level's nodes that still have fewer than
    ``max_children`` children (level 0 hangs off the prefix).  Sets
    ``draft_parent`` and ``draft_mask``: one uint64 per row when every S_j <= 64,
    else [rows, W] uint64 words with W = ceil(max S_j / 64) (bit u % 64 of word
    u // 64: node u)."""
    rng = np.random.default_rng(seed)
    R = wl.total_rows
    parent = np.full(R, -1, np.int32)
    qo = wl.branch_qo_indptr
    max_s = int(np.max(np.diff(qo))) if wl.num_branches else 0
    words = max(1, -(-max_s // 64))
    mask = np.zeros((R, words), np.uint64)
    for j in range(wl.num_branches):
        r0, S = int(qo[j]), int(qo[j + 1] - qo[j])
        par = np.full(S, -1, np.int64)
        prev = [-1]                      # level 0: children of the prefix
        nxt: List[int] = []
        kids = {-1: 0}
        u = 0
        while u < S:
            open_ = [p for p in prev if kids.get(p, 0) < (max_children if p >= 0 else max_children)]
            if not open_:
                prev, nxt = nxt, []
                continue
            p = int(open_[rng.integers(len(open_))])
            par[u] = p
            kids[p] = kids.get(p, 0) + 1
            nxt.append(u)
            u += 1
            if rng.random() < 0.35 and nxt:
                prev, nxt = prev + nxt, []
        m = [0] * S                      # ancestor sets as Python integers
        for u in range(S):
            m[u] = (1 << u) | (m[par[u]] if par[u] >= 0 else 0)
        parent[r0:r0 + S] = par
        for u in range(S):
            for w in range(words):
                mask[r0 + u, w] = np.uint64((m[u] >> (64 * w)) & 0xFFFFFFFFFFFFFFFF)
    wl.draft_parent = parent
    wl.draft_mask = mask[:, 0].copy() if words == 1 else mask
    wl.meta["trees"] = {"seed": seed, "max_children": max_children}
    return wl


# ----------------------------------------------------------------------------
# The five workloads the path is measured and checked on.
# ----------------------------------------------------------------------------

def tiny(values: str = "fp32", keep_logical: bool = True, seed: int = 0) -> Workload:
    """B=2, Hq=Hkv=4, d=64, L=32, topk=2 branches x S=3, pages of 16, shuffled."""
    return build_workload("tiny", [32, 32], [[3, 3], [3, 3]], 4, 4, 64, 16, seed,
                          values, keep_logical=keep_logical)


def gqa(values: str = "bf16", keep_logical: bool = False, seed: int = 1) -> Workload:
    """B=8, Hq=32, Hkv=8, d=128, L=1000, topk=4, S=3."""
    return build_workload("gqa", [1000] * 8, [[3] * 4] * 8, 32, 8, 128, 16, seed,
                          values, keep_logical=keep_logical)


def headline(values: str = "bf16", keep_logical: bool = False, seed: int = 2) -> Workload:
    """B=32, Hq=32, Hkv=8, d=128, L=2000, topk=4, S=5 (8020 vs 2020 KV tokens per request)."""
    return build_workload("headline", [2000] * 32, [[5] * 4] * 32, 32, 8, 128, 16, seed,
                          values, keep_logical=keep_logical)


def ragged(values: str = "bf16", keep_logical: bool = False, seed: int = 3,
           batch: int = 64) -> Workload:
    """B=64, L log-uniform in [512, 32768], topk in {2,4,8}, S in {3..8} per request,
    Hq=64, Hkv=8, d=128."""
    rng = np.random.default_rng(seed)
    logL = rng.uniform(math.log(512.0), math.log(32768.0), size=batch)
    L = np.clip(np.rint(np.exp(logL)), 512, 32768).astype(np.int64)
    topk = rng.choice(np.array([2, 4, 8]), size=batch)
    S = rng.integers(3, 9, size=batch)
    branches = [[int(S[i])] * int(topk[i]) for i in range(batch)]
    return build_workload("ragged", L.tolist(), branches, 64, 8, 128, 16, seed,
                          values, keep_logical=keep_logical, rng=rng)


def prefix_hit(h: float, values: str = "bf16", keep_logical: bool = False, seed: int = 4,
               batch: int = 4, n_tokens: int = 8192) -> Workload:
    """B=4 requests of N=8192 tokens whose first H = floor(h*N) are a prefix-cache
    hit; the M = N - H suffix tokens are the queries, causal over prefix + suffix.
    Expressed as one branch of S = M tokens per request whose pages continue the
    prefix pages."""
    H = int(math.floor(h * n_tokens))
    M = n_tokens - H
    wl = build_workload(f"prefix_hit_h{h}", [H] * batch, [[M]] * batch, 32, 8, 128, 16,
                        seed, values, suffix_in_prefix_pages=True,
                        keep_logical=keep_logical)
    wl.meta.update({"N": n_tokens, "H": H, "M": M, "h": h})
    return wl


def tree_headline(values: str = "bf16", keep_logical: bool = False, seed: int = 6) -> Workload:
    """The headline shapes with one 20-node random draft tree per request instead of
    4 chains of 5: B=32, Hq=32, Hkv=8, d=128, L=2000, pages of 16."""
    wl = build_workload("tree_headline", [2000] * 32, [[20]] * 32, 32, 8, 128, 16, seed,
                        values, keep_logical=keep_logical)
    return attach_random_trees(wl, seed + 100)


CONFIGS = {
    "tiny": tiny,
    "gqa": gqa,
    "headline": headline,
    "ragged": ragged,
}


def with_fp8_kv(wl: Workload, headroom: float = 440.0, per_channel: bool = False,
                channel_spread: float = 0.0, seed: int = 0) -> Workload:
    """The same workload with FP8 KV: per-tensor scales amax(|pool|) / headroom
    (rounded to float32) and E4M3 codes of pool / scale, rounded to nearest
    even by torch's float8_e4m3fn cast.  NaN slots (never-written tokens and
    spare pages) stay NaN codes.  headroom < 448 keeps every finite value
    below the largest code, so nothing saturates.

    per_channel: scales per (kv head, channel) instead, the power of two at or
    above amax over that channel / headroom, with the per-tensor scales set to
    1 (powers of two keep the scaled bf16 query exact).  channel_spread > 0 first
    multiplies each channel of the pools by 2^u, u uniform in
    [-channel_spread, 0] (seeded), so that channels differ in range as real K/V
    do (without growing any value past the unscaled pools' range)."""
    import dataclasses

    import torch

    if channel_spread > 0:
        rng = np.random.default_rng(seed)
        Hkv, d = wl.k_pool.shape[2], wl.k_pool.shape[3]
        fk = np.exp2(rng.uniform(-channel_spread, 0.0, (Hkv, d))).astype(np.float32)
        fv = np.exp2(rng.uniform(-channel_spread, 0.0, (Hkv, d))).astype(np.float32)
        wl = dataclasses.replace(wl, k_pool=(wl.k_pool * fk).astype(np.float32),
                                 v_pool=(wl.v_pool * fv).astype(np.float32),
                                 prefix_k=None, prefix_v=None, draft_k=None, draft_v=None)

    def encode(pool, div):
        x = torch.from_numpy(np.ascontiguousarray(pool, np.float32) / div)
        return x.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()

    def tensor_scale(pool):
        fin = np.isfinite(pool)
        amax = float(np.max(np.abs(pool[fin]))) if fin.any() else 1.0
        return float(np.float32(amax / headroom if amax > 0 else 1.0))

    def channel_scales(pool):   # pool [pages, P, Hkv, d] -> [Hkv, d]
        a = np.where(np.isfinite(pool), np.abs(pool), 0.0).max(axis=(0, 1))
        return np.exp2(np.ceil(np.log2(np.where(a > 0, a / headroom, 1.0)))).astype(np.float32)

    if per_channel:
        kcs, vcs = channel_scales(wl.k_pool), channel_scales(wl.v_pool)
        return dataclasses.replace(wl, name=wl.name + "_fp8c", k_codes=encode(wl.k_pool, kcs),
                                   v_codes=encode(wl.v_pool, vcs), k_scale=1.0, v_scale=1.0,
                                   k_channel_scale=kcs, v_channel_scale=vcs)
    ks, vs = tensor_scale(wl.k_pool), tensor_scale(wl.v_pool)
    return dataclasses.replace(wl, name=wl.name + "_fp8", k_codes=encode(wl.k_pool, np.float32(ks)),
                               v_codes=encode(wl.v_pool, np.float32(vs)), k_scale=ks, v_scale=vs)
