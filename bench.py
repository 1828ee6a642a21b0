"""Benchmark of cascade verify attention on one MI355X.

One step = one cascade_verify_attn call (pass A over every request's prefix,
pass B over every branch's drafts, LSE merge) over the whole batch of the
headline workload: B=32 requests, Hq=32, Hkv=8, d=128, prefix L=2000,
topk=4 branches of S=5 draft tokens, 16-token pages in random physical order.
Inputs are synthetic (seeded N(0,1) values rounded to bf16) and resident in
HBM before timing starts.

Protocol: W warm-up steps, then K timed steps.  Before every timed step a
1 GiB buffer is read (outside the timed interval) so that neither L2 nor the
256 MB Infinity Cache still holds the 265 MB of KV.  The flush reads rather
than writes: a freshly written 1 GiB leaves dirty lines whose write-back then
lands inside the next timed kernel.  Each step is timed with HIP events on
the stream it is launched on.  The same protocol times naive expansion (the
baseline) on the same inputs.

Prints one JSON line.  value = KV GB/s = cascade KV bytes / step time, where
cascade KV bytes = sum_i (L_i + sum_j S_j) * Hkv * d * 2 (K and V) * 2 bytes,
and the step time is the event-timed interval around the call.  The roofline
entry uses the kernel's own duration, from a second pass of K cold steps in
which the library records HIP events on the same stream immediately around
its kernel (cascade_kernel_timing), i.e. without the dispatch latency that an
event pair around the call also measures.

The line also carries the same shapes with one 20-node random draft tree per
request (tree attention mask), the ragged configuration against its mixed
roofline, the KV rate as a share of a plain 1 GiB streaming read measured on
the same box, an 8-layer step (draft-KV append + verify per
layer) eager and graph-captured, and the prefix-hit suffix prefill (B=4, N=8192, hit ratio
h = 0, 0.5, 0.9; three calls, cold protocol) beside the closed-form work
ratio 1 - H(H+1)/(N(N+1)), unless --no-prefix-hit.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "cascade verify attn: KV GB/s (% HBM peak) + query tok/s vs naive expand"
CSRC = os.path.join(ROOT, "cascade_attention_tree_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "verify_headline_traffic.json")
MFMA_FILE = os.path.join(ROOT, "profiles", "verify_headline_mfma.json")
BUILD_SCRIPT = os.path.join(ROOT, "cascade_attention_tree_amd", "build_lib.py")


def kernel_source_hash() -> str:
    """Hash of the kernel sources and the build script (its flags shape the
    code): counter records taken under another hash no longer describe the
    kernel and are not reported."""
    h = hashlib.sha256()
    for path in [os.path.join(CSRC, n) for n in sorted(os.listdir(CSRC))] + [BUILD_SCRIPT]:
        with open(path, "rb") as f:
            h.update(os.path.basename(path).encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def profiled(path, key):
    """A value from a counter record under profiles/, if it was taken on the
    current kernel sources; else None."""
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    return rec.get(key) if rec.get("kernel_hash") == kernel_source_hash() else None


def workload_bytes(wl, kv_elem_bytes=2):
    Hkv, d = wl.num_kv_heads, wl.head_dim
    per_tok = Hkv * d * 2 * kv_elem_bytes
    L = wl.cache_seqlens.astype(np.int64)
    S = np.diff(wl.branch_qo_indptr.astype(np.int64))
    req_of = wl.request_of_branch()
    kv_cascade = int((L.sum() + S.sum()) * per_tok)
    kv_naive = int(sum(L[req_of[j]] + S[j] for j in range(S.shape[0])) * per_tok)
    R, Hq = wl.total_rows, wl.num_qo_heads
    q_bytes = R * Hq * d * 2
    o_bytes = R * Hq * d * 2 + R * Hq * 4   # bf16 output + fp32 LSE
    return kv_cascade, kv_naive, q_bytes, o_bytes


def time_steps(fn, steps, warmup, flush, torch):
    """Per-step event times (ms) under the cold protocol, plus the wall time of
    the K timed steps bracketed by device synchronisation."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        flush()
        starts[k].record(stream)
        fn()
        ends[k].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])
    return ms, wall


def time_kernel(fn, steps, flush, B):
    """Kernel durations (ms) of K cold steps, from the events the library
    records around its kernels; each step waits for its stop event."""
    B.cascade_kernel_timing(True)
    try:
        out = []
        for _ in range(steps):
            flush()
            fn()
            out.append(B.cascade_last_verify_ms())
    finally:
        B.cascade_kernel_timing(False)
    return np.array(out)


def time_warm(fn, steps, torch):
    """Back-to-back steps without flushing (context only)."""
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(steps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def cpu_info():
    """Host CPU model (from /proc/cpuinfo) and the number of CPUs this
    process may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return model, n


def _time_oracle(fn, budget_s):
    reps, t0 = 0, time.perf_counter()
    while True:
        fn()
        reps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    return (time.perf_counter() - t0) / reps, reps


def cpu_baseline(wl, kv_bytes, budget_s):
    """The fp64 oracle (pass A, pass B, merge for every row of the headline
    batch) on the host, as it stands: once with numpy's BLAS on every CPU the
    process may use, once limited to one thread, each repeated until
    `budget_s` seconds of work are done."""
    from oracle import cascade_oracle as O
    from threadpoolctl import threadpool_info, threadpool_limits
    model, ncpu = cpu_info()
    blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    dt_all, reps_all = _time_oracle(lambda: O.cascade(wl), budget_s)
    with threadpool_limits(limits=1):
        dt_one, reps_one = _time_oracle(lambda: O.cascade(wl), budget_s)
    sample = (f"full headline batch ({wl.total_rows} rows x {wl.num_qo_heads} heads, all KV), "
              f"{reps_all} repetitions of {dt_all:.2f} s with numpy BLAS on {blas_threads} threads")
    return {"value": kv_bytes / dt_all / 1e9, "unit": "GB/s", "cores": blas_threads, "kind": "oracle",
            "sample": sample, "query_tok_per_s": wl.total_rows / dt_all, "seconds_per_step": dt_all,
            "cpu_model": model, "nproc": ncpu,
            "single_core": {"value": kv_bytes / dt_one / 1e9, "unit": "GB/s", "cores": 1,
                            "query_tok_per_s": wl.total_rows / dt_one, "seconds_per_step": dt_one,
                            "sample": f"same batch, {reps_one} repetitions, BLAS limited to 1 thread"}}


def gqa_timing(B, W, torch, flush, steps, warmup):
    """The GQA verify configuration (B=8, Hq=32, Hkv=8, d=128, L=1000, topk=4,
    S=3, page 16): fused verify, cold protocol, against its HBM roofline
    (KV + Q + output bytes at 8 TB/s)."""
    wl = W.gqa()
    kv_bytes, kv_naive, q_bytes, o_bytes = workload_bytes(wl)
    x = B.to_device(wl, "cuda", layout="HND")
    ws = B.workspace_for(x)
    o = torch.empty(wl.q.shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(wl.q.shape[:2], dtype=torch.float32, device="cuda")

    def verify():
        B.cascade_verify_attn(x, o=o, lse=lse, workspace=ws)

    def naive():
        B.naive_expand(x, o=o, lse=lse)

    ms, _ = time_steps(verify, steps, warmup, flush, torch)
    k_ms = time_kernel(verify, steps, flush, B)
    ms_n, _ = time_steps(naive, steps, warmup, flush, torch)
    t, kt = float(np.median(ms)), float(np.median(k_ms))
    compulsory = kv_bytes + q_bytes + o_bytes
    t_roof = compulsory / (HBM_PEAK_GBS * 1e9)
    out = {"workload": "GQA verify: B=8, Hq=32, Hkv=8, d=128, L=1000, topk=4, S=3, page 16, HND",
           "median_ms": t, "kernel_median_ms": kt, "kernel_mean_ms": float(np.mean(k_ms)),
           "kv_GBps": kv_bytes / (t * 1e-3) / 1e9, "query_tok_per_s": wl.total_rows / (t * 1e-3),
           "roofline_ms": t_roof * 1e3, "roofline_frac_kernel": t_roof / (kt * 1e-3),
           "split_prefix": ws is not None, "naive_median_ms": float(np.median(ms_n)),
           "speedup_vs_naive": float(np.median(ms_n)) / t}
    del x, ws, o, lse
    torch.cuda.empty_cache()
    return out


def layout_timing(B, W, torch, flush, wl, layout, steps, warmup):
    """The headline verify with the pool in another page layout (same logical
    content): event-timed step and the kernel's own time."""
    kv_bytes, _, q_bytes, o_bytes = workload_bytes(wl)
    x = B.to_device(wl, "cuda", layout=layout)
    ws = B.workspace_for(x)
    o = torch.empty(wl.q.shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(wl.q.shape[:2], dtype=torch.float32, device="cuda")

    def verify():
        B.cascade_verify_attn(x, o=o, lse=lse, workspace=ws)

    ms, _ = time_steps(verify, steps, warmup, flush, torch)
    k_ms = time_kernel(verify, steps, flush, B)
    t, kt = float(np.mean(ms)), float(np.mean(k_ms))
    compulsory = kv_bytes + q_bytes + o_bytes
    out = {"page_layout": layout, "ms_per_step": t, "median_ms": float(np.median(ms)),
           "kv_GBps": kv_bytes / (t * 1e-3) / 1e9, "query_tok_per_s": wl.total_rows / (t * 1e-3),
           "kernel_ms": kt, "roofline_frac": compulsory / (kt * 1e-3) / 1e9 / HBM_PEAK_GBS}
    del x, ws, o, lse
    torch.cuda.empty_cache()
    return out


def ragged_timing(B, W, torch, flush, steps=10, warmup=3):
    """The ragged configuration (B=64, L log-uniform in [512, 32768], topk in
    {2,4,8}, S in {3..8}, Hq=64, Hkv=8, d=128): fused verify, cold protocol,
    against the mixed roofline sum_i max(bytes_i / 8 TB/s, flops_i / 2.5 PFLOP/s)
    (bytes_i: request i's prefix and drafts once, K+V bf16; flops_i: 4 d per
    visible (query row, key) pair and query head)."""
    wl = W.ragged()
    kv_bytes, _, q_bytes, o_bytes = workload_bytes(wl)
    Hkv, d, Hq = wl.num_kv_heads, wl.head_dim, wl.num_qo_heads
    rb, qo = wl.req_branch_indptr, wl.branch_qo_indptr
    t_roof = 0.0
    for i in range(wl.batch_size):
        L = int(wl.cache_seqlens[i])
        S = [int(qo[j + 1] - qo[j]) for j in range(int(rb[i]), int(rb[i + 1]))]
        bytes_i = (L + sum(S)) * Hkv * d * 4
        pairs = sum(s_ * L + s_ * (s_ + 1) // 2 for s_ in S)
        flops_i = 4.0 * d * Hq * pairs
        t_roof += max(bytes_i / (HBM_PEAK_GBS * 1e9), flops_i / 2.5e15)
    x = B.to_device(wl, "cuda", layout="HND")
    ws = B.workspace_for(x)
    o = torch.empty(wl.q.shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(wl.q.shape[:2], dtype=torch.float32, device="cuda")

    def verify():
        B.cascade_verify_attn(x, o=o, lse=lse, workspace=ws)

    ms, _ = time_steps(verify, steps, warmup, flush, torch)
    k_ms = time_kernel(verify, steps, flush, B)
    t, kt = float(np.median(ms)), float(np.mean(k_ms))
    out = {"workload": "ragged: B=64, L log-uniform [512, 32768], topk {2,4,8}, S {3..8}, Hq=64, Hkv=8, "
                       "d=128, page 16, HND",
           "total_prefix_tokens": int(wl.cache_seqlens.sum()), "query_rows": wl.total_rows,
           "median_ms": t, "kernel_ms": kt, "kv_GBps": kv_bytes / (t * 1e-3) / 1e9,
           "query_tok_per_s": wl.total_rows / (t * 1e-3),
           "mixed_roofline_ms": t_roof * 1e3, "frac_of_mixed_roofline": t_roof / (kt * 1e-3)}
    del x, ws, o, lse
    torch.cuda.empty_cache()
    return out


def streaming_read_GBps(B, torch, steps=10, nbytes=1 << 30, with_ms=False):
    """A plain streaming read on the same box (the library's reference read
    kernel over an nbytes buffer, 1 GiB by default, another 1 GiB read between
    runs to evict it), median of the event-timed runs (with_ms: also that
    median time in ms)."""
    a = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    b = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    ts = []
    for k in range(steps + 2):
        B.cascade_stream_read(b, sink)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        B.cascade_stream_read(a, sink)
        e1.record()
        torch.cuda.synchronize()
        if k >= 2:
            ts.append(e0.elapsed_time(e1))
    del a, b
    torch.cuda.empty_cache()
    t = float(np.median(ts))
    gbs = nbytes / (t * 1e-3) / 1e9
    return (gbs, t) if with_ms else gbs


def graph_step_timing(B, torch, flush, wl, x0, n_layers=8, steps=10, warmup=3):
    """A multi-layer verify step at the headline shapes: for each of n_layers
    layers (own K/V pools, same tables) the drafts' K/V are appended into their
    pages, then the fused verify runs.  Timed eagerly and as one captured HIP
    graph (torch.cuda.CUDAGraph), cold protocol per step."""
    import copy
    layers = [x0]
    for _ in range(n_layers - 1):
        x = copy.copy(x0)
        x.k_pool, x.v_pool = x0.k_pool.clone(), x0.v_pool.clone()
        kv = x0.kv
        x.kv = B.PagedKV(x.k_pool.data_ptr(), x.v_pool.data_ptr(), kv.num_pages, kv.page_size,
                         kv.num_kv_heads, kv.head_dim, kv.page_stride, kv.token_stride, kv.head_stride)
        layers.append(x)
    wss = [B.workspace_for(x) for x in layers]
    gen = torch.Generator(device="cuda").manual_seed(5)
    shape = (wl.total_rows, wl.num_kv_heads, wl.head_dim)
    drafts = [(torch.randn(shape, generator=gen, device="cuda").to(torch.bfloat16),
               torch.randn(shape, generator=gen, device="cuda").to(torch.bfloat16)) for _ in layers]
    outs = [torch.empty(wl.q.shape, dtype=torch.bfloat16, device="cuda") for _ in layers]
    lses = [torch.empty(wl.q.shape[:2], dtype=torch.float32, device="cuda") for _ in layers]

    def step():
        for x, (k, v), o, l, ws in zip(layers, drafts, outs, lses, wss):
            B.cascade_append_draft_kv(x, k, v)
            B.cascade_verify_attn(x, o=o, lse=l, workspace=ws)

    ms_e, _ = time_steps(step, steps, warmup, flush, torch)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    ms_g, _ = time_steps(g.replay, steps, warmup, flush, torch)
    te, tg = float(np.median(ms_e)), float(np.median(ms_g))
    return {"layers": n_layers, "eager_ms_per_step": te, "graph_ms_per_step": tg,
            "graph_ms_per_layer": tg / n_layers,
            "workload": "headline shapes per layer; per layer: append the 640 drafts' K/V into their "
                        "pages, then the fused verify"}


def draft_tree_timing(B, W, torch, flush, steps, warmup):
    """The headline shapes with one 20-node random draft tree per request (tree
    attention mask) instead of 4 chains of 5: fused verify, cold protocol."""
    wl = W.tree_headline()
    kv_bytes, _, q_bytes, o_bytes = workload_bytes(wl)
    x = B.to_device(wl, "cuda", layout="HND")
    ws = B.workspace_for(x)
    o = torch.empty(wl.q.shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(wl.q.shape[:2], dtype=torch.float32, device="cuda")

    def verify():
        B.cascade_verify_attn(x, o=o, lse=lse, workspace=ws)

    ms, _ = time_steps(verify, steps, warmup, flush, torch)
    k_ms = time_kernel(verify, steps, flush, B)
    t, kt = float(np.mean(ms)), float(np.mean(k_ms))
    return {"workload": "B=32, Hq=32, Hkv=8, d=128, L=2000, one 20-node draft tree per request, "
                        "page 16, HND",
            "ms_per_step": t, "kv_GBps": kv_bytes / (t * 1e-3) / 1e9,
            "query_tok_per_s": wl.total_rows / (t * 1e-3), "kernel_ms": kt,
            "roofline_frac": (kv_bytes + q_bytes + o_bytes) / (kt * 1e-3) / 1e9 / HBM_PEAK_GBS}


def fp8_timing(B, W, torch, flush, wl_bf16, t_bf16_ms, steps, warmup, layout):
    """The headline workload with FP8 E4M3 KV (per-tensor scales): fused
    verify and naive expansion, cold protocol, plus the verify kernel's own
    time against its roofline (KV bytes halve; Q and the output do not)."""
    wl = W.with_fp8_kv(wl_bf16)
    kv_bytes, kv_naive, q_bytes, o_bytes = workload_bytes(wl, kv_elem_bytes=1)
    x = B.to_device(wl, "cuda", layout=layout)
    ws = B.workspace_for(x)
    o = torch.empty(wl.q.shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(wl.q.shape[:2], dtype=torch.float32, device="cuda")

    def verify():
        B.cascade_verify_attn(x, o=o, lse=lse, workspace=ws)

    def naive():
        B.naive_expand(x, o=o, lse=lse)

    ms, _ = time_steps(verify, steps, warmup, flush, torch)
    k_ms = time_kernel(verify, steps, flush, B)
    ms_n, _ = time_steps(naive, steps, warmup, flush, torch)
    t, kt, tn = float(np.mean(ms)), float(np.mean(k_ms)), float(np.mean(ms_n))
    compulsory = kv_bytes + q_bytes + o_bytes
    return {"workload": "headline shapes, K/V as FP8 E4M3 codes with per-tensor scales, "
                        f"page 16, {layout}",
            "ms_per_step": t, "median_ms": float(np.median(ms)), "kv_bytes": kv_bytes,
            "kv_GBps": kv_bytes / (t * 1e-3) / 1e9,
            "query_tok_per_s": wl.total_rows / (t * 1e-3),
            "kernel_ms": kt, "kernel_median_ms": float(np.median(k_ms)),
            "roofline_frac": compulsory / (kt * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "algorithmic_bytes_per_launch": compulsory,
            "speedup_vs_bf16_verify": t_bf16_ms / t,
            "naive_ms": tn, "speedup_vs_naive_fp8": tn / t}


def prefix_hit_timings(B, W, torch, flush, steps=5, warmup=2):
    """Prefix-hit suffix prefill (B=4 requests of N=8192 tokens, a hit of
    H = floor(h N)): pass A over the hit, pass B causal over the suffix, merge
    (three calls), cold protocol; and the same split and merge as one fused
    verify launch (`fused_*`).  Reported beside the closed-form work ratio
    1 - H(H+1)/(N(N+1)) and against the dense bf16 MFMA peak (2.5 PFLOP/s)."""
    out = {}
    base = None
    for h in (0.0, 0.5, 0.9):
        wl = W.prefix_hit(h)
        N, H, M = wl.meta["N"], wl.meta["H"], wl.meta["M"]
        x = B.to_device(wl, "cuda", layout="HND")
        ws = B.workspace_for(x)
        oa = torch.empty(wl.q.shape, dtype=torch.float32, device="cuda")
        la = torch.empty(wl.q.shape[:2], dtype=torch.float32, device="cuda")
        ob, lb = torch.empty_like(oa), torch.empty_like(la)
        o = torch.empty(wl.q.shape, dtype=torch.bfloat16, device="cuda")
        lse = torch.empty_like(la)

        def step():
            B.cascade_prefix_attn(x, o_a=oa, lse_a=la, workspace=ws)
            B.cascade_draft_attn(x, o_b=ob, lse_b=lb)
            B.merge_state(oa, la, ob, lb, out_dtype=torch.bfloat16, o=o, lse=lse)

        def fused():
            B.cascade_verify_attn(x, o=o, lse=lse, workspace=ws)

        ms, _ = time_steps(step, steps, warmup, flush, torch)
        ms_f, _ = time_steps(fused, steps, warmup, flush, torch)
        t = float(np.median(ms))
        t_f = float(np.median(ms_f))
        base = t if base is None else base
        pairs = wl.batch_size * (M * H + M * (M + 1) // 2)           # visible (query, key) pairs per head
        flops = 4.0 * wl.head_dim * wl.num_qo_heads * pairs
        out[f"h{h}"] = {"H": H, "M": M, "median_ms": t, "tflops": flops / (t * 1e-3) / 1e12,
                        "mfma_frac": flops / (t * 1e-3) / 2.5e15,
                        "time_ratio_vs_h0": t / base,
                        "work_ratio_closed_form": 1.0 - H * (H + 1) / (N * (N + 1)),
                        "fused_median_ms": t_f, "fused_tflops": flops / (t_f * 1e-3) / 1e12}
        del x, ws, oa, la, ob, lb, o, lse
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--only-verify", action="store_true", help="time only the fused verify call")
    ap.add_argument("--layout", choices=("HND", "NHD"), default="HND",
                    help="page layout of the KV pool on the device (same logical content)")
    ap.add_argument("--no-ragged", action="store_true",
                    help="skip the ragged configuration")
    ap.add_argument("--no-graph-step", action="store_true",
                    help="skip the multi-layer graph-captured step")
    ap.add_argument("--no-draft-tree", action="store_true",
                    help="skip the draft-tree variant of the headline shapes")
    ap.add_argument("--no-prefix-hit", action="store_true",
                    help="skip the prefix-hit (suffix prefill) timings")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the FP8 KV variant of the headline")
    ap.add_argument("--fp8-only", action="store_true",
                    help="for profiling: only the FP8 headline verify (cold steps)")
    ap.add_argument("--gqa-only", action="store_true",
                    help="for profiling: only the GQA verify configuration (cold steps)")
    ap.add_argument("--ragged-only", action="store_true",
                    help="for profiling: only the ragged configuration (cold steps)")
    ap.add_argument("--prefix-hit-only", action="store_true",
                    help="for profiling: only the prefix-hit suffix prefill (cold steps)")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="for hardware-counter runs: one plain 256 MiB device copy (known bytes), "
                         "then a few flushed verify steps and naive-expand steps; prints nothing else")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
              "the path runs on a single MI355X here and has no multi-GPU leg.", file=sys.stderr)
        sys.exit(2)

    import torch
    from cascade_attention_tree_amd import binding as B
    from cascade_attention_tree_amd import workload as W

    flush_buf = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    flush_out = torch.empty((), dtype=torch.float32, device="cuda")

    def flush():
        torch.sum(flush_buf, dim=0, out=flush_out)   # reads 1 GiB, writes 4 bytes

    if args.gqa_only or args.ragged_only or args.prefix_hit_only:
        print("bench: profiling leg only", file=sys.stderr, flush=True)
        if args.gqa_only:
            leg, out = "gqa", gqa_timing(B, W, torch, flush, args.steps, args.warmup)
        elif args.ragged_only:
            leg, out = "ragged", ragged_timing(B, W, torch, flush, steps=args.steps, warmup=args.warmup)
        else:
            leg, out = "prefix_hit", prefix_hit_timings(B, W, torch, flush, steps=args.steps, warmup=args.warmup)
        print(json.dumps({"profiling_leg": leg, **out, "kernel_hash": kernel_source_hash()}), flush=True)
        return

    print("bench: generating headline workload", file=sys.stderr, flush=True)
    wl = W.headline()
    kv_casc, kv_naive, q_bytes, o_bytes = workload_bytes(wl)
    x = B.to_device(wl, "cuda", layout=args.layout)
    o = torch.empty(wl.q.shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(wl.q.shape[:2], dtype=torch.float32, device="cuda")
    ws = B.workspace_for(x)

    def verify():
        B.cascade_verify_attn(x, o=o, lse=lse, workspace=ws)

    def naive():
        B.naive_expand(x, o=o, lse=lse)

    oa = torch.empty(wl.q.shape, dtype=torch.float32, device="cuda")
    la = torch.empty(wl.q.shape[:2], dtype=torch.float32, device="cuda")
    ob, lb = torch.empty_like(oa), torch.empty_like(la)

    def three_call():
        B.cascade_prefix_attn(x, o_a=oa, lse_a=la, workspace=ws)
        B.cascade_draft_attn(x, o_b=ob, lse_b=lb)
        B.merge_state(oa, la, ob, lb, out_dtype=torch.bfloat16, o=o, lse=lse)

    if args.fp8_only:
        wl8 = W.with_fp8_kv(wl)
        x8 = B.to_device(wl8, "cuda", layout=args.layout)
        ws8 = B.workspace_for(x8)
        del x
        print("bench: FP8 headline verify only", file=sys.stderr, flush=True)
        if args.traffic_probe:
            src = torch.ones(1 << 26, dtype=torch.float32, device="cuda")   # 256 MiB
            dst = torch.empty_like(src)
            flush()
            dst.copy_(src)
        ms, _ = time_steps(lambda: B.cascade_verify_attn(x8, o=o, lse=lse, workspace=ws8),
                           args.steps, args.warmup, flush, torch)
        print(json.dumps({"fp8_only": True, "ms_per_step": float(np.mean(ms)),
                          "kernel_hash": kernel_source_hash()}), flush=True)
        return

    if args.traffic_probe:
        src = torch.ones(1 << 26, dtype=torch.float32, device="cuda")   # 256 MiB
        dst = torch.empty_like(src)
        flush()
        dst.copy_(src)
        for _ in range(3):
            flush()
            verify()
        for _ in range(3):
            flush()
            naive()
        torch.cuda.synchronize()
        print(json.dumps({"traffic_probe": True, "copy_bytes": src.numel() * 4,
                          "kernel_hash": kernel_source_hash()}), flush=True)
        return

    print("bench: timing cascade_verify_attn", file=sys.stderr, flush=True)
    ms, wall = time_steps(verify, args.steps, args.warmup, flush, torch)
    t_ms = float(np.mean(ms))
    print("bench: timing the verify kernel (events around the kernel)", file=sys.stderr, flush=True)
    k_ms = time_kernel(verify, args.steps, flush, B)
    kernel_ms = float(np.mean(k_ms))
    warm_ms = time_warm(verify, args.steps, torch)
    extra = {}
    if not args.only_verify:
        print("bench: timing naive_expand", file=sys.stderr, flush=True)
        ms_n, _ = time_steps(naive, args.steps, args.warmup, flush, torch)
        print("bench: timing prefix + draft + merge (three calls)", file=sys.stderr, flush=True)
        ms_3, _ = time_steps(three_call, args.steps, args.warmup, flush, torch)
        t_naive = float(np.mean(ms_n))
        extra = {
            "naive": {"ms": t_naive, "median_ms": float(np.median(ms_n)),
                      "kv_GBps_algorithmic": kv_naive / (t_naive * 1e-3) / 1e9,
                      "kv_bytes": kv_naive},
            "speedup_vs_naive": t_naive / t_ms,
            "three_call_ms": float(np.mean(ms_3)),
        }
    kv_gbs = kv_casc / (t_ms * 1e-3) / 1e9
    compulsory = kv_casc + q_bytes + o_bytes
    traffic = profiled(TRAFFIC_FILE, "bytes_per_launch")
    line = {
        "metric": METRIC,
        "value": kv_gbs,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": t_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "headline verify: B=32, Hq=32, Hkv=8, d=128, L=2000, topk=4, S=5, "
                               "page 16, random page table, bf16 in, bf16 out",
                   "page_layout": args.layout,
                   "global_batch": wl.batch_size, "query_tokens": wl.total_rows,
                   "kv_bytes_cascade": kv_casc, "protocol": "cold (1 GiB read between steps)"},
        "pct_hbm_peak": 100.0 * kv_gbs / HBM_PEAK_GBS,
        "query_tok_per_s": wl.total_rows / (t_ms * 1e-3),
        "median_ms": float(np.median(ms)), "p10_ms": float(np.percentile(ms, 10)),
        "p90_ms": float(np.percentile(ms, 90)),
        "warm_ms_per_step": warm_ms,
        "wall_s_timed_region": wall,
        "roofline": {"bound": "hbm", "achieved": compulsory / (kernel_ms * 1e-3) / 1e9,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": compulsory / (kernel_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "traffic": traffic,
                     "kernel": "attn_kernel<128, 5, verify> (key-split kernel, one launch per step)",
                     "algorithmic_bytes_per_launch": compulsory,
                     "kernel_ms": kernel_ms, "kernel_median_ms": float(np.median(k_ms)),
                     "kernel_timing": "HIP events recorded around the kernel launch "
                                      "(hipExtLaunchKernel), mean of K cold steps",
                     "mfma_util_profiled": profiled(MFMA_FILE, "mfma_busy_frac")},
    }
    line.update(extra)
    if not args.only_verify:
        sr = streaming_read_GBps(B, torch)
        line["streaming_read_GBps"] = sr
        line["pct_streaming_read"] = 100.0 * kv_gbs / sr
        # The same read over exactly the step's algorithmic bytes, timed like
        # the step (events around the call): what one launch that only reads
        # those bytes costs on this machine.
        gbs, t_read = streaming_read_GBps(B, torch, nbytes=compulsory, with_ms=True)
        line["same_size_read"] = {"bytes": compulsory, "ms": t_read, "GBps": gbs,
                                  "step_over_read": float(np.median(ms)) / t_read}
    if not args.only_verify:
        other = "NHD" if args.layout == "HND" else "HND"
        print(f"bench: timing the headline verify with {other} pages", file=sys.stderr, flush=True)
        line["other_layout"] = layout_timing(B, W, torch, flush, wl, other, args.steps, args.warmup)
        print("bench: timing the GQA verify configuration", file=sys.stderr, flush=True)
        line["gqa"] = gqa_timing(B, W, torch, flush, args.steps, args.warmup)
    if not args.no_ragged and not args.only_verify:
        print("bench: timing the ragged configuration", file=sys.stderr, flush=True)
        line["ragged"] = ragged_timing(B, W, torch, flush)
    if not args.no_graph_step and not args.only_verify:
        print("bench: timing an 8-layer step (append + verify per layer), eager and graph",
              file=sys.stderr, flush=True)
        line["graph_step"] = graph_step_timing(B, torch, flush, wl, x)
    if not args.no_draft_tree and not args.only_verify:
        print("bench: timing the draft-tree variant", file=sys.stderr, flush=True)
        line["draft_tree"] = draft_tree_timing(B, W, torch, flush, args.steps, args.warmup)
    if not args.no_fp8 and not args.only_verify:
        print("bench: timing the FP8 KV variant", file=sys.stderr, flush=True)
        line["fp8_kv"] = fp8_timing(B, W, torch, flush, wl, t_ms, args.steps, args.warmup, args.layout)
    if not args.no_prefix_hit and not args.only_verify:
        print("bench: timing prefix-hit suffix prefill (h = 0, 0.5, 0.9)", file=sys.stderr, flush=True)
        line["prefix_hit"] = prefix_hit_timings(B, W, torch, flush)
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(wl, kv_casc, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
