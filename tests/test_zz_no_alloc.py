"""GPU: the allocation-free verify entry point (cascade_verify_attn_noalloc)
against cascade_verify_attn with a caller workspace.

Two calls in a row on one GPU, the second with a smaller input, both with a
split prefix so that the built-in workspace carries the partial states; the
outputs must equal those of the caller-workspace entry point bit for bit (the
same kernels over the same partials), and match the oracle.  Shapes that need
more workspace than the built-in array holds are refused before any launch.
"""

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


def _check_against_workspace_call(B, wl, out_dtype):
    x = B.to_device(wl, layout="HND")
    assert B.cascade_workspace_size(x) > 0, "the case is meant to split its prefix"
    note(f"noalloc {wl.name} rows={wl.total_rows} ws={B.cascade_workspace_size(x)}")
    o_n, l_n = B.cascade_verify_attn_noalloc(x, out_dtype=out_dtype)
    o_w, l_w = B.cascade_verify_attn(x, out_dtype=out_dtype, workspace=B.workspace_for(x))
    torch.cuda.synchronize()
    assert torch.equal(o_n, o_w) and torch.equal(l_n, l_w)
    ro, rl = O.cascade(wl)
    o = o_n.float().cpu().numpy().astype(np.float64)
    l = l_n.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(o - ro)) <= 1e-2
    fin = np.isfinite(rl)
    assert np.max(np.abs(l[fin] - rl[fin])) <= 1e-3
    assert np.array_equal(np.isneginf(l), np.isneginf(rl))


def test_noalloc_matches_workspace_entry_point(B):
    # the GQA verify shapes with a 5000-token prefix (split over workgroups),
    # a row-split launch (960 rows per kv head; split prefix and its work list
    # in the built-in workspace), then a smaller split case on the same GPU
    _check_against_workspace_call(
        B, W.build_workload("long_gqa", [5000] * 8, [[3] * 4] * 8, 32, 8, 128, 16, seed=93), torch.float32)
    _check_against_workspace_call(
        B, W.build_workload("rows_noalloc", [6000, 1500], [[40] * 3, [20] * 2], 16, 2, 128, 16, seed=94),
        torch.bfloat16)
    _check_against_workspace_call(
        B, W.build_workload("small_split", [2200, 600], [[3, 2], [4]], 8, 2, 128, 16, seed=91), torch.bfloat16)
    assert B.cascade_device_error(clear=True) == 0


def test_noalloc_refuses_oversized_workspace(B):
    # 2 requests x 120000-token prefixes: the split partials exceed 32 MiB
    wl = W.build_workload("huge", [1, 1], [[64] * 16, [64] * 16], 32, 8, 128, 16, seed=92)
    x = B.to_device(wl)
    x.tree.max_prefix_len = 120000
    x.tree.page_table_stride = 120000 // 16
    need = B.cascade_workspace_size(x)
    assert need > 32 << 20
    with pytest.raises(RuntimeError, match="workspace"):
        B.cascade_verify_attn_noalloc(x)
