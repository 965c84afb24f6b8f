"""The allocation-free entry point, moe_ffn_forward_noalloc, through the C ABI:
its output equals moe_ffn_forward's on the same inputs bitwise (same
kernels, deterministic), on calls in a row with the later ones smaller, at
the tiny and the full shape, under HIP graph capture, and at its size limit.
Needs an MI355X; run with ``-m gpu``."""

from __future__ import annotations

import numpy as np
import pytest

from mixture_experts_ffn_rmsnorm_amd import inputs as gen
from mixture_experts_ffn_rmsnorm_amd import moe
from oracle import moe_ref as ref
from tests.gpu_common import Layer, check_output

pytestmark = [pytest.mark.gpu]

SCORE, HASH = ref.LAYER_SCORE, ref.LAYER_HASH


def _dev(a):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _both(lay, x_np, tok_np, kind):
    """(no-alloc output, workspace-entry output) for the same inputs; the
    workspace call gets a fresh zero-filled workspace."""
    import torch

    x = _dev(x_np.astype(np.float32))
    tok = _dev(tok_np.astype(np.int32)) if tok_np is not None else None
    out_n = torch.full_like(x, float("nan"))
    out_w = torch.full_like(x, float("nan"))
    moe.forward_noalloc(lay.dims, x, tok, kind, lay.cw, out_n)
    torch.cuda.synchronize()
    got = out_n.cpu().numpy()
    moe.forward(lay.dims, x, tok, kind, lay.cw, out_w, moe.alloc_workspace(lay.dims, x.shape[0]))
    torch.cuda.synchronize()
    return got, out_w.cpu().numpy()


def _rows(cfg, rows, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((rows, cfg.hidden)).astype(np.float32),
            rng.integers(0, max(cfg.table_rows, 1), rows).astype(np.int32))


@pytest.fixture(scope="module")
def tiny():
    return Layer(gen.config(0))


def test_noalloc_equals_workspace_entry_tiny(tiny):
    """Calls in a row, each smaller than the one before: prefill (300 and 37
    rows), the two-to-four-row path (3), the one-row path (1); score and
    hash layers.  Also within the bar of the oracle."""
    cfg = tiny.cfg
    for i, (rows, kind) in enumerate(((300, SCORE), (37, HASH), (3, HASH), (3, SCORE), (1, SCORE))):
        x, tok = _rows(cfg, rows, 200 + i)
        got, want = _both(tiny, x, tok, kind)
        assert np.array_equal(got, want), f"rows={rows} kind={kind}: differs from moe_ffn_forward"
        oracle = ref.forward(x, tok, kind, tiny.oracle_w, cfg.top_k, cfg.eps)["out"]
        check_output(got, oracle, what=f"no-alloc rows={rows}")


def test_noalloc_equals_workspace_entry_full():
    """Full shape: the largest call the scratch holds (696 rows), then the
    512-row prefill workload, the 4-row hash cohort and one row."""
    full = Layer(gen.config(1))
    cohort = Layer(gen.config(2), share=full)
    h3 = gen.host_inputs(gen.config(3))
    h2 = cohort.host
    x696, _ = _rows(full.cfg, 696, 210)
    cases = [(full, x696, None, SCORE), (full, h3.x, None, SCORE), (cohort, h2.x, h2.token_ids, HASH),
             (full, full.host.x, None, SCORE)]
    for lay, x, tok, kind in cases:
        got, want = _both(lay, x, tok, kind)
        assert np.array_equal(got, want), f"rows={x.shape[0]}: differs from moe_ffn_forward"
    # the one-row result against the oracle as well
    oracle = ref.forward(full.host.x, None, SCORE, full.oracle_w, 6, full.cfg.eps)["out"]
    check_output(got, oracle, rel=1e-5, maxabs=5e-5, what="no-alloc one row")


def test_noalloc_size_limit(tiny):
    """One row past the scratch's capacity is rejected with MOE_ESCRATCH
    before anything is enqueued; the workspace entry point still takes it."""
    import torch

    cfg = gen.config(1)
    dims = moe.dims_of(cfg)
    assert moe.workspace_bytes(dims, 696) <= moe.NOALLOC_SCRATCH_BYTES < moe.workspace_bytes(dims, 697)
    x = torch.zeros((697, cfg.hidden), dtype=torch.float32, device="cuda")
    out = torch.empty_like(x)
    with pytest.raises(moe.MoeError) as e:
        moe.forward_noalloc(dims, x, None, SCORE, tiny.cw, out)
    assert e.value.code == moe.MOE_ESCRATCH


def test_noalloc_under_graph_capture(tiny):
    """The callers it is for: two chained 4-row hash calls captured in one
    graph (no allocation inside the capture), replayed with new inputs, each
    replay equal to eager moe_ffn_forward calls bitwise."""
    import torch

    cfg = tiny.cfg
    lay1 = Layer(cfg, layer=1)
    rows = 4
    x = torch.empty((rows, cfg.hidden), dtype=torch.float32, device="cuda")
    tok = torch.zeros(rows, dtype=torch.int32, device="cuda")
    mid, out = torch.empty_like(x), torch.empty_like(x)

    def chain():
        moe.forward_noalloc(tiny.dims, x, tok, HASH, tiny.cw, mid)
        moe.forward_noalloc(lay1.dims, mid, tok, HASH, lay1.cw, out)

    xs, ts = _rows(cfg, rows, 220)
    x.copy_(_dev(xs))
    tok.copy_(_dev(ts))
    chain()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        chain()
    torch.cuda.synchronize()
    for i in range(3):
        xs, ts = _rows(cfg, rows, 221 + i)
        x.copy_(_dev(xs))
        tok.copy_(_dev(ts))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        e_mid, e_out = torch.empty_like(x), torch.empty_like(x)
        moe.forward(tiny.dims, x, tok, HASH, tiny.cw, e_mid, moe.alloc_workspace(tiny.dims, rows))
        moe.forward(lay1.dims, e_mid, tok, HASH, lay1.cw, e_out, moe.alloc_workspace(lay1.dims, rows))
        torch.cuda.synchronize()
        assert np.array_equal(got, e_out.cpu().numpy()), f"replay {i}: differs from eager calls"
