"""The forward under HIP graph capture (the ABI's enqueue-only contract): one
forward captured once and replayed, with new inputs written into the
captured buffers between replays, equals the eager forward of the same
inputs on every replay, bitwise.  Between replays the test runs eager work
of its own (an eager forward on another workspace) and synchronises."""

from __future__ import annotations

import numpy as np
import pytest

from mixture_experts_ffn_rmsnorm_amd import inputs as gen
from mixture_experts_ffn_rmsnorm_amd import moe
from oracle import moe_ref as ref
from tests.gpu_common import Layer

pytestmark = [pytest.mark.gpu]


@pytest.fixture(scope="module")
def full():
    return Layer(gen.config(1))


def _replay_matches_eager(layer, rows, kind, tok=None, seeds=(11, 12, 13, 14)):
    import torch

    cfg = layer.cfg
    x = torch.empty((rows, cfg.hidden), dtype=torch.float32, device="cuda")
    out = torch.empty_like(x)
    ws = moe.alloc_workspace(layer.dims, rows)
    tk = None if tok is None else torch.from_numpy(np.ascontiguousarray(tok, dtype=np.int32)).cuda()
    ref_out = torch.empty_like(x)
    ws_eager = moe.alloc_workspace(layer.dims, rows)

    def fill(seed):
        v = np.random.default_rng(seed).standard_normal((rows, cfg.hidden)).astype(np.float32)
        x.copy_(torch.from_numpy(v))

    fill(seeds[0])
    moe.forward(layer.dims, x, tk, kind, layer.cw, out, ws)  # warm-up outside the graph
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.forward(layer.dims, x, tk, kind, layer.cw, out, ws)
    torch.cuda.synchronize()
    for seed in seeds:
        fill(seed)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        moe.forward(layer.dims, x, tk, kind, layer.cw, ref_out, ws_eager)
        torch.cuda.synchronize()
        assert torch.equal(got, ref_out), f"rows={rows} seed={seed}: graph replay differs from the eager forward"
        assert moe.status(ws) == 0


def test_graph_decode_score(full):
    _replay_matches_eager(full, 1, ref.LAYER_SCORE)


def test_graph_decode_cohort_hash(full):
    cfg = gen.config(2)
    lay = Layer(cfg, share=full)
    _replay_matches_eager(lay, 4, ref.LAYER_HASH, tok=lay.host.token_ids)


def test_graph_prefill_score(full):
    _replay_matches_eager(full, 300, ref.LAYER_SCORE, seeds=(21, 22, 23))


def _chain_on_one_workspace(lays, rows, kind, seeds, rel, maxabs):
    """The layers chained (layer l+1 reads layer l's output) and captured
    once in one graph, every call on ONE workspace; replayed with new x and
    token ids each time, with an eager call of the same row count on the
    same workspace between replays.  Each replay's outputs are checked
    against the oracle layer by layer (layer l+1 against the oracle fed the
    GPU's layer-l output), and bitwise against eager calls on fresh
    workspaces."""
    import torch

    from tests.gpu_common import check_output

    cfg = lays[0].cfg
    H, K, L = cfg.hidden, cfg.top_k, len(lays)
    x = torch.empty((rows, H), dtype=torch.float32, device="cuda")
    outs = [torch.empty_like(x) for _ in lays]
    tok = torch.zeros(rows, dtype=torch.int32, device="cuda")
    ws = moe.alloc_workspace(lays[0].dims, rows)
    x2, out2 = torch.empty_like(x), torch.empty_like(x)

    def chain():
        src = x
        for lay, dst in zip(lays, outs):
            moe.forward(lay.dims, src, tok, kind, lay.cw, dst, ws)
            src = dst

    rng = np.random.default_rng(seeds[0])

    def fill(dst_x):
        v = rng.standard_normal((rows, H)).astype(np.float32)
        t = rng.integers(0, max(cfg.table_rows, 1), rows).astype(np.int32)  # unused by score layers
        dst_x.copy_(torch.from_numpy(v))
        tok.copy_(torch.from_numpy(t))
        return v, t

    fill(x)
    chain()  # outside the graph first
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        chain()
    torch.cuda.synchronize()
    for i, _ in enumerate(seeds):
        xv, tv = fill(x)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [o.cpu().numpy() for o in outs]
        assert moe.status(ws) == 0
        # the oracle, layer by layer
        src = xv
        for l, lay in enumerate(lays):
            want = ref.forward(src, tv, kind, lay.oracle_w, K, cfg.eps)["out"]
            check_output(got[l], want, rel, maxabs, what=f"replay {i} layer {l}")
            src = got[l]
        # bitwise against eager calls on fresh workspaces
        src = x
        for l, lay in enumerate(lays):
            e = torch.empty_like(x)
            moe.forward(lay.dims, src, tok, kind, lay.cw, e, moe.alloc_workspace(lay.dims, rows))
            torch.cuda.synchronize()
            assert np.array_equal(e.cpu().numpy(), got[l]), \
                f"replay {i} layer {l}: differs from eager calls on fresh workspaces"
            src = e
        # an eager call on the shared workspace between replays
        x2v, t2v = xv[::-1].copy(), tv[::-1].copy()
        x2.copy_(torch.from_numpy(x2v))
        tok.copy_(torch.from_numpy(t2v))
        moe.forward(lays[-1].dims, x2, tok, kind, lays[-1].cw, out2, ws)
        torch.cuda.synchronize()
        want2 = ref.forward(x2v, t2v, kind, lays[-1].oracle_w, K, cfg.eps)["out"]
        check_output(out2.cpu().numpy(), want2, rel, maxabs, what=f"eager call after replay {i}")


def test_graph_two_layers_one_workspace_tiny():
    cfg = gen.config(0)
    lay0, lay1 = Layer(cfg, layer=0), Layer(cfg, layer=1)
    for rows in (2, 4):
        _chain_on_one_workspace([lay0, lay1], rows, ref.LAYER_HASH, (61, 62, 63, 64), 1e-5, 5e-5)


def test_graph_two_layers_one_workspace_full(full):
    """The decode cohort's shape: two consecutive 4-row hash layers with
    different weights, one workspace."""
    cfg = gen.config(2)
    lay0 = Layer(cfg, share=full)
    lay1 = Layer(cfg, layer=1)
    _chain_on_one_workspace([lay0, lay1], 4, ref.LAYER_HASH, (71, 72, 73), 1e-5, 5e-5)


def test_graph_decode_four_layer_chain_one_row_full(full):
    """The one-row decode pipeline: four consecutive score layers with
    distinct weights, one workspace, one graph -- the pattern of a model's
    decode step over its layers."""
    cfg = gen.config(1)
    lays = [full] + [Layer(cfg, layer=l) for l in (1, 2, 3)]
    _chain_on_one_workspace(lays, 1, ref.LAYER_SCORE, (81, 82), 1e-5, 5e-5)


def test_graph_decode_three_layer_chain_tiny_all_row_counts():
    """Chains of three tiny score layers at every decode row count: one row
    (the one-row path) and two to four (the counted-in routing), each chain
    on one workspace."""
    cfg = gen.config(0)
    lays = [Layer(cfg, layer=l) for l in (0, 1, 2)]
    for rows in (1, 2, 3, 4):
        _chain_on_one_workspace(lays, rows, ref.LAYER_SCORE, (90 + rows, 95 + rows), 1e-5, 5e-5)
