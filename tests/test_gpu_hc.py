"""The hyper-connection-wrapped layer (moe_ffn_forward_hc) through the C ABI
against the float64 oracle (oracle/hc_ref.py) on the same seeded inputs:
each step on its own -- mixes, maps, FFN input, the FFN on the GPU's own
input, the new state from the GPU's own FFN output and maps -- then end to
end.  The split / pre / post arithmetic is the oracle's stated reading
(parity unpinned beyond it).  Needs an MI355X; run with ``-m gpu``."""

from __future__ import annotations

import numpy as np
import pytest

from mixture_experts_ffn_rmsnorm_amd import inputs as gen
from mixture_experts_ffn_rmsnorm_amd import moe
from oracle import hc_ref as hcr
from oracle import moe_ref as ref
from tests.gpu_common import Layer, check_forward, check_output

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]

SCORE, HASH = ref.LAYER_SCORE, ref.LAYER_HASH


class HcLayer:
    """An FFN layer plus the wrapper's parameters, on the device and in the
    oracle."""

    def __init__(self, lay: Layer, hc: int, rows: int):
        import torch

        self.lay, self.cfg, self.hc = lay, lay.cfg, hc
        self.host = gen.hc_inputs(lay.cfg, hc, rows=rows)
        h = self.host
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        self.fn = t(h.hc_fn.view(np.int16)).view(torch.bfloat16)
        self.scale, self.base = t(h.hc_scale), t(h.hc_base)
        self.hw = moe.make_hc_weights(self.fn, self.scale, self.base, hc, h.iters)
        self.oracle_hw = hcr.HcWeights(h.hc_fn, h.hc_scale, h.hc_base, hc, h.iters)

    def run(self, state_np, tok_np, kind, ws=None):
        import torch

        R = state_np.shape[0]
        st = torch.from_numpy(np.ascontiguousarray(state_np, dtype=np.float32)).cuda()
        tok = torch.from_numpy(np.ascontiguousarray(tok_np, dtype=np.int32)).cuda() if tok_np is not None else None
        out = torch.full_like(st, float("nan"))
        ws = moe.alloc_hc_workspace(self.lay.dims, self.hc, R) if ws is None else ws
        moe.forward_hc(self.lay.dims, st, tok, kind, self.lay.cw, self.hw, out, ws)
        mixes, maps, fin, fout = (v.cpu().numpy() for v in moe.hc_view(self.lay.dims, self.hc, R, ws))
        lg, idx, w = (v.cpu().numpy() for v in moe.routing_view(self.lay.dims, R, ws))
        stat = moe.status(ws)
        torch.cuda.synchronize()
        return dict(out=out.cpu().numpy(), mixes=mixes, maps=maps, ffn_in=fin, ffn_out=fout, logits=lg, idx=idx, w=w,
                    status=stat)


def check_hc(hl: HcLayer, state, tok, kind, g, ffn_tol):
    """Step by step, then end to end."""
    cfg, hc = hl.cfg, hl.hc
    res = hcr.forward(state, tok, kind, hl.lay.oracle_w, hl.oracle_hw, cfg.top_k, cfg.eps)
    # mixes: f32 dots over hc*hidden products of O(0.02) weights
    scale = np.abs(res["mixes"]).max()
    np.testing.assert_allclose(g["mixes"], res["mixes"], rtol=0, atol=2e-5 * max(scale, 1.0))
    # maps from the GPU's own mixes (the split alone), then against the oracle's
    pre, post, comb = hcr.split_sinkhorn(g["mixes"], hl.host.hc_scale, hl.host.hc_base, hc, hl.host.iters)
    own = np.concatenate([pre, post, comb.reshape(len(pre), -1)], axis=1)
    np.testing.assert_allclose(g["maps"], own, rtol=0, atol=5e-6)
    ref_maps = np.concatenate([res["pre"], res["post"], res["comb"].reshape(len(pre), -1)], axis=1)
    np.testing.assert_allclose(g["maps"], ref_maps, rtol=0, atol=5e-5)
    # FFN input from the GPU's own maps
    np.testing.assert_allclose(g["ffn_in"], hcr.hc_pre(state, g["maps"][:, :hc]), rtol=0, atol=2e-6)
    check_output(g["ffn_in"], res["ffn_input"], rel=1e-5, maxabs=5e-5, what="ffn input")
    # the FFN on the GPU's own input, under the FFN's own rules
    check_forward(hl.lay, g["ffn_in"], tok, kind, g["ffn_out"], g["logits"], g["idx"], g["w"], rel=ffn_tol,
                  maxabs=5 * ffn_tol)
    # new state from the GPU's own FFN output and maps
    gp, gq = g["maps"][:, :hc], g["maps"][:, hc:2 * hc]
    gc = g["maps"][:, 2 * hc:].reshape(-1, hc, hc)
    np.testing.assert_allclose(g["out"], hcr.hc_post(g["ffn_out"], state, gq, gc), rtol=0, atol=2e-5)
    assert gp.shape == (state.shape[0], hc)
    # end to end (the maps' f32 rounding moves the state term by ~1e-5)
    tol = max(ffn_tol, 5e-5)
    check_output(g["out"].reshape(len(state), -1), res["out"].reshape(len(state), -1), rel=tol, maxabs=5 * tol,
                 what=f"hc={hc} new state")
    # invariant: the comb columns sum to one, so the streams' total is
    # (sum_j post_j) * ffn_output + the old total
    tot = g["out"].sum(axis=1)
    want = gq.sum(axis=1)[:, None] * g["ffn_out"] + state.sum(axis=1)
    np.testing.assert_allclose(tot, want, rtol=0, atol=1e-4 * max(1.0, np.abs(want).max()))
    return res


@pytest.fixture(scope="module")
def tiny():
    return Layer(gen.config(0))


@pytest.mark.parametrize("hc", [1, 2, 3, 4])
@pytest.mark.parametrize("rows", [1, 3, 5, 37])
def test_tiny_hc(tiny, hc, rows):
    hl = HcLayer(tiny, hc, rows)
    state = hl.host.state
    g = hl.run(state, None, SCORE)
    assert g["status"] == 0
    check_hc(hl, state, None, SCORE, g, 1e-5 if rows <= 4 else 2e-3)


@pytest.mark.parametrize("rows", [4, 300])
def test_tiny_hc_hash_and_reuse(tiny, rows):
    """A hash layer, and one workspace reused by a second call with fewer
    rows (the mix launch's arrival counts return to zero)."""
    hl = HcLayer(tiny, 4, rows)
    tok = np.random.default_rng(40 + rows).integers(0, tiny.cfg.table_rows, rows).astype(np.int32)
    ws = moe.alloc_hc_workspace(tiny.dims, 4, rows)
    g = hl.run(hl.host.state, tok, HASH, ws)
    check_hc(hl, hl.host.state, tok, HASH, g, 1e-5 if rows <= 4 else 2e-3)
    again = hl.run(hl.host.state, tok, HASH, ws)
    np.testing.assert_array_equal(again["out"], g["out"])  # bitwise reproducible
    sub = hl.host.state[: rows // 2 + 1]
    g2 = hl.run(sub, tok[: rows // 2 + 1], HASH, ws)
    check_hc(hl, sub, tok[: rows // 2 + 1], HASH, g2, 1e-5 if len(sub) <= 4 else 2e-3)


@pytest.fixture(scope="module")
def full():
    return Layer(gen.config(1))


@pytest.mark.parametrize("rows", [1, 4, 512])
def test_full_hc(full, rows):
    """The full shape (hc 4 streams of 4096), every row."""
    cfg = gen.config(1 if rows == 1 else 3)
    lay = full if rows == 1 else Layer(cfg, share=full)
    hl = HcLayer(lay, 4, rows)
    g = hl.run(hl.host.state, None, SCORE)
    assert g["status"] == 0
    check_hc(hl, hl.host.state, None, SCORE, g, 1e-5 if rows <= 4 else 2e-3)
