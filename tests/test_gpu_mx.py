"""The layer with block-scaled 8-bit (MXFP8) expert weights, through the C
ABI (moe_ffn_forward_mxfp8), against the float64 oracle that decodes the same
codes and scales exactly; and against the bf16 path on a layer holding the
same weight values.  Needs an MI355X; run with ``-m gpu``."""

from __future__ import annotations

import numpy as np
import pytest

from mixture_experts_ffn_rmsnorm_amd import inputs as gen
from mixture_experts_ffn_rmsnorm_amd import moe
from oracle import moe_ref as ref
from tests.gpu_common import check_forward, check_output, report_near_ties

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]

SCORE, HASH = ref.LAYER_SCORE, ref.LAYER_HASH


class MxLayer:
    """One layer with MXFP8 experts on the device, and the oracle's view of
    the same codes and scales."""

    def __init__(self, cfg: gen.Config, layer: int = 0):
        import torch

        self.cfg = cfg
        hi = gen.host_inputs(cfg, layer=layer)
        self.host = hi
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        self.norm_w, self.bias = t(hi.norm_w), t(hi.sel_bias)
        self.router = t(hi.router.view(np.int16)).view(torch.bfloat16)
        self.table = t(hi.tid2eid) if hi.tid2eid is not None else None
        routed, shared = gen.mx_expert_weights(cfg, "cuda", layer)
        self.routed, self.shared = routed, shared
        self._cache = {}

        def expert(e):
            if e not in self._cache:
                self._cache[e] = tuple(gen.mx_host((m[0][e], m[1][e])) for m in routed)
            return self._cache[e]

        self.oracle_w = ref.Weights(hi.norm_w, hi.router, hi.sel_bias, hi.tid2eid, expert,
                                    tuple(gen.mx_host(m) for m in shared))
        self.dims = moe.dims_of(cfg)
        self.cw = moe.make_mx_weights(self.norm_w, self.router, self.bias, self.table, *routed, *shared)

    def run(self, x_np, tok_np, kind):
        import torch

        R = x_np.shape[0]
        x = torch.from_numpy(np.ascontiguousarray(x_np, dtype=np.float32)).cuda()
        tok = torch.from_numpy(np.ascontiguousarray(tok_np, dtype=np.int32)).cuda() if tok_np is not None else None
        out = torch.full((R, self.cfg.hidden), float("nan"), dtype=torch.float32, device="cuda")
        ws = moe.alloc_workspace(self.dims, R)
        moe.forward_mxfp8(self.dims, x, tok, kind, self.cw, out, ws)
        lg, idx, w = moe.routing_view(self.dims, R, ws)
        st = moe.status(ws)
        torch.cuda.synchronize()
        return out.cpu().numpy(), lg.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy(), st

    def bf16_twin(self):
        """bf16 device weights holding exactly the MX values (E4M3 * 2^k fits
        bf16), bound for moe_ffn_forward."""
        import torch

        def b16(pair):
            q, s = pair
            v = q.view(torch.float8_e4m3fn).to(torch.float32)
            sc = torch.exp2(s.to(torch.float32) - 127.0).repeat_interleave(gen.MX_BLOCK, dim=-1)
            return (v * sc).to(torch.bfloat16)

        self._twin = [b16(m) for m in self.routed] + [b16(m) for m in self.shared]
        return moe.make_weights(self.norm_w, self.router, self.bias, self.table, *self._twin)


def _x(cfg, rows, seed):
    return np.random.default_rng(seed).standard_normal((rows, cfg.hidden)).astype(np.float32)


def _tok(cfg, rows, seed):
    return np.random.default_rng(seed).integers(0, cfg.table_rows, rows).astype(np.int32)


@pytest.fixture(scope="module")
def tiny_mx():
    return MxLayer(gen.config(0))


@pytest.mark.parametrize("rows", [1, 2, 3, 4])
@pytest.mark.parametrize("kind", [SCORE, HASH])
def test_tiny_mx_decode(tiny_mx, rows, kind):
    cfg = tiny_mx.cfg
    x = _x(cfg, rows, 300 + rows)
    tok = _tok(cfg, rows, 310 + rows) if kind == HASH else None
    out, lg, idx, w, st = tiny_mx.run(x, tok, kind)
    assert st == 0
    check_forward(tiny_mx, x, tok, kind, out, lg, idx, w, rel=1e-5, maxabs=5e-5)


def test_tiny_mx_matches_bf16_twin(tiny_mx):
    """The MX path and the bf16 path on the same weight values agree to f32
    rounding (the MX path scales each lane's 8-term partial once per 32-
    column block instead of every weight)."""
    import torch

    cfg = tiny_mx.cfg
    twin = tiny_mx.bf16_twin()
    for rows in (1, 4):
        x = _x(cfg, rows, 320 + rows)
        out_mx = tiny_mx.run(x, None, SCORE)[0]
        xd = torch.from_numpy(x).cuda()
        ob = torch.empty_like(xd)
        moe.forward(tiny_mx.dims, xd, None, SCORE, twin, ob, moe.alloc_workspace(tiny_mx.dims, rows))
        torch.cuda.synchronize()
        check_output(out_mx, ob.cpu().numpy(), rel=1e-6, maxabs=1e-5, what=f"mx vs bf16 twin, {rows} rows")


@pytest.fixture(scope="module")
def full_mx():
    return MxLayer(gen.config(1))


def test_full_mx_decode_one_row(full_mx):
    hi = full_mx.host
    out, lg, idx, w, st = full_mx.run(hi.x, None, SCORE)
    assert st == 0
    check_forward(full_mx, hi.x, None, SCORE, out, lg, idx, w, rel=1e-5, maxabs=5e-5)


def test_full_mx_decode_cohort(full_mx):
    cfg = gen.config(2)
    lay = MxLayer(cfg)
    hi = lay.host
    out, lg, idx, w, st = lay.run(hi.x, hi.token_ids, HASH)
    assert st == 0
    check_forward(lay, hi.x, hi.token_ids, HASH, out, lg, idx, w, rel=1e-5, maxabs=5e-5)


@pytest.mark.parametrize("rows", [2, 3])
def test_full_mx_decode_ragged(full_mx, rows):
    x = _x(full_mx.cfg, rows, 330 + rows)
    out, lg, idx, w, st = full_mx.run(x, None, SCORE)
    near = check_forward(full_mx, x, None, SCORE, out, lg, idx, w, rel=1e-5, maxabs=5e-5)
    report_near_ties(f"mx {rows} rows", near, rows)
