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


E2M1 = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0)


class MxLayer:
    """One layer with block-scaled experts on the device (``fmt`` "mxfp8" or
    "mxfp4"), and the oracle's view of the same codes and scales."""

    def __init__(self, cfg: gen.Config, layer: int = 0, fmt: str = "mxfp8"):
        import torch

        self.cfg = cfg
        self.fmt = fmt
        tag = (ref.MXFP4,) if fmt == "mxfp4" else ()
        hi = gen.host_inputs(cfg, layer=layer)
        self.host = hi
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        self.norm_w, self.bias = t(hi.norm_w), t(hi.sel_bias)
        self.router = t(hi.router.view(np.int16)).view(torch.bfloat16)
        self.table = t(hi.tid2eid) if hi.tid2eid is not None else None
        draw = gen.mx4_expert_weights if fmt == "mxfp4" else gen.mx_expert_weights
        routed, shared = draw(cfg, "cuda", layer)
        self.routed, self.shared = routed, shared

        def expert(e):  # fetched per call: the oracle asks once per expert
            return tuple(gen.mx_host((m[0][e], m[1][e])) + tag for m in self.routed)

        self.oracle_w = ref.Weights(hi.norm_w, hi.router, hi.sel_bias, hi.tid2eid, expert,
                                    tuple(gen.mx_host(m) + tag for m in shared))
        self.dims = moe.dims_of(cfg)
        self.cw = moe.make_mx_weights(self.norm_w, self.router, self.bias, self.table, *routed, *shared)

    def set_scale(self, mat, e, row, block, value):
        """Overwrite one block scale of routed matrix `mat` (0 gate, 1 up,
        2 down) of expert e on the device (the oracle reads it from there)."""
        self.routed[mat][1][e, row, block] = value

    def run(self, x_np, tok_np, kind):
        import torch

        R = x_np.shape[0]
        x = torch.from_numpy(np.ascontiguousarray(x_np, dtype=np.float32)).cuda()
        tok = torch.from_numpy(np.ascontiguousarray(tok_np, dtype=np.int32)).cuda() if tok_np is not None else None
        out = torch.full((R, self.cfg.hidden), float("nan"), dtype=torch.float32, device="cuda")
        ws = moe.alloc_workspace(self.dims, R)
        (moe.forward_mxfp4 if self.fmt == "mxfp4" else moe.forward_mxfp8)(self.dims, x, tok, kind, self.cw, out, ws)
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
            if self.fmt == "mxfp4":
                codes = torch.stack([q & 15, q >> 4], dim=-1).flatten(-2).long()
                v = torch.tensor(E2M1, device=q.device)[codes]
            else:
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


# ------------------------------------------------------------ prefill ---
# rows > 4: the grouped GEMM with 8-bit B tiles (37 rows: the small row tile
# with the cross-tile stream; 300: the big tile), fp16 operands
PREFILL_TOL = 2e-3


@pytest.mark.parametrize("rows", [5, 8, 37, 300])
def test_tiny_mx_prefill_score(tiny_mx, rows):
    cfg = tiny_mx.cfg
    x = _x(cfg, rows, 340 + rows)
    out, lg, idx, w, st = tiny_mx.run(x, None, SCORE)
    assert st == 0
    check_forward(tiny_mx, x, None, SCORE, out, lg, idx, w, rel=PREFILL_TOL, maxabs=PREFILL_TOL * 5)


@pytest.mark.parametrize("rows", [8, 37, 300])
def test_tiny_mx_prefill_hash(tiny_mx, rows):
    cfg = tiny_mx.cfg
    x = _x(cfg, rows, 350 + rows)
    tok = _tok(cfg, rows, 360 + rows)
    out, lg, idx, w, st = tiny_mx.run(x, tok, HASH)
    assert st == 0
    check_forward(tiny_mx, x, tok, HASH, out, lg, idx, w, rel=PREFILL_TOL, maxabs=PREFILL_TOL * 5)


@pytest.mark.parametrize("rows", [37, 300])
def test_tiny_mx_prefill_matches_bf16_twin(tiny_mx, rows):
    """Both formats give the matrix cores the same fp16 weights (the decoded
    value fits bf16 exactly and both round it to fp16 the same way); only the
    k order inside the MFMAs differs, so the outputs agree far below the
    oracle tolerance, up to the odd 1-ulp flip of an fp16-rounded h."""
    import torch

    cfg = tiny_mx.cfg
    twin = tiny_mx.bf16_twin()
    x = _x(cfg, rows, 370 + rows)
    out_mx = tiny_mx.run(x, None, SCORE)[0]
    xd = torch.from_numpy(x).cuda()
    ob = torch.empty_like(xd)
    moe.forward(tiny_mx.dims, xd, None, SCORE, twin, ob, moe.alloc_workspace(tiny_mx.dims, rows))
    torch.cuda.synchronize()
    check_output(out_mx, ob.cpu().numpy(), rel=1e-4, maxabs=5e-4, what=f"mx vs bf16 twin, {rows} rows")


@pytest.mark.parametrize("rows", [3, 37, 300])
def test_tiny_mx_special_scales(rows):
    """A block scale of 0 (2^-127: the block's weights vanish below fp16 and
    f32 resolution) and one of 255 (NaN: every output of the rows routed to
    that expert is NaN, on the oracle too).  Finite rows match the oracle; the
    NaN rows are the same rows; the fp16 path reports them."""
    lay = MxLayer(gen.config(0), layer=3)
    cfg = lay.cfg
    x = _x(cfg, rows, 380 + rows)
    _, _, idx0, _, _ = lay.run(x, None, SCORE)
    e_nan = int(idx0[0, 0])                              # row 0's first expert
    e_zero = int(idx0[rows - 1, -1]) if int(idx0[rows - 1, -1]) != e_nan else int(idx0[rows - 1, 0])
    lay.set_scale(0, e_nan, 5, 1, 255)                  # gate row 5, inputs 32..63
    lay.set_scale(2, e_zero, 7, 0, 0)                   # down row 7, inputs 0..31
    out, lg, idx, w, st = lay.run(x, None, SCORE)
    res = ref.forward(x, None, SCORE, lay.oracle_w, cfg.top_k, cfg.eps)
    np.testing.assert_array_equal(idx, idx0)  # the router does not see expert weights
    nan_rows = np.isnan(res["out"]).any(axis=1)
    assert nan_rows[0] and not nan_rows.all()
    np.testing.assert_array_equal(np.isnan(out).any(axis=1), nan_rows)
    assert np.isnan(out[nan_rows]).all()
    if rows > 4:
        assert st & moe.FLAG_F16_RANGE
    tol = 1e-5 if rows <= 4 else PREFILL_TOL
    check_output(out[~nan_rows], res["out"][~nan_rows], rel=tol, maxabs=tol * 5, what="finite rows")


def test_full_mx_prefill_512(full_mx):
    """Every row of the 512-row prefill with MXFP8 experts."""
    cfg = gen.config(3)
    lay = MxLayer(cfg)
    hi = lay.host
    out, lg, idx, w, st = lay.run(hi.x, None, SCORE)
    assert st == 0
    near = check_forward(lay, hi.x, None, SCORE, out, lg, idx, w)
    report_near_ties(f"mx {cfg.name}", near, cfg.rows)


def test_full_mx_prefill_8192_skewed():
    """Every row of the 8192-row skewed prefill (16 hot experts: the big
    tile, dynamically dealt tail tiles) with MXFP8 experts; bitwise
    reproducible."""
    cfg = gen.config(4)
    lay = MxLayer(cfg)
    hi = lay.host
    out, lg, idx, w, st = lay.run(hi.x, None, SCORE)
    assert st == 0
    assert np.isin(idx, hi.hot).all()
    near = check_forward(lay, hi.x, None, SCORE, out, lg, idx, w)
    report_near_ties(f"mx {cfg.name}", near, cfg.rows)
    np.testing.assert_array_equal(out, lay.run(hi.x, None, SCORE)[0])


# ------------------------------------------------------------- MXFP4 ---
@pytest.fixture(scope="module")
def tiny_mx4():
    return MxLayer(gen.config(0), fmt="mxfp4")


@pytest.mark.parametrize("rows", [1, 2, 3, 4])
@pytest.mark.parametrize("kind", [SCORE, HASH])
def test_tiny_mx4_decode(tiny_mx4, rows, kind):
    cfg = tiny_mx4.cfg
    x = _x(cfg, rows, 400 + rows)
    tok = _tok(cfg, rows, 410 + rows) if kind == HASH else None
    out, lg, idx, w, st = tiny_mx4.run(x, tok, kind)
    assert st == 0
    check_forward(tiny_mx4, x, tok, kind, out, lg, idx, w, rel=1e-5, maxabs=5e-5)


def test_tiny_mx4_matches_bf16_twin(tiny_mx4):
    """E2M1 * 2^k fits bf16 exactly: the bf16 path on the same values agrees
    to f32 rounding."""
    import torch

    cfg = tiny_mx4.cfg
    twin = tiny_mx4.bf16_twin()
    for rows in (1, 4):
        x = _x(cfg, rows, 420 + rows)
        out_mx = tiny_mx4.run(x, None, SCORE)[0]
        xd = torch.from_numpy(x).cuda()
        ob = torch.empty_like(xd)
        moe.forward(tiny_mx4.dims, xd, None, SCORE, twin, ob, moe.alloc_workspace(tiny_mx4.dims, rows))
        torch.cuda.synchronize()
        check_output(out_mx, ob.cpu().numpy(), rel=1e-6, maxabs=1e-5, what=f"mx4 vs bf16 twin, {rows} rows")


@pytest.mark.parametrize("rows", [3, 37])
def test_tiny_mx4_special_scales(rows):
    """Scale 255 (NaN) poisons exactly the rows routed to its expert; scale 0
    (2^-127) makes its block vanish."""
    lay = MxLayer(gen.config(0), layer=3, fmt="mxfp4")
    cfg = lay.cfg
    x = _x(cfg, rows, 430)
    _, _, idx0, _, _ = lay.run(x, None, SCORE)
    e_nan = int(idx0[0, 0])
    e_zero = int(idx0[rows - 1, -1]) if int(idx0[rows - 1, -1]) != e_nan else int(idx0[rows - 1, 0])
    lay.set_scale(0, e_nan, 5, 1, 255)
    lay.set_scale(2, e_zero, 7, 0, 0)
    out, lg, idx, w, st = lay.run(x, None, SCORE)
    res = ref.forward(x, None, SCORE, lay.oracle_w, cfg.top_k, cfg.eps)
    nan_rows = np.isnan(res["out"]).any(axis=1)
    assert nan_rows[0] and not nan_rows.all()
    np.testing.assert_array_equal(np.isnan(out).any(axis=1), nan_rows)
    if rows > 4:
        assert st & moe.FLAG_F16_RANGE
    tol = 1e-5 if rows <= 4 else PREFILL_TOL
    check_output(out[~nan_rows], res["out"][~nan_rows], rel=tol, maxabs=5 * tol, what="finite rows")


@pytest.mark.parametrize("rows", [5, 37, 300])
def test_tiny_mx4_prefill(tiny_mx4, rows):
    """More than 4 rows: 4-bit B tiles (37 rows the small tile, 300 the big
    one) converted to fp16 with their scales."""
    cfg = tiny_mx4.cfg
    x = _x(cfg, rows, 440 + rows)
    out, lg, idx, w, st = tiny_mx4.run(x, None, SCORE)
    assert st == 0
    check_forward(tiny_mx4, x, None, SCORE, out, lg, idx, w, rel=PREFILL_TOL, maxabs=PREFILL_TOL * 5)
    tok = _tok(cfg, rows, 445 + rows)
    out, lg, idx, w, st = tiny_mx4.run(x, tok, HASH)
    assert st == 0
    check_forward(tiny_mx4, x, tok, HASH, out, lg, idx, w, rel=PREFILL_TOL, maxabs=PREFILL_TOL * 5)


@pytest.mark.parametrize("rows", [37, 300])
def test_tiny_mx4_prefill_matches_bf16_twin(tiny_mx4, rows):
    """The same fp16 operands as the bf16 path on the same values; only the
    k order inside the MFMAs differs."""
    import torch

    cfg = tiny_mx4.cfg
    twin = tiny_mx4.bf16_twin()
    x = _x(cfg, rows, 460 + rows)
    out_mx = tiny_mx4.run(x, None, SCORE)[0]
    xd = torch.from_numpy(x).cuda()
    ob = torch.empty_like(xd)
    moe.forward(tiny_mx4.dims, xd, None, SCORE, twin, ob, moe.alloc_workspace(tiny_mx4.dims, rows))
    torch.cuda.synchronize()
    check_output(out_mx, ob.cpu().numpy(), rel=1e-4, maxabs=5e-4, what=f"mx4 vs bf16 twin, {rows} rows")


def test_full_mx4_prefill_512():
    cfg = gen.config(3)
    lay = MxLayer(cfg, fmt="mxfp4")
    hi = lay.host
    out, lg, idx, w, st = lay.run(hi.x, None, SCORE)
    assert st == 0
    near = check_forward(lay, hi.x, None, SCORE, out, lg, idx, w)
    report_near_ties(f"mx4 {cfg.name}", near, cfg.rows)


def test_full_mx4_prefill_8192_skewed():
    cfg = gen.config(4)
    lay = MxLayer(cfg, fmt="mxfp4")
    hi = lay.host
    out, lg, idx, w, st = lay.run(hi.x, None, SCORE)
    assert st == 0
    near = check_forward(lay, hi.x, None, SCORE, out, lg, idx, w)
    report_near_ties(f"mx4 {cfg.name}", near, cfg.rows)
    np.testing.assert_array_equal(out, lay.run(hi.x, None, SCORE)[0])


@pytest.fixture(scope="module")
def full_mx4():
    return MxLayer(gen.config(1), fmt="mxfp4")


def test_full_mx4_decode_one_row(full_mx4):
    hi = full_mx4.host
    out, lg, idx, w, st = full_mx4.run(hi.x, None, SCORE)
    assert st == 0
    check_forward(full_mx4, hi.x, None, SCORE, out, lg, idx, w, rel=1e-5, maxabs=5e-5)


def test_full_mx4_decode_cohort():
    lay = MxLayer(gen.config(2), fmt="mxfp4")
    hi = lay.host
    out, lg, idx, w, st = lay.run(hi.x, hi.token_ids, HASH)
    assert st == 0
    check_forward(lay, hi.x, hi.token_ids, HASH, out, lg, idx, w, rel=1e-5, maxabs=5e-5)


@pytest.mark.parametrize("rows", [2, 3])
def test_full_mx4_decode_ragged(full_mx4, rows):
    x = _x(full_mx4.cfg, rows, 450 + rows)
    out, lg, idx, w, st = full_mx4.run(x, None, SCORE)
    near = check_forward(full_mx4, x, None, SCORE, out, lg, idx, w, rel=1e-5, maxabs=5e-5)
    report_near_ties(f"mx4 {rows} rows", near, rows)
