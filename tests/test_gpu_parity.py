"""Parity of the HIP path (through the C ABI) with the float64 oracle on the
same seeded inputs.  Needs an MI355X; run with ``-m gpu``."""

from __future__ import annotations

import numpy as np
import pytest

from mixture_experts_ffn_rmsnorm_amd import inputs as gen
from mixture_experts_ffn_rmsnorm_amd import moe
from oracle import moe_ref as ref
from tests.gpu_common import LOGIT_ATOL_PREFILL, Layer, check_forward, check_output, check_routing_exact

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]

SCORE, HASH = ref.LAYER_SCORE, ref.LAYER_HASH


@pytest.fixture(scope="module")
def tiny():
    return Layer(gen.config(0))


def _x(cfg, rows, seed=5):
    return np.random.default_rng(seed).standard_normal((rows, cfg.hidden)).astype(np.float32)


def _tok(cfg, rows, seed=6):
    return np.random.default_rng(seed).integers(0, cfg.table_rows, rows).astype(np.int32)


# ------------------------------------------------------------------ tiny ---
@pytest.mark.parametrize("rows", [1, 2, 3, 4, 5, 8, 37, 300])
def test_tiny_score(tiny, rows):
    x = _x(tiny.cfg, rows)
    out, lg, idx, w, st = tiny.run(x, None, SCORE)
    assert st == 0
    tight = 1e-5 if rows <= 4 else 2e-3  # f32 decode path vs fp16 matrix-core path
    check_forward(tiny, x, None, SCORE, out, lg, idx, w, rel=tight, maxabs=tight * 5)


@pytest.mark.parametrize("rows", [1, 4, 8, 37])
def test_tiny_hash(tiny, rows):
    x = _x(tiny.cfg, rows, seed=9)
    tok = _tok(tiny.cfg, rows)
    out, lg, idx, w, st = tiny.run(x, tok, HASH)
    assert st == 0
    tight = 1e-5 if rows <= 4 else 2e-3
    check_forward(tiny, x, tok, HASH, out, lg, idx, w, rel=tight, maxabs=tight * 5)


def test_tiny_seeded_rows_config0(tiny):
    """The tiny workload exactly as generated (8 rows of the seeded x)."""
    hi = tiny.host
    out, lg, idx, w, st = tiny.run(hi.x, None, SCORE)
    check_forward(tiny, hi.x, None, SCORE, out, lg, idx, w)


@pytest.mark.parametrize("rows", [3, 12])
def test_tiny_zero_input_closed_form(tiny, rows):
    x = np.zeros((rows, tiny.cfg.hidden), np.float32)
    out, lg, idx, w, st = tiny.run(x, None, SCORE)
    assert np.all(out == 0.0) and np.all(lg == 0.0)
    want = np.argsort(-tiny.host.sel_bias.astype(np.float64), kind="stable")[:6]
    assert (idx == want[None, :]).all()
    assert np.all(w == np.float32(1.0 / 6.0))


@pytest.mark.parametrize("rows", [2, 9])
def test_tiny_invalid_tokens_and_entries(tiny, rows):
    cfg = tiny.cfg
    table = tiny.host.tid2eid.copy()
    tok = _tok(cfg, rows, seed=11)
    tok[0] = -3                    # bad token id: whole row masked
    tok[1] = cfg.table_rows        # one past the end
    bad_entry_tok = 17
    table[bad_entry_tok, 2] = cfg.experts + 5
    table[bad_entry_tok, 4] = -1
    if rows > 2:
        tok[2] = bad_entry_tok
    lay = Layer(cfg).with_table(table)
    x = _x(cfg, rows, seed=12)
    out, lg, idx, w, st = lay.run(x, tok, HASH)
    exp = moe.FLAG_BAD_TOKEN | (moe.FLAG_BAD_TABLE_ENTRY if rows > 2 else 0)
    assert st == exp
    assert (idx[0] == -1).all() and (w[0] == 0).all()
    check_forward(lay, x, tok, HASH, out, lg, idx, w)


def test_tiny_duplicate_table_entries(tiny):
    """A malformed table row that lists one expert twice: each slot still
    contributes with its own weight."""
    cfg = tiny.cfg
    table = tiny.host.tid2eid.copy()
    table[5] = [3, 3, 7, 3, 9, 11]
    lay = Layer(cfg).with_table(table)
    for rows in (4, 10):
        tok = _tok(cfg, rows, seed=13)
        tok[1] = 5
        x = _x(cfg, rows, seed=14)
        out, lg, idx, w, st = lay.run(x, tok, HASH)
        assert st == 0
        check_forward(lay, x, tok, HASH, out, lg, idx, w)


def test_tiny_hash_equals_score(tiny):
    cfg = tiny.cfg
    rows = 16
    x = _x(cfg, rows, seed=21)
    out_s, lg, idx_s, w_s, _ = tiny.run(x, None, SCORE)
    tok = (np.arange(rows) * 31 + 3).astype(np.int32)
    table = np.zeros((cfg.table_rows, cfg.top_k), np.int32)
    table[tok] = idx_s
    lay = Layer(cfg).with_table(table)
    out_h, _, idx_h, w_h, _ = lay.run(x, tok, HASH)
    np.testing.assert_array_equal(idx_h, idx_s)
    np.testing.assert_array_equal(w_h, w_s)
    np.testing.assert_array_equal(out_h, out_s)


@pytest.mark.parametrize("rows", [1, 4, 64])
def test_tiny_deterministic(tiny, rows):
    x = _x(tiny.cfg, rows, seed=31)
    a = tiny.run(x, None, SCORE)[0]
    b = tiny.run(x, None, SCORE)[0]
    np.testing.assert_array_equal(a, b)


# ------------------------------------------------------------ moe_route ---
def _route_gpu(layer, logits, tok, kind):
    import torch

    lg = torch.from_numpy(np.ascontiguousarray(logits, np.float32)).cuda()
    tk = None if tok is None else torch.from_numpy(np.ascontiguousarray(tok, np.int32)).cuda()
    R, K = logits.shape[0], layer.cfg.top_k
    idx = torch.empty((R, K), dtype=torch.int32, device="cuda")
    w = torch.empty((R, K), dtype=torch.float32, device="cuda")
    moe.route(layer.dims, lg, tk, kind, layer.cw, idx, w)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), w.cpu().numpy()


class _RouteOnly:
    """The routing parameters of a layer, on the device and for the oracle."""

    def __init__(self, cfg):
        import torch

        hi = gen.host_inputs(cfg)
        if hi.tid2eid is None:
            hi.tid2eid = gen.distinct_table(cfg.param_seed, 4096, cfg.experts, cfg.top_k)
        self.cfg, self.host = cfg, hi
        self.dims = moe.make_dims(cfg.hidden, cfg.experts, cfg.top_k, cfg.inter, hi.tid2eid.shape[0], cfg.eps)
        self.bias = torch.from_numpy(hi.sel_bias).cuda()
        self.table = torch.from_numpy(hi.tid2eid).cuda()
        self.cw = moe.WeightsC(None, None, self.bias.data_ptr(), self.table.data_ptr(), None, None, None, None, None,
                               None)
        self.oracle_w = ref.Weights(hi.norm_w, hi.router, hi.sel_bias, hi.tid2eid, None, None)


@pytest.mark.parametrize("cfg_i", [0, 1, 4])
def test_route_bit_exact_on_oracle_logits(cfg_i):
    lay = _RouteOnly(gen.config(cfg_i))
    cfg = lay.cfg
    rows = 3000
    rng = np.random.default_rng(41)
    xn = rng.standard_normal((rows, cfg.hidden))
    logits = ref.router_logits(xn, lay.host.router).astype(np.float32)
    logits[:4] = 0.0                          # exact ties: bias decides, then index
    logits[4:8] = np.round(logits[4:8])       # many exact ties
    idx, w = _route_gpu(lay, logits, None, SCORE)
    o_idx, o_w, _ = ref.score_route(logits.astype(np.float64), lay.host.sel_bias, cfg.top_k)
    np.testing.assert_array_equal(idx, o_idx)
    np.testing.assert_allclose(w, o_w, rtol=2e-7, atol=1e-9)
    assert np.abs(w.sum(1) - 1).max() <= 4e-7
    tok = rng.integers(-2, lay.oracle_w.tid2eid.shape[0] + 2, rows).astype(np.int32)
    idx, w = _route_gpu(lay, logits, tok, HASH)
    o_idx, o_w, _ = ref.hash_route(logits.astype(np.float64), tok, lay.oracle_w.tid2eid, cfg.top_k)
    np.testing.assert_array_equal(idx, o_idx)
    np.testing.assert_allclose(w, o_w, rtol=2e-7, atol=1e-9)


# ------------------------------------------------------------- full size ---
@pytest.fixture(scope="module")
def full():
    return Layer(gen.config(1))


def test_full_decode_config1(full):
    hi = full.host
    out, lg, idx, w, st = full.run(hi.x, None, SCORE)
    assert st == 0
    check_forward(full, hi.x, None, SCORE, out, lg, idx, w, rel=1e-5, maxabs=5e-5)


def test_full_decode_cohort_config2(full):
    cfg = gen.config(2)
    hi = gen.host_inputs(cfg)
    lay = Layer(cfg, share=full)
    out, lg, idx, w, st = lay.run(hi.x, hi.token_ids, HASH)
    assert st == 0
    check_forward(lay, hi.x, hi.token_ids, HASH, out, lg, idx, w, rel=1e-5, maxabs=5e-5)


@pytest.mark.parametrize("rows", [2, 3, 5, 129])
def test_full_ragged_rows(full, rows):
    x = _x(full.cfg, rows, seed=50 + rows)
    out, lg, idx, w, st = full.run(x, None, SCORE)
    sample = np.unique(np.linspace(0, rows - 1, min(rows, 6)).astype(int))
    tight = 1e-5 if rows <= 4 else 2e-3
    check_forward(full, x, None, SCORE, out, lg, idx, w, rows=sample, rel=tight, maxabs=tight * 5)
    check_routing_exact(full, lg, idx, w, None, SCORE)


@pytest.mark.parametrize("rows", [1500, 3000])
def test_full_prefill_router_slices(full, rows):
    """Batches whose router splits the experts over 4 (1500 rows) and 2 (3000
    rows) blocks per 32-row group, each with a ragged last group: every row's
    logits against the oracle router, every row's routing exact, sampled
    outputs end to end."""
    cfg = full.cfg
    x = _x(cfg, rows, seed=70 + rows)
    out, lg, idx, w, st = full.run(x, None, SCORE)
    assert st == 0
    xn = ref.rms_norm(x, full.host.norm_w, cfg.eps)
    np.testing.assert_allclose(lg, ref.router_logits(xn, full.host.router), rtol=0, atol=LOGIT_ATOL_PREFILL)
    check_routing_exact(full, lg, idx, w, None, SCORE)
    check_forward(full, x, None, SCORE, out, lg, idx, w, rows=[0, 31, 32, rows // 2, rows - 2, rows - 1])


def test_full_decode_one_row_hash(full):
    """One hash-routed row at full size (the one-row path: keys and sigmoids
    from the router launch, routing inside every routed gate/up block), a
    normal token and then a bad one."""
    cfg = gen.config(2)
    lay = Layer(cfg, share=full)
    x = _x(cfg, 1, seed=91)
    tok = _tok(cfg, 1, seed=92)
    out, lg, idx, w, st = lay.run(x, tok, HASH)
    assert st == 0
    check_routing_exact(lay, lg, idx, w, tok, HASH)
    check_forward(lay, x, tok, HASH, out, lg, idx, w)
    tok_bad = np.array([-1], dtype=np.int32)
    out, lg, idx, w, st = lay.run(x, tok_bad, HASH)
    assert st == moe.FLAG_BAD_TOKEN and (idx == -1).all() and (w == 0).all()
    check_forward(lay, x, tok_bad, HASH, out, lg, idx, w)


def test_full_prefill_hash(full):
    """A hash-routed layer through the prefill path (700 rows: 22 groups, the
    last one ragged, experts sliced 8 ways in the router)."""
    cfg = gen.config(2)
    lay = Layer(cfg, share=full)
    rows = 700
    x = _x(cfg, rows, seed=77)
    tok = _tok(cfg, rows, seed=78)
    out, lg, idx, w, st = lay.run(x, tok, HASH)
    assert st == 0
    check_routing_exact(lay, lg, idx, w, tok, HASH)
    check_forward(lay, x, tok, HASH, out, lg, idx, w, rows=[0, 5, 350, 671, 672, 699])


def test_full_prefill_hash_invalid(full):
    """Bad token ids and bad table entries through the full-size prefill path
    (40 rows: two 32-row groups, experts sliced 8 ways): masked slots,
    status bits, and the weights renormalised over the slots left."""
    cfg = gen.config(2)
    rows = 40
    table = gen.host_inputs(cfg).tid2eid.copy()
    tok = _tok(cfg, rows, seed=81)
    tok[0] = -7                    # bad token id: the whole row is masked
    tok[33] = cfg.table_rows       # one past the end, in the second group
    bad = int(tok[5])
    table[bad, 1] = cfg.experts    # a bad entry: that slot is masked
    table[bad, 3] = -2
    lay = Layer(cfg, table=table, share=full)
    x = _x(cfg, rows, seed=82)
    out, lg, idx, w, st = lay.run(x, tok, HASH)
    assert st == moe.FLAG_BAD_TOKEN | moe.FLAG_BAD_TABLE_ENTRY
    assert (idx[0] == -1).all() and (w[0] == 0).all() and (idx[33] == -1).all()
    # a bad entry keeps its raw value as the index, with weight 0
    assert idx[5, 1] == cfg.experts and idx[5, 3] == -2 and w[5, 1] == 0 and w[5, 3] == 0
    assert abs(float(w[5].sum()) - 1.0) < 1e-5
    check_forward(lay, x, tok, HASH, out, lg, idx, w, rows=[0, 5, 6, 33, 39])


def test_full_prefill_config3(full):
    cfg = gen.config(3)
    lay = Layer(cfg, share=full)
    hi = lay.host
    out, lg, idx, w, st = lay.run(hi.x, None, SCORE)
    assert st == 0
    check_routing_exact(lay, lg, idx, w, None, SCORE)
    # logits of every row against the oracle router
    xn = ref.rms_norm(hi.x, hi.norm_w, cfg.eps)
    np.testing.assert_allclose(lg, ref.router_logits(xn, hi.router), rtol=0, atol=LOGIT_ATOL_PREFILL)
    check_forward(lay, hi.x, None, SCORE, out, lg, idx, w, rows=[0, 1, 137, 255, 400, 511])


def test_full_prefill_skewed_config4(full):
    cfg = gen.config(4)
    lay = Layer(cfg, share=full)
    hi = lay.host
    out, lg, idx, w, st = lay.run(hi.x, None, SCORE)
    assert st == 0
    assert np.isin(idx, hi.hot).all(), "skewed bias should send every slot to a hot expert"
    check_routing_exact(lay, lg, idx, w, None, SCORE)
    check_forward(lay, hi.x, None, SCORE, out, lg, idx, w, rows=[0, 1, 2, 4095, 5000, 8190, 8191])
    again = lay.run(hi.x, None, SCORE)[0]
    np.testing.assert_array_equal(out, again)


def test_workspace_and_overlap_errors_with_real_buffers(tiny):
    import torch

    d = tiny.dims
    x = torch.randn(8, tiny.cfg.hidden, device="cuda")
    out = torch.empty_like(x)
    ws = moe.alloc_workspace(d, 8)
    with pytest.raises(moe.MoeError) as e:
        moe.forward(d, x, None, SCORE, tiny.cw, out, ws[: ws.numel() - 256])
    assert e.value.code == moe.MOE_EWORKSPACE
    with pytest.raises(moe.MoeError) as e:
        moe.forward(d, x, None, SCORE, tiny.cw, x, ws)
    assert e.value.code == moe.MOE_EOVERLAP
