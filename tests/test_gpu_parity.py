"""Parity of the HIP path (through the C ABI) with the float64 oracle on the
same seeded inputs.  Needs an MI355X; run with ``-m gpu``."""

from __future__ import annotations

import numpy as np
import pytest

from mixture_experts_ffn_rmsnorm_amd import inputs as gen
from mixture_experts_ffn_rmsnorm_amd import moe
from oracle import moe_ref as ref
from tests.gpu_common import Layer, check_forward, check_output, check_routing_exact, report_near_ties

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


def _one_row_table_edge_cases(lay, x):
    """One row through the one-row path (routing inside the routed gate/up
    blocks, plan in slot order): a table row with two bad entries (the valid
    slots compact into four groups), a row that names one expert three
    times (each slot its own group, adding its own weight), and a token id
    past the table."""
    cfg = lay.cfg
    table = lay.host.tid2eid.copy()
    table[17, 2] = cfg.experts + 5
    table[17, 4] = -1
    table[5] = [3, 3, 7, 3, 9, 11]
    lay.with_table(table)
    for t, flags in ((17, moe.FLAG_BAD_TABLE_ENTRY), (5, 0), (cfg.table_rows, moe.FLAG_BAD_TOKEN)):
        tok = np.array([t], dtype=np.int32)
        out, lg, idx, w, st = lay.run(x, tok, HASH)
        assert st == flags, f"token {t}: status {st:#x}, want {flags:#x}"
        if t == 17:
            assert idx[0, 2] == cfg.experts + 5 and idx[0, 4] == -1 and w[0, 2] == 0 and w[0, 4] == 0
        check_forward(lay, x, tok, HASH, out, lg, idx, w)


def test_tiny_one_row_table_edge_cases():
    cfg = gen.config(0)
    _one_row_table_edge_cases(Layer(cfg), _x(cfg, 1, seed=15))


def _one_row_every_valid_count(lay, x):
    """One row whose table row holds v valid experts for every v = 0..top_k
    (the rest -1, at rotating positions): the one-row down streams 2(v+1)
    weight rows per wave, each count its own unrolled code."""
    cfg = lay.cfg
    K = cfg.top_k
    table = lay.host.tid2eid.copy()
    for v in range(K + 1):
        row = table[40 + v].copy()
        for j in range(K - v):
            row[(3 * v + j) % K] = -1
        table[40 + v] = row
    lay.with_table(table)
    for v in range(K + 1):
        tok = np.array([40 + v], dtype=np.int32)
        out, lg, idx, w, st = lay.run(x, tok, HASH)
        assert int((idx[0] >= 0).sum()) == v
        assert st == (moe.FLAG_BAD_TABLE_ENTRY if v < K else 0), f"{v} valid: status {st:#x}"
        check_forward(lay, x, tok, HASH, out, lg, idx, w)


def test_tiny_one_row_every_valid_count():
    cfg = gen.config(0)
    _one_row_every_valid_count(Layer(cfg), _x(cfg, 1, seed=16))


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


# ------------------------------------------------------- exact key ties ---
def tie_lead(e, E, pattern):
    """The expert whose router row and bias expert e copies: groups of four
    with bitwise-equal router rows and equal biases, so equal logits and
    equal selection keys.  'adjacent': {4j, .., 4j+3}; 'strided': {g, g+E/4,
    g+2E/4, g+3E/4} (at E = 256 one expert in each 64-expert block of the
    wave selectors' lane layout)."""
    return (e // 4) * 4 if pattern == "adjacent" else e % (E // 4)


def tie_layer(cfg, pattern, share=None):
    hi = gen.host_inputs(cfg)
    E = cfg.experts
    lead = np.array([tie_lead(e, E, pattern) for e in range(E)])
    return Layer(cfg, share=share, router=hi.router[lead], bias=hi.sel_bias[lead]), lead


def check_ties(lay, lead, x, out, lg, idx, w, rel, maxabs):
    """Tied experts get bitwise-equal logits on the GPU, the selection keeps
    the lowest indices of a tied group (a chosen group member never has an
    unchosen lower one), equal keys come out in ascending index order, and
    the indices equal the oracle's routing of the GPU logits bit for bit."""
    E, K = lay.cfg.experts, lay.cfg.top_k
    np.testing.assert_array_equal(lg, lg[:, lead])
    for r in range(idx.shape[0]):
        chosen = set(idx[r].tolist())
        for e in chosen:
            assert all(m in chosen for m in range(E) if lead[m] == lead[e] and m < e), \
                f"row {r}: expert {e} chosen over a lower tied one"
        for k in range(K - 1):
            if lead[idx[r, k]] == lead[idx[r, k + 1]]:
                assert idx[r, k] < idx[r, k + 1], f"row {r}: tied slots out of index order"
    return check_forward(lay, x, None, SCORE, out, lg, idx, w, rel=rel, maxabs=maxabs)


@pytest.fixture(scope="module", params=["adjacent", "strided"])
def tiny_ties(request):
    return tie_layer(gen.config(0), request.param)


@pytest.mark.parametrize("rows", [1, 2, 4, 8, 37])
def test_tiny_exact_ties_in_forward(tiny_ties, rows):
    """Exact key ties through the forward's own selectors: one row (keys from
    the router launch), two to four rows (the plan block's wave selector)
    and the prefill router's 8-lane selector; row 0 is all zeros for rows >=
    2, so its keys are 0.5 + bias, tied in the same groups."""
    lay, lead = tiny_ties
    x = _x(lay.cfg, rows, seed=101 + rows)
    if rows >= 2:
        x[0] = 0.0
    out, lg, idx, w, st = lay.run(x, None, SCORE)
    assert st == 0
    tight = 1e-5 if rows <= 4 else 2e-3
    check_ties(lay, lead, x, out, lg, idx, w, tight, tight * 5)


# ------------------------------------------------- fp16 operand domain ---
def _scaled_bits(bits, k):
    """bf16 bits times 2^k (exact: only the exponent changes)."""
    f = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32) * np.float32(2.0 ** k)
    return gen.f32_to_bf16_bits(f)


def _scaled_tiny(k_gu, k_down=0, poke=None):
    """The tiny layer with gate/up weights times 2^k_gu and down times
    2^k_down (routed and shared); `poke` = (matrix, expert, row, col, value)
    sets one weight."""
    cfg = gen.config(0)
    G, U, D = gen.all_experts_host(cfg)
    sg, su, sd = gen.shared_host(cfg)
    G, U, sg, su = (_scaled_bits(m, k_gu) for m in (G, U, sg, su))
    D, sd = (_scaled_bits(m, k_down) for m in (D, sd))
    if poke is not None:
        m, e, i, j, v = poke
        {"gate": G, "up": U, "down": D}[m][e, i, j] = gen.f32_to_bf16_bits(np.float32([v]))[0]
    return Layer(cfg, experts=((G, U, D), (sg, su, sd)))


def test_prefill_f16_domain_near_the_bound():
    """Gate/up weights 128x the workload's (SwiGLU outputs up to ~2e4, routed
    down outputs up to ~4e3): the fp16 path still meets the bar against the
    oracle, no range flag, and agrees with the f32 decode path on the same
    rows (5 rows through the matrix cores, the first 4 through decode)."""
    lay = _scaled_tiny(7)
    x = _x(lay.cfg, 5, seed=131)
    out, lg, idx, w, st = lay.run(x, None, SCORE)
    assert st == 0
    check_forward(lay, x, None, SCORE, out, lg, idx, w)
    res = ref.forward(x, None, SCORE, lay.oracle_w, lay.cfg.top_k, lay.cfg.eps)
    h_max = 0.0
    for e in np.unique(res["idx"]):
        hh, _ = ref.expert_ffn(res["xn"], *lay.oracle_w.expert(e)[:3])
        h_max = max(h_max, float(np.abs(hh).max()))
    assert 1e4 < h_max < 65504, f"the scaled layer should approach fp16's range (max |h| {h_max:.3g})"
    out4 = lay.run(x[:4], None, SCORE)[0]
    check_output(out[:4], out4, what="prefill vs decode near the fp16 bound")


def test_prefill_f16_domain_beyond_the_bound():
    """Gate/up weights 1024x: some SwiGLU outputs exceed 65504.  The decode
    path (f32) still matches the oracle with no flag; the matrix-core path
    reports MOE_FLAG_F16_RANGE."""
    lay = _scaled_tiny(10)
    x = _x(lay.cfg, 8, seed=132)
    out4, lg, idx, w, st = lay.run(x[:4], None, SCORE)
    assert st == 0
    check_forward(lay, x[:4], None, SCORE, out4, lg, idx, w, rel=1e-5, maxabs=5e-5)
    out, lg, idx, w, st = lay.run(x, None, SCORE)
    assert st & moe.FLAG_F16_RANGE, f"status {st}: fp16 overflow not reported"


def test_prefill_f16_domain_weight_beyond_fp16():
    """One routed weight of 2^17 (a bf16 value fp16 cannot hold) in an
    expert every row uses: reported on the matrix-core path, exact on the
    decode path."""
    cfg = gen.config(0)
    plain = Layer(cfg)
    x = _x(cfg, 6, seed=133)
    idx0 = plain.run(x, None, SCORE)[2]
    e = int(np.bincount(idx0.reshape(-1)).argmax())
    lay = _scaled_tiny(0, poke=("gate", e, 3, 7, 2.0 ** 17))
    out, lg, idx, w, st = lay.run(x, None, SCORE)
    assert st & moe.FLAG_F16_RANGE
    out2, lg, idx, w, st = lay.run(x[:2], None, SCORE)
    assert st == 0
    check_forward(lay, x[:2], None, SCORE, out2, lg, idx, w, rel=1e-5, maxabs=5e-5)


def test_prefill_f16_domain_huge_norm_weight():
    """An RMSNorm weight of 1e6 makes a normalised input beyond fp16: the
    router logits are not finite and the flag is set."""
    cfg = gen.config(0)
    g = gen.host_inputs(cfg).norm_w.copy()
    g[11] = 1e6
    lay = Layer(cfg, norm_w=g)
    x = _x(cfg, 7, seed=134)
    st = lay.run(x, None, SCORE)[4]
    assert st & moe.FLAG_F16_RANGE


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
    tight = 1e-5 if rows <= 4 else 2e-3
    near = check_forward(full, x, None, SCORE, out, lg, idx, w, rel=tight, maxabs=tight * 5)
    report_near_ties(f"ragged {rows} rows", near, rows)


@pytest.mark.parametrize("pattern", ["adjacent", "strided"])
def test_full_exact_ties_in_forward(full, pattern):
    """Exact key ties at full size through the one-row, two-to-four-row and
    prefill (router sliced 8 ways) selectors."""
    lay, lead = tie_layer(full.cfg, pattern, share=full)
    for rows in (1, 3, 4, 40, 300):
        x = _x(lay.cfg, rows, seed=111 + rows)
        if rows >= 2:
            x[0] = 0.0
        out, lg, idx, w, st = lay.run(x, None, SCORE)
        assert st == 0
        tight = 1e-5 if rows <= 4 else 2e-3
        near = check_ties(lay, lead, x, out, lg, idx, w, tight, tight * 5)
        report_near_ties(f"ties {pattern} {rows} rows", near, rows)


@pytest.mark.parametrize("rows", [1500, 3000])
def test_full_prefill_router_slices(full, rows):
    """Batches whose router splits the experts over 4 (1500 rows) and 2 (3000
    rows) blocks per 32-row group, each with a ragged last group: every row
    end to end (logits, routing, output)."""
    cfg = full.cfg
    x = _x(cfg, rows, seed=70 + rows)
    out, lg, idx, w, st = full.run(x, None, SCORE)
    assert st == 0
    near = check_forward(full, x, None, SCORE, out, lg, idx, w)
    report_near_ties(f"router slices {rows} rows", near, rows)


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


def test_full_decode_one_row_table_edge_cases(full):
    cfg = gen.config(2)
    _one_row_table_edge_cases(Layer(cfg, share=full), _x(cfg, 1, seed=93))


def test_full_decode_one_row_every_valid_count(full):
    cfg = gen.config(2)
    _one_row_every_valid_count(Layer(cfg, share=full), _x(cfg, 1, seed=94))


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
    assert check_forward(lay, x, tok, HASH, out, lg, idx, w) == 0


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
    check_forward(lay, x, tok, HASH, out, lg, idx, w)


def test_full_prefill_config3(full):
    cfg = gen.config(3)
    lay = Layer(cfg, share=full)
    hi = lay.host
    out, lg, idx, w, st = lay.run(hi.x, None, SCORE)
    assert st == 0
    # every row: logits, routing exact, output
    near = check_forward(lay, hi.x, None, SCORE, out, lg, idx, w)
    report_near_ties(cfg.name, near, cfg.rows)


def test_full_prefill_skewed_config4(full):
    cfg = gen.config(4)
    lay = Layer(cfg, share=full)
    hi = lay.host
    out, lg, idx, w, st = lay.run(hi.x, None, SCORE)
    assert st == 0
    assert np.isin(idx, hi.hot).all(), "skewed bias should send every slot to a hot expert"
    # every row of the 8192 (49152 routed slots, 16 groups, the dynamically
    # dealt tail tiles included): logits, routing exact, output
    near = check_forward(lay, hi.x, None, SCORE, out, lg, idx, w)
    report_near_ties(cfg.name, near, cfg.rows)
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
