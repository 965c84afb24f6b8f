"""Pins of the hyper-connection oracle (oracle/hc_ref.py) to its stated
readings: closed forms of the Sinkhorn limit, conservation, special cases and
brute force, each chosen so that a plausible slip in the oracle fails one of
them (the planted mistakes at the end).  The pages print no formula or value
for the split / pre / post steps, so these pin the oracle to its readings,
not to the pages (parity unpinned there)."""

from __future__ import annotations

import numpy as np
import pytest

from oracle import hc_ref as hcr
from oracle import moe_ref as ref
from mixture_experts_ffn_rmsnorm_amd import inputs as gen

ONE_BF16 = np.uint16(0x3F80)
_HC_POST = hcr.hc_post  # the unpatched post-mix, for the mutants built on it


def check_norm_hand_example():
    # v = (3, 4, 0, 0): mean square 25/4; with eps = 1 the divisor is sqrt(7.25)
    out = hcr.rms_norm_no_scale(np.array([[3.0, 4.0, 0.0, 0.0]]), 1.0)
    np.testing.assert_allclose(out, [[3 / np.sqrt(7.25), 4 / np.sqrt(7.25), 0, 0]], rtol=1e-15)
    out0 = hcr.rms_norm_no_scale(np.array([[3.0, 4.0, 0.0, 0.0]]), 0.0)
    np.testing.assert_allclose(out0, [[1.2, 1.6, 0, 0]], rtol=1e-15)


def check_norm_spans_all_streams():
    # a one-hot hc_fn row picks one flattened element; the divisor is the RMS
    # over all hc * hidden values of the row, not over its own stream
    rng = np.random.default_rng(1)
    hc, H = 3, 8
    state = rng.standard_normal((2, hc, H))
    fn = np.zeros((hcr.mix_width(hc), hc * H), np.uint16)
    fn[0, 5] = ONE_BF16          # stream 0, element 5
    fn[1, 2 * H + 7] = ONE_BF16  # stream 2, element 7
    m = hcr.hc_mixes(state, fn, 0.0)
    rms = np.sqrt(np.mean(state.reshape(2, -1) ** 2, axis=1))
    np.testing.assert_allclose(m[:, 0], state[:, 0, 5] / rms, rtol=1e-14)
    np.testing.assert_allclose(m[:, 1], state[:, 2, 7] / rms, rtol=1e-14)
    assert np.all(m[:, 2:] == 0)


def check_mixes_triple_loop():
    rng = np.random.default_rng(2)
    hc, H, R = 2, 5, 3
    state = rng.standard_normal((R, hc, H))
    fn = gen.f32_to_bf16_bits(rng.standard_normal((hcr.mix_width(hc), hc * H)))
    wf = ref.bf16_to_f64(fn)
    m = hcr.hc_mixes(state, fn, 1e-6)
    for r in range(R):
        flat = [state[r, i, h] for i in range(hc) for h in range(H)]
        ms = sum(v * v for v in flat) / len(flat)
        for c in range(hcr.mix_width(hc)):
            want = sum(flat[k] * wf[c, k] for k in range(len(flat))) / np.sqrt(ms + 1e-6)
            assert abs(m[r, c] - want) <= 1e-12 * (1 + abs(want))


def check_sinkhorn_2x2_limit():
    # The limit D1 M D2 of a positive 2x2 matrix is [[p, 1-p], [1-p, p]]; the
    # cross ratio m11 m22 / (m12 m21) is unchanged by diagonal scaling, so
    # p^2 / (1-p)^2 = ad / (bc): p = sqrt(ad) / (sqrt(ad) + sqrt(bc)).
    a, b, c, d = 3.0, 0.5, 2.0, 7.0
    p = np.sqrt(a * d) / (np.sqrt(a * d) + np.sqrt(b * c))
    got = hcr.sinkhorn(np.array([[[a, b], [c, d]]]), 200)[0]
    np.testing.assert_allclose(got, [[p, 1 - p], [1 - p, p]], atol=1e-13)


def check_sinkhorn_rank_one_is_uniform():
    # exp(a_j + b_i) is rank one: one round gives 1/hc everywhere
    hc = 4
    m = np.exp(np.add.outer(np.array([0.3, -1.0, 2.0, 0.5]), np.array([1.0, 0.0, -0.7, 0.2])))
    np.testing.assert_allclose(hcr.sinkhorn(m[None], 1)[0], np.full((hc, hc), 1 / hc), atol=1e-15)


def check_sinkhorn_round_order():
    # each round ends with the column step: columns sum to exactly one after
    # every round count, rows only in the limit
    m = np.exp(np.random.default_rng(3).standard_normal((5, 4, 4)) * 2)
    for it in (1, 2, 5):
        s = hcr.sinkhorn(m, it)
        np.testing.assert_allclose(s.sum(axis=-2), 1.0, atol=1e-14)
    assert np.abs(hcr.sinkhorn(m, 1).sum(axis=-1) - 1).max() > 1e-3
    np.testing.assert_allclose(hcr.sinkhorn(m, 300).sum(axis=-1), 1.0, atol=1e-12)


def check_sinkhorn_permutation_equivariant():
    m = np.exp(np.random.default_rng(4).standard_normal((4, 4)))
    p, q = [2, 0, 3, 1], [1, 3, 0, 2]
    np.testing.assert_allclose(hcr.sinkhorn(m[p][:, q][None], 7)[0], hcr.sinkhorn(m[None], 7)[0][p][:, q],
                               atol=1e-15)


def check_split_zero_scale():
    # scale 0: the maps come from the offsets alone; offsets 0 give
    # pre = 1/2, post = 1 and the uniform comb
    hc = 3
    m = np.random.default_rng(5).standard_normal((2, hcr.mix_width(hc)))
    pre, post, comb = hcr.split_sinkhorn(m, [0, 0, 0], np.zeros(hcr.mix_width(hc)), hc, 20)
    np.testing.assert_allclose(pre, 0.5, rtol=1e-15)
    np.testing.assert_allclose(post, 1.0, rtol=1e-15)
    np.testing.assert_allclose(comb, 1 / hc, rtol=1e-14)


def check_split_comb_from_exp_of_logits():
    # hc = 2, scale 0, comb offsets log(a, b, c, d): the 2x2 closed form above
    a, b, c, d = 3.0, 0.5, 2.0, 7.0
    base = np.concatenate([[0.1, -0.2, 0.3, 0.4], np.log([a, b, c, d])])
    _, _, comb = hcr.split_sinkhorn(np.zeros((1, 8)), [1, 1, 0], base, 2, 200)
    p = np.sqrt(a * d) / (np.sqrt(a * d) + np.sqrt(b * c))
    np.testing.assert_allclose(comb[0], [[p, 1 - p], [1 - p, p]], atol=1e-13)


def check_split_layout_and_post_mix():
    # pre logits +40, post logits -40, comb logit 40 at (j, (j+1) % hc):
    # pre ~ 1, post ~ 0, comb ~ the cyclic shift, so new_j = state_{j+1}
    hc, H = 4, 6
    m = np.zeros((1, hcr.mix_width(hc)))
    m[0, :hc] = 40.0
    m[0, hc:2 * hc] = -40.0
    for j in range(hc):
        m[0, 2 * hc + j * hc + (j + 1) % hc] = 40.0
    pre, post, comb = hcr.split_sinkhorn(m, [1, 1, 1], np.zeros(hcr.mix_width(hc)), hc, 20)
    np.testing.assert_allclose(pre, 1.0, atol=1e-15)
    np.testing.assert_allclose(post, 0.0, atol=1e-15)
    state = np.random.default_rng(6).standard_normal((1, hc, H))
    new = hcr.hc_post(np.ones((1, H)), state, post, comb)
    np.testing.assert_allclose(new[0], state[0][[(j + 1) % hc for j in range(hc)]], atol=1e-12)


def check_pre_one_hot_and_linear():
    state = np.random.default_rng(7).standard_normal((3, 4, 5))
    pre = np.zeros((3, 4))
    pre[np.arange(3), [2, 0, 3]] = 1.0
    np.testing.assert_allclose(hcr.hc_pre(state, pre), state[np.arange(3), [2, 0, 3]], rtol=0)
    w = np.random.default_rng(8).random((3, 4))
    np.testing.assert_allclose(hcr.hc_pre(state, w), sum(w[:, i, None] * state[:, i] for i in range(4)), rtol=1e-14)


def check_post_conserves_streams():
    # with comb columns summing to one (any round count), the streams' total
    # is (sum_j post_j) * ffn_output + the old total
    rng = np.random.default_rng(9)
    hc, H = 4, 7
    state = rng.standard_normal((2, hc, H))
    f = rng.standard_normal((2, H))
    post = rng.random((2, hc)) * 2
    comb = hcr.sinkhorn(np.exp(rng.standard_normal((2, hc, hc)) * 3), 1)
    new = hcr.hc_post(f, state, post, comb)
    np.testing.assert_allclose(new.sum(axis=1), post.sum(axis=1)[:, None] * f + state.sum(axis=1), atol=1e-12)


def check_hc1_wraps_the_ffn():
    # one stream: comb = [[1]], so new = post * FFN(pre * state) + state with
    # pre = sigmoid(s0 * m0 + b0), post = 2 sigmoid(s1 * m1 + b1)
    cfg = gen.config(0)
    hi = gen.host_inputs(cfg)
    G, U, D = gen.all_experts_host(cfg)
    w = ref.Weights(hi.norm_w, hi.router, hi.sel_bias, hi.tid2eid, lambda e: (G[e], U[e], D[e]), gen.shared_host(cfg))
    rng = np.random.default_rng(10)
    state = rng.standard_normal((3, 1, cfg.hidden))
    fn = gen.f32_to_bf16_bits(rng.standard_normal((3, cfg.hidden)) * 0.02)
    hw = hcr.HcWeights(fn, [0.7, 1.3, 2.0], [0.2, -0.1, 0.5], 1, 20)
    res = hcr.forward(state, None, ref.LAYER_SCORE, w, hw, cfg.top_k, cfg.eps)
    m = res["mixes"]
    pre = 1 / (1 + np.exp(-(0.7 * m[:, 0] + 0.2)))
    post = 2 / (1 + np.exp(-(1.3 * m[:, 1] - 0.1)))
    f = ref.forward(pre[:, None] * state[:, 0], None, ref.LAYER_SCORE, w, cfg.top_k, cfg.eps)["out"]
    np.testing.assert_allclose(res["comb"], 1.0, rtol=1e-15)
    np.testing.assert_allclose(res["out"][:, 0], post[:, None] * f + state[:, 0], rtol=1e-12, atol=1e-12)


ALL_CHECKS = [
    check_norm_hand_example, check_norm_spans_all_streams, check_mixes_triple_loop, check_sinkhorn_2x2_limit,
    check_sinkhorn_rank_one_is_uniform, check_sinkhorn_round_order, check_sinkhorn_permutation_equivariant,
    check_split_zero_scale, check_split_comb_from_exp_of_logits, check_split_layout_and_post_mix,
    check_pre_one_hot_and_linear, check_post_conserves_streams, check_hc1_wraps_the_ffn,
]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_hc_pin(check):
    check()


# ---- planted mistakes: each must fail at least one pin --------------------
def _mut_eps_outside(v, eps):
    v = np.asarray(v, np.float64)
    return v / (np.sqrt(np.mean(v * v, axis=-1, keepdims=True)) + eps)


def _mut_norm_per_stream(state, hc_fn, eps):
    s = np.asarray(state, np.float64)
    n = s / np.sqrt(np.mean(s * s, axis=-1, keepdims=True) + eps)
    return n.reshape(s.shape[0], -1) @ ref.weight_f64(hc_fn).T


def _mut_columns_first(m, iters):
    m = np.array(m, np.float64)
    for _ in range(iters):
        m = m / m.sum(axis=-2, keepdims=True)
        m = m / m.sum(axis=-1, keepdims=True)
    return m


def _split_with(pre_f, post_f, comb_f):
    def split(mixes, hc_scale, hc_base, hc, iters):
        m = np.asarray(mixes, np.float64)
        sc, b = np.asarray(hc_scale, np.float64), np.asarray(hc_base, np.float64)
        return (pre_f(sc, b, m, hc), post_f(sc, b, m, hc), comb_f(sc, b, m, hc, iters))
    return split


_pre_ok = lambda sc, b, m, hc: hcr.sigmoid(sc[0] * m[:, :hc] + b[:hc])
_post_ok = lambda sc, b, m, hc: 2 * hcr.sigmoid(sc[1] * m[:, hc:2 * hc] + b[hc:2 * hc])
_comb_ok = lambda sc, b, m, hc, it: hcr.sinkhorn(np.exp(sc[2] * m[:, 2 * hc:] + b[2 * hc:]).reshape(-1, hc, hc), it)

MUTANTS = {
    "norm_eps_outside_root": ("rms_norm_no_scale", _mut_eps_outside),
    "norm_per_stream": ("hc_mixes", _mut_norm_per_stream),
    "sinkhorn_columns_first": ("sinkhorn", _mut_columns_first),
    "post_without_factor_2": ("split_sinkhorn", _split_with(
        _pre_ok, lambda sc, b, m, hc: hcr.sigmoid(sc[1] * m[:, hc:2 * hc] + b[hc:2 * hc]), _comb_ok)),
    "pre_post_swapped": ("split_sinkhorn", _split_with(
        lambda sc, b, m, hc: hcr.sigmoid(sc[0] * m[:, hc:2 * hc] + b[hc:2 * hc]),
        lambda sc, b, m, hc: 2 * hcr.sigmoid(sc[1] * m[:, :hc] + b[:hc]), _comb_ok)),
    "comb_without_exp": ("split_sinkhorn", _split_with(
        _pre_ok, _post_ok,
        lambda sc, b, m, hc, it: hcr.sinkhorn(np.abs(sc[2] * m[:, 2 * hc:] + b[2 * hc:]).reshape(-1, hc, hc) + 1e-300,
                                              it))),
    "comb_transposed": ("hc_post", lambda f, s, post, comb: _HC_POST(f, s, post, np.swapaxes(comb, -1, -2))),
    "pre_mix_uses_post_order": ("hc_pre", lambda state, pre: np.einsum(
        "ri,rih->rh", np.asarray(pre)[:, ::-1], np.asarray(state, np.float64))),
    "post_mix_drops_residual": ("hc_post", lambda f, s, post, comb: np.asarray(post)[:, :, None] *
                                np.asarray(f)[:, None, :]),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_hc_pins_catch_planted_mistakes(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(hcr, attr, fn)
    failed = []
    for check in ALL_CHECKS:
        try:
            check()
        except Exception:  # an assertion or a shape error both count as caught
            failed.append(check.__name__)
    assert failed, f"planted mistake {name} passed every pin"
