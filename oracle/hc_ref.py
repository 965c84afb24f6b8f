"""Float64 CPU oracle for the hyper-connection wrapper around the FFN layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library and imports nothing from it (the FFN in the middle is
``moe_ref.forward``).

``forward_ffn_rows`` on the docs.rs source page "hf2q 0.1.3 --
src/inference/models/deepseek4/ffn_forward.rs" (*ffn_forward.rs*) takes the
residual state as F32 ``[rows, hc, hidden]`` (hc = the model's
``hyper_connection_count``) and returns a new state of the same shape.  Around
the FFN it dispatches, in this order (the hyper-connection prelude, then the
post-mix after the weighted reduce):

  1. ``rms_norm_no_scale_f32`` over each row's flattened state
     ``[hc * hidden]``, with ``rms_norm_eps``;
  2. the "HC FFN function" ``raw_matmul`` with ``hc_ffn_fn`` into
     ``mixes [rows, (2 + hc) * hc]``;
  3. ``dispatch_hc_split_sinkhorn(mixes, hc_ffn_scale, hc_ffn_base)`` into
     ``pre [rows, hc]``, ``post [rows, hc]`` and ``comb [rows, hc, hc]``;
  4. ``dispatch_hc_pre(state, pre)`` into ``ffn_input [rows, hidden]``;
  5. the FFN of ``moe_ref.forward`` on ``ffn_input`` -> ``ffn_output``;
  6. ``dispatch_hc_post(ffn_output, state, post, comb)`` into the new state.

The page fixes those names, shapes, dtypes and the order, and prints none of
the arithmetic of steps 3, 4 and 6.  The readings below are the published
manifold-constrained hyper-connection formulation, whose three maps (a
pre-mix of the streams into the layer input, a post-mix of the layer output
back into the streams, and a doubly stochastic residual mix made by Sinkhorn
normalisation) match those names and shapes one for one:

  * ``rms_norm_no_scale``: ``v * (mean(v^2) + eps)^(-1/2)`` (no weight).
  * ``mixes = norm(state_flat) @ hc_fn^T``; mix columns ``[0, hc)`` are the
    pre logits, ``[hc, 2hc)`` the post logits, ``[2hc, (2+hc)hc)`` the comb
    logits in row-major (output stream j, input stream i) order.
  * ``hc_scale`` holds three scalars (pre, post, comb); ``hc_base`` one offset
    per mix column.
  * ``pre = sigmoid(s0 * m_pre + b_pre)``; ``post = 2 * sigmoid(s1 * m_post +
    b_post)``.
  * ``comb`` = Sinkhorn normalisation of ``exp(s2 * m_comb + b_comb)``:
    ``iters`` rounds, each dividing every row by its sum and then every
    column by its sum.
  * ``hc_pre``: ``ffn_input = sum_i pre_i * state_i``.
  * ``hc_post``: ``new_j = post_j * ffn_output + sum_i comb[j, i] * state_i``.

PARITY UNPINNED for steps 3, 4 and 6: the pages give neither a formula nor a
value for them, so the pins in tests/test_oracle_hc.py hold this code to the
readings above (closed forms of the Sinkhorn limit, conservation, special
cases, brute force), not to the pages.  Steps 1, 2 and the composition order
follow the page.
"""

from __future__ import annotations

import numpy as np

from oracle import moe_ref as ref

MIX_PRE, MIX_POST, MIX_COMB = 0, 1, 2  # indices into hc_scale


def mix_width(hc: int) -> int:
    """Mix columns of one row: pre (hc) + post (hc) + comb (hc * hc)."""
    return (2 + hc) * hc


def rms_norm_no_scale(v, eps: float) -> np.ndarray:
    """``rms_norm_no_scale_f32`` over the last axis: ``v / sqrt(mean(v^2) + eps)``."""
    v = np.asarray(v, dtype=np.float64)
    return v / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps)


def hc_mixes(state, hc_fn, eps: float) -> np.ndarray:
    """Steps 1-2: ``[rows, hc, hidden]`` state -> ``[rows, (2+hc)*hc]`` mixes.
    ``hc_fn`` is ``[(2+hc)*hc, hc*hidden]`` (bf16 bits or values)."""
    s = np.asarray(state, dtype=np.float64)
    flat = s.reshape(s.shape[0], -1)
    return rms_norm_no_scale(flat, eps) @ ref.weight_f64(hc_fn).T


def sigmoid(v) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-np.asarray(v, dtype=np.float64)))


def sinkhorn(m, iters: int) -> np.ndarray:
    """``iters`` rounds of row then column normalisation of the positive
    matrices ``m[..., j, i]``."""
    m = np.array(m, dtype=np.float64)
    for _ in range(iters):
        m = m / m.sum(axis=-1, keepdims=True)
        m = m / m.sum(axis=-2, keepdims=True)
    return m


def split_sinkhorn(mixes, hc_scale, hc_base, hc: int, iters: int):
    """Step 3: mixes -> (pre [rows, hc], post [rows, hc], comb [rows, hc, hc])."""
    m = np.asarray(mixes, dtype=np.float64)
    sc = np.asarray(hc_scale, dtype=np.float64)
    b = np.asarray(hc_base, dtype=np.float64)
    pre = sigmoid(sc[MIX_PRE] * m[:, :hc] + b[:hc])
    post = 2.0 * sigmoid(sc[MIX_POST] * m[:, hc:2 * hc] + b[hc:2 * hc])
    logits = sc[MIX_COMB] * m[:, 2 * hc:] + b[2 * hc:]
    comb = sinkhorn(np.exp(logits).reshape(-1, hc, hc), iters)
    return pre, post, comb


def hc_pre(state, pre) -> np.ndarray:
    """Step 4: ``ffn_input[r] = sum_i pre[r, i] * state[r, i]``."""
    return np.einsum("ri,rih->rh", np.asarray(pre, np.float64), np.asarray(state, np.float64))


def hc_post(ffn_output, state, post, comb) -> np.ndarray:
    """Step 6: ``new[r, j] = post[r, j] * ffn_output[r] + sum_i comb[r, j, i] * state[r, i]``."""
    f = np.asarray(ffn_output, np.float64)
    s = np.asarray(state, np.float64)
    return np.asarray(post, np.float64)[:, :, None] * f[:, None, :] + np.einsum("rji,rih->rjh", comb, s)


class HcWeights:
    """The wrapper's parameters: ``hc_fn`` ``[(2+hc)*hc, hc*hidden]`` (bf16
    bits), ``hc_scale`` ``[3]`` and ``hc_base`` ``[(2+hc)*hc]`` (f32), and the
    Sinkhorn round count."""

    def __init__(self, hc_fn, hc_scale, hc_base, hc: int, iters: int):
        self.hc_fn, self.hc_scale, self.hc_base = hc_fn, hc_scale, hc_base
        self.hc, self.iters = int(hc), int(iters)


def forward(state, token_ids, layer_kind: int, weights: ref.Weights, hw: HcWeights, top_k: int, eps: float):
    """The wrapped layer: ``[rows, hc, hidden]`` state in and out.  Returns a
    dict with every intermediate: ``mixes``, ``pre``, ``post``, ``comb``,
    ``ffn_input``, the FFN's dict under ``ffn``, and ``out``."""
    mixes = hc_mixes(state, hw.hc_fn, eps)
    pre, post, comb = split_sinkhorn(mixes, hw.hc_scale, hw.hc_base, hw.hc, hw.iters)
    x = hc_pre(state, pre)
    ffn = ref.forward(x, token_ids, layer_kind, weights, top_k, eps)
    out = hc_post(ffn["out"], state, post, comb)
    return {"mixes": mixes, "pre": pre, "post": post, "comb": comb, "ffn_input": x, "ffn": ffn, "out": out}
