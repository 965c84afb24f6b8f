"""Float64 CPU oracle for the routed MoE FFN layer with RMSNorm.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library and imports nothing from it.

What it computes follows the dataflow of ``forward_ffn_rows`` on the docs.rs
source page "hf2q 0.1.3 -- src/inference/models/deepseek4/ffn_forward.rs"
(cited below as *ffn_forward.rs*).  The page is host code that dispatches GPU
ops by name; it names each step and its buffer shapes and dtypes but prints no
formula.  The arithmetic of each step is the plainest reading those names
support, written out here in float64:

  1. RMSNorm of the FFN input with ``ffn_norm.weight`` and ``rms_norm_eps``
     (the ``rms_norm`` call that produces ``ffn_norm``).
  2. Router logits ``ffn_norm @ ffn_gate_inp^T`` (the "MoE gate" matmul,
     F32 ``[rows, experts]``).
  3. Routing: either the score route (logits + ``exp_probs_b.bias``) or the
     hash route (logits + token ids + ``ffn_gate_tid2eid`` table), both giving
     I32 indices ``[rows, top_k]`` and F32 weights ``[rows, top_k]``.
  4. Index sanitising: I32 indices -> U32 "safe" indices used for the expert
     weight reads; the raw indices still go to the weighted reduce.
  5. Routed and shared gate/up projections, then SwiGLU ("routed gate",
     "routed up", "shared gate", "shared up", two ``deepseek_moe_swiglu``).
  6. Routed and shared down projections ("routed down", "shared down").
  7. Weighted reduce of the routed outputs plus the shared output
     (``deepseek_moe_weighted_reduce`` taking indices, weights, routed_down
     and shared_down).

Readings taken where the page is silent (each is listed with its reason in
the design notes of the repository):
  * RMSNorm is ``x * (mean(x^2) + eps)^(-1/2) * g`` (eps inside the root,
    multiply by ``g`` itself).
  * The score of expert e is ``sigmoid(logit_e)``; selection ranks the key
    ``sigmoid(logit_e) + bias_e`` (evaluated in float64) in descending order,
    equal keys going to the lower expert index; the routing weight of a
    chosen expert is its *unbiased* sigmoid score divided by the sum over the
    chosen set (no extra scaling factor).
  * The hash route takes the table row of the token id in table column order
    and weights those experts by their renormalised sigmoid scores (no bias).
  * An out-of-range table entry or token id makes the slot (or the whole
    row) invalid: its safe index is 0, it contributes nothing, and the
    remaining valid slots are renormalised among themselves.
  * SwiGLU is ``silu(gate) * up`` with ``silu(v) = v / (1 + exp(-v))``.
  * The shared expert is added with weight 1.
  * Weights are bf16 bit patterns, widened exactly to float64; every
    activation stays in float64.

Block-scaled weights: an expert matrix may be given as OCP MXFP8 codes and
scales, or OCP MXFP4 packed codes and scales, instead of bf16 bits;
``mx_dequant`` / ``mx4_dequant`` decode it exactly (FP8 E4M3, FP4 E2M1 and
E8M0 values are all exact in float64) and the layer is then computed the
same way.

Parity pins (tests/test_oracle_pins.py): brute-force top-k ranks and subset
enumeration, sum-to-one weights, hash == score when the table holds the score
route's choice, the closed form at x = 0, a hand-worked micro example
(tests/golden/micro_h2.txt), RMSNorm scale invariance and mean-square identity,
row independence, expert relabelling, identical experts, matmul against a
plain triple loop, bf16 widening of known bit patterns, and the MX decoders
against hand-derived codes (tests/golden/mx_codes.txt), against torch's
float8 E4M3 / E8M0 types for all 256 codes, and through a whole layer whose
MX weights hold the same values as a bf16 layer.
"""

from __future__ import annotations

import numpy as np

LAYER_SCORE = 0
LAYER_HASH = 1


# --------------------------------------------------------------------------
# dtype helpers
# --------------------------------------------------------------------------
def bf16_to_f64(bits) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) exactly to float64.

    bf16 is the upper half of an IEEE binary32, so shifting the 16 bits into
    the top of a 32-bit word gives the same value as a float32, which float64
    holds exactly.
    """
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# block-scaled 8-bit weights (OCP Microscaling "MXFP8": FP8 E4M3 elements,
# one E8M0 power-of-two scale per 32 consecutive elements of a row).  The
# FFN page binds its expert matrices as GGML-typed raw matrices without
# naming the type; the only MXFP8 on the pages (the attention page's
# activation fake-quant) uses blocks of 64.  Weights here follow the OCP
# layout: blocks of MX_BLOCK along the input dimension of each row.
# --------------------------------------------------------------------------
MX_BLOCK = 32


def e4m3_to_f64(codes) -> np.ndarray:
    """OCP FP8 E4M3 codes (uint8) -> float64.  Bit 7 is the sign, bits 6..3
    the exponent (bias 7), bits 2..0 the mantissa.  Exponent 0 encodes
    subnormals m/8 * 2^-6; exponent 15 with mantissa 7 is NaN; the format has
    no infinities (so 448 = 2^8 * 1.75 is the largest finite value)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign, ex, man = c >> 7, (c >> 3) & 15, c & 7
    mag = np.where(ex == 0, man / 8.0 * 2.0 ** -6, (1.0 + man / 8.0) * np.exp2(ex - 7.0))
    mag = np.where((ex == 15) & (man == 7), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


def e8m0_to_f64(scales) -> np.ndarray:
    """E8M0 scale codes (uint8) -> float64: 2^(s - 127); 255 is NaN."""
    s = np.asarray(scales, dtype=np.uint8).astype(np.int64)
    return np.where(s == 255, np.nan, np.exp2(s - 127.0))


def mx_dequant(codes, scales, block: int = MX_BLOCK) -> np.ndarray:
    """Decode an MX matrix exactly: ``w[..., o, i] = e4m3(codes[..., o, i]) *
    e8m0(scales[..., o, i // block])``."""
    v = e4m3_to_f64(codes)
    sc = e8m0_to_f64(scales)
    assert sc.shape[-1] * block == v.shape[-1], "one scale per block of the input dimension"
    return v * np.repeat(sc, block, axis=-1)


# OCP MXFP4: FP4 E2M1 elements packed two per byte (the element of the lower
# input index in the low nibble), one E8M0 scale per 32 elements as above.
def e2m1_to_f64(nibbles) -> np.ndarray:
    """OCP FP4 E2M1 codes (0..15) -> float64.  Bit 3 is the sign, bits 2..1
    the exponent (bias 1), bit 0 the mantissa: exponent 0 encodes the
    subnormals 0 and 0.5, so the magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6;
    the format has no infinities and no NaN."""
    c = np.asarray(nibbles, dtype=np.uint8).astype(np.int64)
    sign, ex, man = (c >> 3) & 1, (c >> 1) & 3, c & 1
    mag = np.where(ex == 0, man * 0.5, (1.0 + man / 2.0) * np.exp2(ex - 1.0))
    return np.where(sign == 1, -mag, mag)


def unpack_fp4(packed) -> np.ndarray:
    """Bytes ``[..., n/2]`` -> E2M1 codes ``[..., n]``: byte k holds elements
    2k (low nibble) and 2k + 1 (high nibble)."""
    b = np.asarray(packed, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = b & 15
    out[..., 1::2] = b >> 4
    return out


def mx4_dequant(packed, scales, block: int = MX_BLOCK) -> np.ndarray:
    """Decode an MXFP4 matrix exactly: ``w[..., o, i] = e2m1(code i of row o)
    * e8m0(scales[..., o, i // block])``."""
    v = e2m1_to_f64(unpack_fp4(packed))
    sc = e8m0_to_f64(scales)
    assert sc.shape[-1] * block == v.shape[-1], "one scale per block of the input dimension"
    return v * np.repeat(sc, block, axis=-1)


MXFP4 = "mxfp4"  # tag of a (packed codes, scales, MXFP4) weight tuple


def weight_f64(w) -> np.ndarray:
    """One weight matrix in float64: bf16 bit patterns (uint16) widened
    exactly, an MXFP8 matrix given as ``(codes, scales)`` or an MXFP4 one as
    ``(packed codes, scales, MXFP4)`` decoded exactly, or an array of values
    taken as they are."""
    if isinstance(w, tuple):
        if len(w) == 3 and w[2] == MXFP4:
            return mx4_dequant(w[0], w[1])
        return mx_dequant(*w)
    w = np.asarray(w)
    return bf16_to_f64(w) if w.dtype == np.uint16 else w.astype(np.float64)


# --------------------------------------------------------------------------
# step 1: RMSNorm  (ffn_forward.rs, forward_ffn_rows: rms_norm of the FFN
# input with ffn_norm.weight and the model's rms_norm_eps over `hidden`)
# --------------------------------------------------------------------------
def rms_norm(x, g, eps: float) -> np.ndarray:
    """``x[r, :] * (mean_j x[r, j]^2 + eps)^(-1/2) * g[:]`` in float64."""
    x = np.asarray(x, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + float(eps)) * g


# --------------------------------------------------------------------------
# step 2: router  (ffn_forward.rs, the "MoE gate" raw_matmul into F32 logits
# [rows, experts] from ffn_norm and ffn_gate_inp)
# --------------------------------------------------------------------------
def router_logits(xn, router_bits) -> np.ndarray:
    """``logits[r, e] = sum_j xn[r, j] * Wr[e, j]`` (Wr given as bf16 bits)."""
    return np.asarray(xn, dtype=np.float64) @ bf16_to_f64(router_bits).T


def sigmoid(v) -> np.ndarray:
    """``1 / (1 + exp(-v))`` in float64 (exp overflow gives exactly 0)."""
    v = np.asarray(v, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-v))


# --------------------------------------------------------------------------
# step 3a: score route  (ffn_forward.rs: deepseek_moe_score_route takes the
# logits and exp_probs_b.bias and writes I32 indices and F32 weights)
# --------------------------------------------------------------------------
def score_route(logits, bias, top_k: int):
    """Top-k by ``sigmoid(l) + b`` (desc, ties to lower index); weights are
    the chosen unbiased sigmoid scores renormalised to sum 1.

    Returns ``(idx int32 [R, K], w float64 [R, K], valid bool [R, K])``.
    """
    logits = np.atleast_2d(np.asarray(logits, dtype=np.float64))
    b = np.asarray(bias, dtype=np.float64)
    sig = sigmoid(logits)
    key = sig + b[None, :]
    rows, experts = key.shape
    idx = np.empty((rows, top_k), dtype=np.int32)
    w = np.empty((rows, top_k), dtype=np.float64)
    for r in range(rows):
        # stable sort of -key keeps equal keys in ascending expert order
        order = np.argsort(-key[r], kind="stable")[:top_k]
        idx[r] = order
        s = sig[r, order]
        w[r] = s / s.sum()
    return idx, w, np.ones((rows, top_k), dtype=bool)


# --------------------------------------------------------------------------
# step 3b: hash route  (ffn_forward.rs: deepseek_moe_hash_route takes the
# logits, the I32 token ids, the ffn_gate_tid2eid lookup and vocab_size)
# --------------------------------------------------------------------------
def hash_route(logits, token_ids, tid2eid, top_k: int):
    """Experts from the token's table row (column order); weights are the
    router sigmoid scores of those experts renormalised over the valid slots.

    A token id outside ``[0, table_rows)`` invalidates all of the row's
    slots; a table entry outside ``[0, experts)`` invalidates that slot.
    Invalid slots carry index -1 (bad token) or the raw entry (bad entry),
    weight 0 and ``valid = False``.
    """
    logits = np.atleast_2d(np.asarray(logits, dtype=np.float64))
    rows, experts = logits.shape
    table = np.asarray(tid2eid, dtype=np.int64)
    tok = np.asarray(token_ids, dtype=np.int64).reshape(-1)
    sig = sigmoid(logits)
    idx = np.full((rows, top_k), -1, dtype=np.int32)
    w = np.zeros((rows, top_k), dtype=np.float64)
    valid = np.zeros((rows, top_k), dtype=bool)
    for r in range(rows):
        t = int(tok[r])
        if t < 0 or t >= table.shape[0]:
            continue
        ent = table[t, :top_k]
        idx[r] = ent.astype(np.int32)
        ok = (ent >= 0) & (ent < experts)
        valid[r] = ok
        if ok.any():
            s = np.where(ok, sig[r, np.where(ok, ent, 0)], 0.0)
            w[r] = s / s.sum()
    return idx, w, valid


# --------------------------------------------------------------------------
# step 4: sanitise  (ffn_forward.rs: deepseek_moe_sanitize_indices turns the
# I32 indices into U32 safe indices for the indexed expert matmuls)
# --------------------------------------------------------------------------
def sanitize(idx, experts: int):
    """``safe = idx`` where ``0 <= idx < experts`` else 0; plus the mask."""
    idx = np.asarray(idx, dtype=np.int64)
    ok = (idx >= 0) & (idx < experts)
    return np.where(ok, idx, 0).astype(np.uint32), ok


# --------------------------------------------------------------------------
# steps 5-6: one expert  (ffn_forward.rs: expert_matmul / raw_matmul for
# gate and up with [inter, hidden] matrices, deepseek_moe_swiglu, then the
# down matmul with a [hidden, inter] matrix)
# --------------------------------------------------------------------------
def silu(v) -> np.ndarray:
    v = np.asarray(v, dtype=np.float64)
    return v * sigmoid(v)


def swiglu(gate, up) -> np.ndarray:
    """``silu(gate) * up``."""
    return silu(gate) * np.asarray(up, dtype=np.float64)


def expert_ffn(xn_rows, gate_bits, up_bits, down_bits):
    """One expert on a block of rows: ``down @ (silu(gate @ xn) * (up @ xn))``.

    ``gate_bits``/``up_bits`` are ``[inter, hidden]``, ``down_bits`` is
    ``[hidden, inter]`` (row-major [out][in]), each as bf16 bits or an MX
    ``(codes, scales)`` pair (see ``weight_f64``).  Returns ``(h, d)``.
    """
    xn_rows = np.asarray(xn_rows, dtype=np.float64)
    g = xn_rows @ weight_f64(gate_bits).T
    u = xn_rows @ weight_f64(up_bits).T
    h = swiglu(g, u)
    d = h @ weight_f64(down_bits).T
    return h, d


# --------------------------------------------------------------------------
# step 7 and the whole layer
# --------------------------------------------------------------------------
class Weights:
    """Host view of one layer's parameters.

    ``expert(e)`` returns ``(gate [I,H], up [I,H], down [H,I])`` of routed
    expert e, each bf16 bits or an MX ``(codes, scales)`` pair; it may fetch
    lazily, so a full-size layer need not be held in host memory.  ``shared``
    is the same triple for the shared expert.  The router is bf16 bits.
    """

    def __init__(self, norm_w, router, sel_bias, tid2eid, expert, shared):
        self.norm_w = np.asarray(norm_w, dtype=np.float32)
        self.router = np.asarray(router, dtype=np.uint16)
        self.sel_bias = None if sel_bias is None else np.asarray(sel_bias, dtype=np.float32)
        self.tid2eid = None if tid2eid is None else np.asarray(tid2eid, dtype=np.int32)
        self._expert = expert
        self.shared = shared

    def expert(self, e: int):
        return self._expert(int(e))


def route(logits, token_ids, layer_kind: int, weights: Weights, top_k: int):
    """Route rows from given logits by the layer's routing source."""
    if layer_kind == LAYER_HASH:
        if weights.tid2eid is None:
            raise ValueError("hash layer needs a tid2eid table")
        return hash_route(logits, token_ids, weights.tid2eid, top_k)
    if layer_kind == LAYER_SCORE:
        if weights.sel_bias is None:
            raise ValueError("score layer needs a selection bias")
        return score_route(logits, weights.sel_bias, top_k)
    raise ValueError(f"unknown layer kind {layer_kind}")


def forward_given_routing(xn, idx, w, valid, weights: Weights):
    """``out[r] = sum_k valid w[r,k] * d_{idx[r,k]}(xn[r]) + shared(xn[r])``.

    Routed outputs are computed expert by expert (rows gathered per expert)
    and summed per row in slot order k = 0..K-1, then the shared expert is
    added (weight 1).
    """
    xn = np.asarray(xn, dtype=np.float64)
    rows, top_k = np.asarray(idx).shape
    hidden = xn.shape[1]
    experts = weights.router.shape[0]
    safe, ok = sanitize(idx, experts)
    ok = ok & np.asarray(valid, dtype=bool)
    d_slot = np.zeros((rows, top_k, hidden), dtype=np.float64)
    for e in np.unique(safe[ok]):
        rr, kk = np.nonzero((safe == e) & ok)
        gate, up, down = weights.expert(int(e))
        _, d = expert_ffn(xn[rr], gate, up, down)
        d_slot[rr, kk] = d
    out = np.zeros((rows, hidden), dtype=np.float64)
    wv = np.where(ok, np.asarray(w, dtype=np.float64), 0.0)
    for k in range(top_k):
        out += wv[:, k:k + 1] * d_slot[:, k, :]
    _, ds = expert_ffn(xn, *weights.shared)
    return out + ds


def forward(x, token_ids, layer_kind: int, weights: Weights, top_k: int, eps: float):
    """The whole layer.  Returns a dict of every intermediate the GPU path
    exposes: ``xn``, ``logits``, ``idx``, ``w``, ``valid``, ``out``."""
    xn = rms_norm(x, weights.norm_w, eps)
    logits = router_logits(xn, weights.router)
    idx, w, valid = route(logits, token_ids, layer_kind, weights, top_k)
    out = forward_given_routing(xn, idx, w, valid, weights)
    return {"xn": xn, "logits": logits, "idx": idx, "w": w, "valid": valid, "out": out}
