"""Seeded synthetic inputs for the MoE FFN layer.

This module only draws random numbers and lays them out; it holds none of
the layer's arithmetic.  Both the HIP path and the float64 oracle receive
exactly the arrays made here.

Recipe (per tensor an independent stream):
  * Small tensors -- x, token ids, RMSNorm weight, router, selection bias,
    hash table, and every expert of the tiny layer -- come from numpy
    ``Generator(Philox(key=[seed, tensor_id << 32 | index]))`` on the host,
    so any process regenerates them bit for bit.
  * Full-size expert weights (256 experts x 3 matrices of 2048 x 4096, 12 GiB
    in bf16) come from torch's Philox generator on the target device, one
    ``manual_seed`` per (tensor, expert); the oracle receives host copies of
    the experts it needs.
  * Normal samples are drawn in float32, scaled by the stated standard
    deviation and rounded to bf16 with round-to-nearest-even.
  * Block-scaled (MXFP8) expert weights, the layer's second weight format:
    E4M3 codes of N(0,1) * 8 samples (rounded to E4M3 by torch) and one
    E8M0 scale per 32 inputs drawn from 2^-10, 2^-9, 2^-8, from torch's
    generator with one seed per (tensor, expert) as above.
  * Block-scaled 4-bit (MXFP4) expert weights: N(0, 1.5^2) samples rounded
    to the nearest E2M1 magnitude (0, 0.5, 1, 1.5, 2, 3, 4, 6; ties to the
    smaller), packed two per byte (lower input index in the low nibble), and
    one E8M0 scale per 32 inputs drawn from 2^-8, 2^-7, 2^-6 (weights of
    standard deviation 0.006-0.023), from torch's generator as above.
  * Hyper-connection wrapper (hc residual streams): the state is N(0,1) per
    stream (like x); hc_fn is bf16 N(0, 0.02) [(2+hc)*hc, hc*hidden] (mixes
    of standard deviation 0.02 * sqrt(hc*hidden), 2.6 at the full shape);
    hc_scale = (0.25, 0.25, 0.5); hc_base: pre and post offsets N(0, 0.5),
    comb offsets 2 on the diagonal plus N(0, 0.5) (a residual mix near the
    identity); 20 Sinkhorn rounds.
"""

from __future__ import annotations

import dataclasses

import numpy as np

LAYER_SCORE = 0
LAYER_HASH = 1

# tensor ids of the per-tensor streams
_T_X, _T_TOK, _T_NORM, _T_ROUTER, _T_BIAS, _T_TABLE, _T_HOT = 1, 2, 3, 4, 5, 6, 7
_T_GATE, _T_UP, _T_DOWN, _T_SGATE, _T_SUP, _T_SDOWN = 10, 11, 12, 13, 14, 15
_T_HC_STATE, _T_HC_FN, _T_HC_BASE = 40, 41, 42
HC_SCALE = (0.25, 0.25, 0.5)
HC_ITERS = 20


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    rows: int
    hidden: int
    experts: int
    top_k: int
    inter: int
    layer_kind: int
    router_std: float
    table_rows: int = 0          # hash table rows (token-id range)
    hot_experts: int = 0         # experts whose bias is exactly +hot_bias
    hot_bias: float = 2.0
    weight_std: float = 0.02
    bias_std: float = 0.1
    norm_std: float = 0.05
    eps: float = 1e-6
    seed: int = 1000             # activations and token ids
    param_seed: int = 1000       # layer parameters (shared by the full-size workloads)

    @property
    def routed_slots(self) -> int:
        return self.rows * self.top_k


def _cfg(i, **kw):
    # the four full-size workloads share one set of layer parameters
    return Config(seed=1000 + i, param_seed=1000 if i == 0 else 1001, **kw)


# The five workloads: tiny CPU-seconds layer; full-size decode (score route);
# the B=4 decode cohort on a hash layer; 512-row prefill; 8192-row prefill
# with 16 hot experts.
CONFIGS = [
    _cfg(0, name="tiny-h512-e32-r8-score", rows=8, hidden=512, experts=32, top_k=6,
         inter=256, layer_kind=LAYER_SCORE, router_std=1.0 / np.sqrt(512.0), table_rows=1024),
    _cfg(1, name="decode-r1-score", rows=1, hidden=4096, experts=256, top_k=6, inter=2048,
         layer_kind=LAYER_SCORE, router_std=1.0 / 64.0),
    _cfg(2, name="decode-cohort-r4-hash", rows=4, hidden=4096, experts=256, top_k=6,
         inter=2048, layer_kind=LAYER_HASH, router_std=1.0 / 64.0, table_rows=131072),
    _cfg(3, name="prefill-r512-score", rows=512, hidden=4096, experts=256, top_k=6,
         inter=2048, layer_kind=LAYER_SCORE, router_std=1.0 / 64.0, table_rows=131072),
    _cfg(4, name="prefill-r8192-score-skewed", rows=8192, hidden=4096, experts=256, top_k=6,
         inter=2048, layer_kind=LAYER_SCORE, router_std=1.0 / 64.0, table_rows=131072,
         hot_experts=16),
]


def config(i_or_name) -> Config:
    if isinstance(i_or_name, int):
        return CONFIGS[i_or_name]
    for c in CONFIGS:
        if c.name == i_or_name:
            return c
    raise KeyError(i_or_name)


def _rng(seed: int, tensor: int, index: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(key=[int(seed), (int(tensor) << 32) | int(index)]))


def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 to bf16 (round to nearest, ties to even); uint16 bits."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def _normal_bf16(seed, tensor, index, shape, std) -> np.ndarray:
    a = _rng(seed, tensor, index).standard_normal(shape, dtype=np.float32)
    a *= np.float32(std)
    return f32_to_bf16_bits(a)


@dataclasses.dataclass
class HostInputs:
    """Everything but the full-size expert weights, as numpy arrays."""
    x: np.ndarray            # f32 [rows, hidden]
    token_ids: np.ndarray    # i32 [rows]
    norm_w: np.ndarray       # f32 [hidden]
    router: np.ndarray       # bf16 bits [experts, hidden]
    sel_bias: np.ndarray     # f32 [experts]
    tid2eid: np.ndarray | None  # i32 [table_rows, top_k]
    hot: np.ndarray          # i32 [hot_experts]


def host_inputs(cfg: Config, layer: int = 0, rows: int | None = None) -> HostInputs:
    """Activations, token ids and the small per-layer parameters.

    ``layer`` selects an independent set of layer parameters (router, bias,
    norm weight, table) while x and token ids stay the same.
    """
    s = cfg.seed
    ls = cfg.param_seed + 7919 * layer
    R = cfg.rows if rows is None else rows
    x = _rng(s, _T_X).standard_normal((R, cfg.hidden), dtype=np.float32)
    tok = _rng(s, _T_TOK).integers(0, max(cfg.table_rows, 1), size=R, dtype=np.int64).astype(np.int32)
    norm_w = (1.0 + cfg.norm_std * _rng(ls, _T_NORM).standard_normal(cfg.hidden, dtype=np.float32)).astype(np.float32)
    router = _normal_bf16(ls, _T_ROUTER, 0, (cfg.experts, cfg.hidden), cfg.router_std)
    bias = (cfg.bias_std * _rng(ls, _T_BIAS).standard_normal(cfg.experts, dtype=np.float32)).astype(np.float32)
    hot = np.zeros(0, dtype=np.int32)
    if cfg.hot_experts:
        hot = np.sort(_rng(s + 7919 * layer, _T_HOT).choice(cfg.experts, cfg.hot_experts,
                                                              replace=False)).astype(np.int32)
        bias[hot] = np.float32(cfg.hot_bias)
    table = None
    if cfg.table_rows:
        table = distinct_table(ls, cfg.table_rows, cfg.experts, cfg.top_k)
    return HostInputs(x=x, token_ids=tok, norm_w=norm_w, router=router, sel_bias=bias,
                      tid2eid=table, hot=hot)


def distinct_table(seed: int, table_rows: int, experts: int, top_k: int) -> np.ndarray:
    """``table_rows`` rows of ``top_k`` distinct experts in random order."""
    out = np.empty((table_rows, top_k), dtype=np.int32)
    rng = _rng(seed, _T_TABLE)
    chunk = 8192
    for r0 in range(0, table_rows, chunk):
        n = min(chunk, table_rows - r0)
        keys = rng.random((n, experts), dtype=np.float32)
        part = np.argpartition(keys, top_k - 1, axis=1)[:, :top_k]
        order = np.argsort(np.take_along_axis(keys, part, axis=1), axis=1, kind="stable")
        out[r0:r0 + n] = np.take_along_axis(part, order, axis=1)
    return out


def expert_host(cfg: Config, e: int, layer: int = 0):
    """bf16 bits ``(gate [I,H], up [I,H], down [H,I])`` of routed expert e,
    drawn on the host (used for the tiny layer)."""
    ls = cfg.param_seed + 7919 * layer
    I, H = cfg.inter, cfg.hidden
    return (_normal_bf16(ls, _T_GATE, e, (I, H), cfg.weight_std),
            _normal_bf16(ls, _T_UP, e, (I, H), cfg.weight_std),
            _normal_bf16(ls, _T_DOWN, e, (H, I), cfg.weight_std))


def shared_host(cfg: Config, layer: int = 0):
    ls = cfg.param_seed + 7919 * layer
    I, H = cfg.inter, cfg.hidden
    return (_normal_bf16(ls, _T_SGATE, 0, (I, H), cfg.weight_std),
            _normal_bf16(ls, _T_SUP, 0, (I, H), cfg.weight_std),
            _normal_bf16(ls, _T_SDOWN, 0, (H, I), cfg.weight_std))


def all_experts_host(cfg: Config, layer: int = 0):
    """Stacked host arrays ``(gate [E,I,H], up [E,I,H], down [E,H,I])``."""
    trip = [expert_host(cfg, e, layer) for e in range(cfg.experts)]
    return tuple(np.stack([t[j] for t in trip]) for j in range(3))


def expert_weights_device(cfg: Config, device, layer: int = 0):
    """Full-size expert weights drawn directly on ``device`` with torch.

    Returns bf16 tensors ``gate [E,I,H], up [E,I,H], down [E,H,I]`` and the
    shared triple ``[I,H], [I,H], [H,I]``.  One generator seed per (tensor,
    expert) keeps every expert reproducible on its own.
    """
    import torch

    ls = cfg.param_seed + 7919 * layer
    I, H, E = cfg.inter, cfg.hidden, cfg.experts
    gen = torch.Generator(device=device)

    def fill(dst, tensor_id, e):
        gen.manual_seed((ls * 1_000_003 + tensor_id * 65_537 + e) & 0x7FFF_FFFF_FFFF_FFFF)
        tmp = torch.randn(dst.shape, generator=gen, device=device, dtype=torch.float32)
        tmp.mul_(cfg.weight_std)
        dst.copy_(tmp.to(torch.bfloat16))

    gate = torch.empty((E, I, H), dtype=torch.bfloat16, device=device)
    up = torch.empty((E, I, H), dtype=torch.bfloat16, device=device)
    down = torch.empty((E, H, I), dtype=torch.bfloat16, device=device)
    for e in range(E):
        fill(gate[e], _T_GATE, e)
        fill(up[e], _T_UP, e)
        fill(down[e], _T_DOWN, e)
    sg = torch.empty((I, H), dtype=torch.bfloat16, device=device)
    su = torch.empty((I, H), dtype=torch.bfloat16, device=device)
    sd = torch.empty((H, I), dtype=torch.bfloat16, device=device)
    fill(sg, _T_SGATE, 0)
    fill(su, _T_SUP, 0)
    fill(sd, _T_SDOWN, 0)
    return (gate, up, down), (sg, su, sd)


# --------------------------------------------------------------------------
# block-scaled 8-bit expert weights (OCP MXFP8: E4M3 codes, one E8M0 scale
# per MX_BLOCK elements along the input dimension)
# --------------------------------------------------------------------------
MX_BLOCK = 32
_T_MX = 20  # tensor-id offset of the MX weight streams


def _mx_matrix(gen, out, inn, device):
    """Codes: N(0,1) * 8 (within E4M3's +-448) rounded to E4M3 by torch;
    scales: 2^-10, 2^-9 or 2^-8 per block, so the weights have a standard
    deviation of 0.008-0.03 like the bf16 workloads' 0.02."""
    import torch

    v = torch.randn((out, inn), generator=gen, device=device, dtype=torch.float32).mul_(8.0).clamp_(-448.0, 448.0)
    codes = v.to(torch.float8_e4m3fn).view(torch.uint8)
    sc = torch.randint(117, 120, (out, inn // MX_BLOCK), generator=gen, device=device, dtype=torch.int32)
    return codes, sc.to(torch.uint8)


def mx_expert_weights(cfg: Config, device, layer: int = 0):
    """MXFP8 expert weights drawn on ``device`` (host for ``"cpu"``): returns
    ``(gate, up, down)`` and the shared ``(gate, up, down)``, each matrix a
    ``(codes uint8 [..., out, in], scales uint8 [..., out, in/32])`` pair of
    torch tensors (routed: a leading expert dimension).  One generator seed
    per (tensor, expert)."""
    import torch

    ls = cfg.param_seed + 7919 * layer
    I, H, E = cfg.inter, cfg.hidden, cfg.experts
    gen = torch.Generator(device=device)

    def mat(tensor_id, e, out, inn):
        gen.manual_seed((ls * 1_000_003 + (_T_MX + tensor_id) * 65_537 + e) & 0x7FFF_FFFF_FFFF_FFFF)
        return _mx_matrix(gen, out, inn, device)

    def stack(tensor_id, out, inn):
        q = torch.empty((E, out, inn), dtype=torch.uint8, device=device)
        s = torch.empty((E, out, inn // MX_BLOCK), dtype=torch.uint8, device=device)
        for e in range(E):
            q[e], s[e] = mat(tensor_id, e, out, inn)
        return q, s

    routed = (stack(_T_GATE, I, H), stack(_T_UP, I, H), stack(_T_DOWN, H, I))
    shared = (mat(_T_SGATE, 0, I, H), mat(_T_SUP, 0, I, H), mat(_T_SDOWN, 0, H, I))
    return routed, shared


_T_MX4 = 30
_E2M1_MAG = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def _mx4_matrix(gen, out, inn, device):
    """Packed E2M1 codes [out, inn/2] and E8M0 scales [out, inn/32]."""
    import torch

    v = torch.randn((out, inn), generator=gen, device=device, dtype=torch.float32).mul_(1.5)
    mag = torch.tensor(_E2M1_MAG, device=device, dtype=torch.float32)
    idx = (v.abs().unsqueeze(-1) - mag).abs().argmin(dim=-1).to(torch.uint8)  # first minimum: ties to the smaller
    codes = idx | ((v < 0).to(torch.uint8) << 3)
    packed = codes[:, 0::2] | (codes[:, 1::2] << 4)
    sc = torch.randint(119, 122, (out, inn // MX_BLOCK), generator=gen, device=device, dtype=torch.int32)
    return packed.contiguous(), sc.to(torch.uint8)


def mx4_expert_weights(cfg: Config, device, layer: int = 0):
    """MXFP4 expert weights drawn on ``device``: ``(gate, up, down)`` and the
    shared ``(gate, up, down)``, each a ``(packed codes uint8 [..., out,
    in/2], scales uint8 [..., out, in/32])`` pair (routed: a leading expert
    dimension).  One generator seed per (tensor, expert)."""
    import torch

    ls = cfg.param_seed + 7919 * layer
    I, H, E = cfg.inter, cfg.hidden, cfg.experts
    gen = torch.Generator(device=device)

    def mat(tensor_id, e, out, inn):
        gen.manual_seed((ls * 1_000_003 + (_T_MX4 + tensor_id) * 65_537 + e) & 0x7FFF_FFFF_FFFF_FFFF)
        return _mx4_matrix(gen, out, inn, device)

    def stack(tensor_id, out, inn):
        q = torch.empty((E, out, inn // 2), dtype=torch.uint8, device=device)
        s = torch.empty((E, out, inn // MX_BLOCK), dtype=torch.uint8, device=device)
        for e in range(E):
            q[e], s[e] = mat(tensor_id, e, out, inn)
        return q, s

    routed = (stack(_T_GATE, I, H), stack(_T_UP, I, H), stack(_T_DOWN, H, I))
    shared = (mat(_T_SGATE, 0, I, H), mat(_T_SUP, 0, I, H), mat(_T_SDOWN, 0, H, I))
    return routed, shared


def mx_host(pair):
    """Host numpy copy ``(codes, scales)`` of one MX matrix (or one expert's
    slice of a stacked one)."""
    q, s = pair
    return q.detach().contiguous().cpu().numpy(), s.detach().contiguous().cpu().numpy()


def bf16_tensor_bits(t) -> np.ndarray:
    """Host uint16 copy of a bf16 torch tensor's bits."""
    import torch

    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@dataclasses.dataclass
class HcInputs:
    """The hyper-connection wrapper's state and parameters, numpy."""
    state: np.ndarray     # f32 [rows, hc, hidden]
    hc_fn: np.ndarray     # bf16 bits [(2+hc)*hc, hc*hidden]
    hc_scale: np.ndarray  # f32 [3]
    hc_base: np.ndarray   # f32 [(2+hc)*hc]
    hc: int
    iters: int


def hc_inputs(cfg: Config, hc: int = 4, layer: int = 0, rows: int | None = None) -> HcInputs:
    """Seeded state and wrapper parameters (recipe in the module docstring)."""
    ls = cfg.param_seed + 7919 * layer
    R = cfg.rows if rows is None else rows
    mw = (2 + hc) * hc
    state = _rng(cfg.seed, _T_HC_STATE, hc).standard_normal((R, hc, cfg.hidden), dtype=np.float32)
    fn = _normal_bf16(ls, _T_HC_FN, hc, (mw, hc * cfg.hidden), 0.02)
    base = (0.5 * _rng(ls, _T_HC_BASE, hc).standard_normal(mw, dtype=np.float32)).astype(np.float32)
    base[2 * hc:] += (2.0 * np.eye(hc, dtype=np.float32)).reshape(-1)
    return HcInputs(state=state, hc_fn=fn, hc_scale=np.array(HC_SCALE, dtype=np.float32), hc_base=base, hc=hc,
                    iters=HC_ITERS)
