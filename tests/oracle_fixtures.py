"""Helpers that assemble oracle inputs from the seeded generators and the
golden fixtures.  Test-side only."""

from __future__ import annotations

import os

import numpy as np

from mixture_experts_ffn_rmsnorm_amd import inputs as gen
from oracle import moe_ref as ref

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_golden(name: str) -> dict:
    """Parse a ``[section]`` / ``key: values`` text fixture (``#`` comments)."""
    out: dict = {}
    sec = None
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            if line.startswith("[") and line.endswith("]"):
                sec = out.setdefault(line[1:-1], {})
                continue
            k, v = line.split(":", 1)
            sec[k.strip()] = np.array([float(t) for t in v.split()], dtype=np.float64)
    return out


def micro_weights(g: dict):
    """Oracle weights of the micro example (values are exact in bf16)."""
    inp = g["inputs"]
    H, I, E = int(inp["hidden"][0]), int(inp["inter"][0]), int(inp["experts"][0])
    b16 = lambda a, shape: gen.f32_to_bf16_bits(np.asarray(a, np.float32).reshape(shape))
    experts = [(b16(inp[f"gate_e{e}"], (I, H)), b16(inp[f"up_e{e}"], (I, H)), b16(inp[f"down_e{e}"], (H, I)))
               for e in range(E)]
    shared = (b16(inp["gate_sh"], (I, H)), b16(inp["up_sh"], (I, H)), b16(inp["down_sh"], (H, I)))
    return ref.Weights(norm_w=inp["norm_w"].astype(np.float32), router=b16(inp["router"], (E, H)),
                       sel_bias=inp["sel_bias"].astype(np.float32), tid2eid=None,
                       expert=lambda e: experts[e], shared=shared)


def tiny_weights(cfg=None, layer: int = 0):
    cfg = cfg or gen.config(0)
    hi = gen.host_inputs(cfg, layer=layer)
    G, U, D = gen.all_experts_host(cfg, layer=layer)
    w = ref.Weights(norm_w=hi.norm_w, router=hi.router, sel_bias=hi.sel_bias, tid2eid=hi.tid2eid,
                    expert=lambda e: (G[e], U[e], D[e]), shared=gen.shared_host(cfg, layer=layer))
    return hi, w, (G, U, D)


def weights_from_arrays(norm_w, router, sel_bias, tid2eid, G, U, D, shared):
    return ref.Weights(norm_w=norm_w, router=router, sel_bias=sel_bias, tid2eid=tid2eid,
                       expert=lambda e: (G[e], U[e], D[e]), shared=shared)
