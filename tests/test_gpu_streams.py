"""Calls on several streams at once, each with its own workspace, give the
outputs of the same calls made one at a time, bitwise: the library keeps
no state outside the workspace, and each call's cross-workgroup words live
in its own workspace.  The concurrent calls mix the one-row decode path,
the batched decode path and the prefill path."""

from __future__ import annotations

import numpy as np
import pytest

from mixture_experts_ffn_rmsnorm_amd import inputs as gen
from mixture_experts_ffn_rmsnorm_amd import moe
from tests.gpu_common import Layer

pytestmark = pytest.mark.gpu


def _run_concurrently(layer, cases, seed, reps):
    import torch

    cfg = layer.cfg
    rng = np.random.default_rng(seed)
    xs, toks, outs, wss = [], [], [], []
    for r, _ in cases:
        xs.append(torch.from_numpy(rng.standard_normal((r, cfg.hidden)).astype(np.float32)).cuda())
        toks.append(torch.from_numpy(rng.integers(0, cfg.table_rows, r).astype(np.int32)).cuda())
        wss.append(moe.alloc_workspace(layer.dims, r))
        outs.append(torch.empty((r, cfg.hidden), dtype=torch.float32, device="cuda"))
    # one at a time, on the current stream
    ref = []
    for (r, kind), x, tok, out, ws in zip(cases, xs, toks, outs, wss):
        moe.forward(layer.dims, x, tok, kind, layer.cw, out, ws)
        torch.cuda.synchronize()
        ref.append(out.clone())
    # all at once: each call on its own stream (default priority)
    streams = [torch.cuda.Stream() for _ in cases]
    for rep in range(reps):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        for (r, kind), x, tok, out, ws, st in zip(cases, xs, toks, outs, wss, streams):
            moe.forward(layer.dims, x, tok, kind, layer.cw, out, ws, stream=st)
        torch.cuda.synchronize()
        for case, o, e in zip(cases, outs, ref):
            assert torch.equal(o, e), f"rows/kind {case}, concurrent round {rep}"


def test_concurrent_streams_tiny():
    S, H = moe.LAYER_SCORE, moe.LAYER_HASH
    _run_concurrently(Layer(gen.config(0)), [(1, S), (1, H), (3, H), (4, S), (37, H), (300, S)], seed=31, reps=4)


def test_concurrent_streams_full_size():
    S, H = moe.LAYER_SCORE, moe.LAYER_HASH
    lay = Layer(gen.config(2))  # hash table present; score calls ignore it
    _run_concurrently(lay, [(1, S), (4, H), (1, H), (40, S)], seed=32, reps=2)
