#!/usr/bin/env python3
"""Throughput of the routed MoE FFN layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--only] [--layers L] [--graph]

A step is one moe_ffn_forward call (RMSNorm, router, routing, sort, gate/up +
SwiGLU, down, weighted reduce + shared expert) over one batch of synthetic
rows with every input already in HBM.  Steps cycle over L independently drawn
layers of weights (4 for decode, 1 for prefill) on one workspace, so that a
decode step never finds the previous step's experts in the 256 MB Infinity
Cache.  Kernel durations come from HIP start/stop events the library records
at each kernel's own start and end; the dominant kernel is reported against
the MI355X roofline.

The headline (`value`, `roofline`, ...) is the named workload, by default the
one-row score-routed decode.  Unless --only is given, the same JSON line also
carries `workloads`: one record per other full-size workload (the 4-row hash
cohort, 512-row prefill, 8192-row skewed prefill) with its rows/s, dominant
kernel roofline, step fractions and per-kernel timings, and its float64
oracle run over the whole batch with the GPU's agreement on every row.  The
headline's `cpu_baseline` times the oracle on a bounded sample beside it.

Prints one JSON line on stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer rows/sec at 1/4/512/8192 rows; HBM GB/s and MFMA % of peak"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16/bf16 matrix cores
# bytes per expert weight: bf16, or an MXFP8 code plus 1/32 of its block's E8M0 scale
WEIGHT_BYTES = {"bf16": 2.0, "mxfp8": 1.0 + 1.0 / 32, "mxfp4": 0.5 + 1.0 / 32}
EXPERT_BYTES = lambda H, I, wb=2.0: 3 * H * I * wb  # gate + up + down


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def alg_bytes(kernel, cfg, U, R, hc=4):
    """Algorithmic HBM bytes of one launch: every touched weight once, plus
    activations in and out (U = distinct routed experts of the step; a
    routed (expert, row) pair per slot, R*K of them).  Launch names ending in
    "_mx" read MXFP8 expert weights (the router stays bf16)."""
    H, I, E, K = cfg.hidden, cfg.inter, cfg.experts, cfg.top_k
    wb = WEIGHT_BYTES["bf16"]
    if kernel.endswith("_mx4"):
        kernel, wb = kernel[:-4], WEIGHT_BYTES["mxfp4"]
    elif kernel.endswith("_mx"):
        kernel, wb = kernel[:-3], WEIGHT_BYTES["mxfp8"]
    x = R * H * 4
    S = R * K
    if kernel == "dec_head":         # router + routing plan + shared gate/up
        return E * H * 2 + 2 * I * H * wb + 2 * x + H * 4 + R * E * 12 + R * (H + I) * 4
    if kernel == "dec_gateup":       # shared down + routed gate/up
        return H * I * wb + U * 2 * I * H * wb + R * (I + H) * 4 + R * K * (H + I) * 4
    if kernel == "dec_down":         # routed down: h in, per-entry partials out
        return U * H * I * wb + R * K * (I + H) * 4
    if kernel == "dec_reduce":       # partials and shared down in, out
        return R * K * H * 4 + R * H * 4 + x
    if kernel == "dec1_router":      # one-row path: router, logits + keys + sigmoids + xn out
        return E * H * 2 + x + H * 4 + R * E * 4 + R * H * 4 + R * E * 16
    if kernel == "dec1_gateup":      # shared + routed gate/up, routing from the keys
        return (U + 1) * 2 * I * H * wb + R * E * 16 + R * H * 4 + (R * K + R) * I * 4 + R * K * 12
    if kernel == "dec1_down_reduce":  # routed + shared down + weighted reduce, formed in place
        return (U + 1) * H * I * wb + (R * K + R) * I * 4 + R * H * 4
    if kernel == "pre_norm":         # x in, xn16 + xlo16 out
        return x + 2 * R * H * 2
    if kernel == "pre_router":       # xn16 + xlo16 in, logits + routing out, router weights once
        return E * H * 2 + 2 * R * H * 2 + R * E * 4 + S * 12
    if kernel == "pre_sort":         # row masks in; row lists, slot ranks and counts out
        return E * ((R + 31) // 32) * 4 + S * 4 * 2 + (E + 1) * 4
    if kernel == "gemm_gateup_swiglu":
        return (U + 1) * 2 * I * H * wb + (S + R) * H * 2 + (S + R) * I * 2
    if kernel == "gemm_down":        # routed experts: h16 in, d16 out
        return U * H * I * wb + S * I * 2 + S * H * 2
    if kernel == "gemm_down_shared_reduce":  # shared expert + weighted reduce of d16
        return H * I * wb + R * I * 2 + S * H * 2 + R * H * 4 + S * 12
    mw = (2 + hc) * hc  # hyper-connection wrapper: hc streams of H per row
    if kernel == "hc_mix":           # state in, hc_fn once, partial sums out
        return R * hc * H * 4 + mw * hc * H * 2 + R * (mw + 1) * 4 * ((hc * H + 1023) // 1024)
    if kernel == "hc_pre":           # partial sums and state in; mixes, maps, FFN input out
        return R * (mw + 1) * 4 * ((hc * H + 1023) // 1024) + R * hc * H * 4 + 2 * R * mw * 4 + R * H * 4
    if kernel == "hc_post":          # state, maps and FFN output in; new state out
        return 2 * R * hc * H * 4 + R * mw * 4 + R * H * 4
    return None


def alg_flops(kernel, cfg, R):
    kernel = kernel[:-4] if kernel.endswith("_mx4") else kernel[:-3] if kernel.endswith("_mx") else kernel
    H, I, E, K = cfg.hidden, cfg.inter, cfg.experts, cfg.top_k
    S = R * K
    if kernel == "pre_router":       # hi and lo passes
        return 2 * 2 * R * E * H
    if kernel == "gemm_gateup_swiglu":
        return 2 * (S + R) * 2 * I * H
    if kernel == "gemm_down":
        return 2 * S * H * I
    if kernel == "gemm_down_shared_reduce":
        return 2 * R * H * I
    return None


def step_flops(cfg, R):
    """Algorithmic flops of one layer call: the router plus 7 expert units
    (6 routed slots and the shared expert) of 2*3*H*I per row."""
    H, I, E, K = cfg.hidden, cfg.inter, cfg.experts, cfg.top_k
    return R * (2 * E * H + (K + 1) * 2 * 3 * H * I)


def step_bytes(cfg, U, R, fmt="bf16"):
    H, I, E = cfg.hidden, cfg.inter, cfg.experts
    return (U + 1) * EXPERT_BYTES(H, I, WEIGHT_BYTES[fmt]) + E * H * 2 + 2 * R * H * 4 + H * 4 + E * 4


# the hyper-connection-wrapped layer (moe_ffn_forward_hc, hc streams), bf16
HC_WORKLOADS = ("decode-r1-score", "prefill-r512-score")
HC_STREAMS = 4

SUB_WORKLOADS = ("decode-cohort-r4-hash", "prefill-r512-score", "prefill-r8192-score-skewed")
# the same workloads with MXFP8 expert weights (moe_ffn_forward_mxfp8)
MX_WORKLOADS = ("decode-r1-score", "decode-cohort-r4-hash", "prefill-r512-score", "prefill-r8192-score-skewed")
# and with MXFP4 expert weights (moe_ffn_forward_mxfp4)
MX4_WORKLOADS = ("decode-r1-score", "decode-cohort-r4-hash", "prefill-r512-score", "prefill-r8192-score-skewed")


def draw_layers(cfg, L):
    """Device expert weights of L independently drawn layers (the full-size
    workloads share one parameter seed, so one set serves all of them)."""
    from mixture_experts_ffn_rmsnorm_amd import inputs as gen

    out = []
    for l in range(L):
        out.append(gen.expert_weights_device(cfg, "cuda", layer=l))
        log(f"layer {l} weights ready")
    return out


def draw_layers_mx(cfg, L, fmt="mxfp8"):
    """Device block-scaled expert weights of L layers ((codes, scales) per
    matrix; MXFP8 codes, or MXFP4 codes packed two per byte)."""
    from mixture_experts_ffn_rmsnorm_amd import inputs as gen

    draw = gen.mx4_expert_weights if fmt == "mxfp4" else gen.mx_expert_weights
    out = []
    for l in range(L):
        out.append(draw(cfg, "cuda", layer=l))
        log(f"layer {l} {fmt.upper()} weights ready")
    return out


def bind_layers(cfg, big, L, fmt="bf16"):
    """Per workload: small per-layer parameters (router, bias with the hot
    experts, norm weight, table) on the device, bound with the big weights.
    Each layer is (host inputs, kept tensors, C weight struct, format)."""
    import numpy as np
    import torch

    from mixture_experts_ffn_rmsnorm_amd import inputs as gen
    from mixture_experts_ffn_rmsnorm_amd import moe

    layers = []
    for l in range(L):
        hi = gen.host_inputs(cfg, layer=l)
        (g, u, d), (gs, us, ds) = big[l]
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        keep = [t(hi.norm_w), t(hi.router.view(np.int16)).view(torch.bfloat16), t(hi.sel_bias),
                t(hi.tid2eid) if hi.tid2eid is not None else None, g, u, d, gs, us, ds]
        cw = moe.make_weights(*keep) if fmt == "bf16" else moe.make_mx_weights(*keep)
        layers.append((hi, keep, cw, fmt))
    return layers


def forward_fn(fmt):
    from mixture_experts_ffn_rmsnorm_amd import moe

    return {"bf16": moe.forward, "mxfp8": moe.forward_mxfp8, "mxfp4": moe.forward_mxfp4}[fmt]


def time_workload(cfg, layers, steps, warmup, graph=False):
    """One workload on the device: throughput, per-kernel event timings and
    their rooflines, latency, and layer 0's output for the parity check."""
    import numpy as np
    import torch

    from mixture_experts_ffn_rmsnorm_amd import moe

    R = cfg.rows
    L = len(layers)
    dims = moe.dims_of(cfg)
    hi0 = layers[0][0]
    x = torch.from_numpy(hi0.x).cuda()
    tok = torch.from_numpy(hi0.token_ids).cuda()
    out = torch.empty_like(x)
    ws = moe.alloc_workspace(dims, R)  # one workspace for every layer, as a model runs them
    torch.cuda.synchronize()

    fmt = layers[0][3]
    fwd = forward_fn(fmt)

    def step(i):
        fwd(dims, x, tok, cfg.layer_kind, layers[i % L][2], out, ws)

    log(f"{cfg.name}: warmup {warmup}")
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    U = []  # distinct routed experts of each layer's step, from its routing
    for l in range(L):
        step(l)
        torch.cuda.synchronize()
        idx = moe.routing_view(dims, R, ws)[1].cpu().numpy()
        U.append(len(np.unique(idx[(idx >= 0) & (idx < cfg.experts)])))
    log(f"{cfg.name}: distinct routed experts per layer {U}; timing {steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / steps
    u_mean = float(np.mean([U[i % L] for i in range(steps)]))
    # kernel pass: each kernel bracketed by HIP events taken at its own start
    # and end, on the stream it runs on
    moe.stage_timing_begin()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    stages = moe.stage_timing_end()
    # latency pass: each step between events on the launch stream
    lat = []
    for i in range(steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        step(i)
        e1.record()
        lat.append((e0, e1))
    torch.cuda.synchronize()
    lat_us = np.array([a.elapsed_time(b) * 1e3 for a, b in lat])

    kernels = {}
    for name, (ms, n) in stages.items():
        kernels[name] = {"avg_us": ms * 1e3 / n, "launches": n}
    dom = max(stages, key=lambda k: stages[k][0])
    avg_s = stages[dom][0] / stages[dom][1] / 1e3
    flops = alg_flops(dom, cfg, R)
    b = alg_bytes(dom, cfg, u_mean, R)
    if b is None and flops is None:  # a kernel this accounting does not know
        roof = {"kernel": dom, "bound": None, "achieved": None, "peak": None, "unit": None, "frac": None,
                "traffic": None}
    elif flops is not None and (b is None or flops / (MFMA_F16_PEAK_TFLOPS * 1e12) > b / (HBM_PEAK_GBPS * 1e9)):
        ach = flops / avg_s / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": ach, "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": ach / MFMA_F16_PEAK_TFLOPS, "traffic": None}
    else:
        ach = b / avg_s / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": ach / HBM_PEAK_GBPS, "traffic": None}
    # HBM bytes per launch of the dominant kernel, from the committed counter
    # summary of the same workload, if it was measured on these sources
    from mixture_experts_ffn_rmsnorm_amd import profiling

    measured = profiling.read_traffic(profiling.profile_key(cfg.name, layers[0][3]))
    if measured and dom in measured:
        roof["traffic"] = measured[dom]
    launch_bytes = []  # algorithmic bytes of each launch of a step
    for name, k in kernels.items():
        kb, kf = alg_bytes(name, cfg, u_mean, R), alg_flops(name, cfg, R)
        if kb is not None:
            launch_bytes += [kb] * max(1, round(k["launches"] / steps))
        secs = k["avg_us"] * 1e-6
        if kb is not None:
            k["hbm_frac"] = kb / secs / 1e9 / HBM_PEAK_GBPS
        if kf is not None:
            k["mfma_frac"] = kf / secs / 1e12 / MFMA_F16_PEAK_TFLOPS
    sb, sf = step_bytes(cfg, u_mean, R, fmt), step_flops(cfg, R)
    step_s = ms_per_step / 1e3
    rec = {
        "rows": R, "rows_per_s": R / step_s, "ms_per_step": ms_per_step, "layers_cycled": L, "weights": fmt,
        "distinct_routed_experts": u_mean,
        "latency_us": {"median": float(np.median(lat_us)), "p10": float(np.percentile(lat_us, 10)),
                       "p90": float(np.percentile(lat_us, 90))},
        "step_alg_bytes": sb, "step_hbm_GBps": sb / step_s / 1e9, "step_hbm_frac": sb / step_s / 1e9 / HBM_PEAK_GBPS,
        "step_alg_flops": sf, "step_TFLOPs": sf / step_s / 1e12,
        "step_mfma_frac": sf / step_s / 1e12 / MFMA_F16_PEAK_TFLOPS,
        "roofline": roof, "kernels": kernels, "launch_bytes": launch_bytes,
    }
    if graph:
        rec["graph"] = graph_chain(dims, cfg, layers, x, tok, ws, steps, ms_per_step)
    # one call of layer 0 for the parity check and the status word
    fwd(dims, x, tok, cfg.layer_kind, layers[0][2], out, ws)
    torch.cuda.synchronize()
    rec["status_flags"] = moe.status(ws)
    gpu0 = (out.cpu().numpy(), moe.routing_view(dims, R, ws)[1].cpu().numpy())
    del x, tok, out, ws
    return rec, gpu0


def time_hc(cfg, layers, hc, steps, warmup, ffn_ms):
    """The wrapped layer (moe_ffn_forward_hc) on the same layers: time per
    step, the wrapper's kernels against their algorithmic bytes, and what
    the wrapper adds to the bare layer's step."""
    import numpy as np
    import torch

    from mixture_experts_ffn_rmsnorm_amd import inputs as gen
    from mixture_experts_ffn_rmsnorm_amd import moe

    R, L = cfg.rows, len(layers)
    dims = moe.dims_of(cfg)
    h = gen.hc_inputs(cfg, hc)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    fn = t(h.hc_fn.view(np.int16)).view(torch.bfloat16)
    sc, base = t(h.hc_scale), t(h.hc_base)
    hw = moe.make_hc_weights(fn, sc, base, hc, h.iters)
    state = t(h.state)
    tok = t(layers[0][0].token_ids)
    out = torch.empty_like(state)
    ws = moe.alloc_hc_workspace(dims, hc, R)

    def step(i):
        moe.forward_hc(dims, state, tok, cfg.layer_kind, layers[i % L][2], hw, out, ws)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    moe.stage_timing_begin()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    stages = moe.stage_timing_end()
    kernels = {}
    for name, (kms, n) in stages.items():
        k = {"avg_us": kms * 1e3 / n, "launches": n}
        if name.startswith("hc_"):
            b = alg_bytes(name, cfg, 0, R, hc)
            k["alg_bytes"] = b
            k["hbm_frac"] = b / (k["avg_us"] * 1e-6) / 1e9 / HBM_PEAK_GBPS
        kernels[name] = k
    wrapper_us = sum(k["avg_us"] for n, k in kernels.items() if n.startswith("hc_"))
    log(f"{cfg.name} hc{hc}: {ms * 1e3:.1f} us per step ({ffn_ms * 1e3:.1f} bare), wrapper kernels {wrapper_us:.1f} us")
    del state, out, ws
    return {"rows": R, "hc": hc, "rows_per_s": R / (ms / 1e3), "ms_per_step": ms, "bare_ms_per_step": ffn_ms,
            "added_us_per_step": (ms - ffn_ms) * 1e3, "wrapper_kernels_us": wrapper_us, "kernels": kernels,
            "dtype": "f32" if R <= 4 else "f16", "weights": "bf16"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode-r1-score")
    ap.add_argument("--only", action="store_true",
                    help="time the named workload alone (no sub-records of the other full-size workloads)")
    ap.add_argument("--layers", type=int, default=None, help="distinct weight sets cycled (default 4 decode, 1 prefill)")
    ap.add_argument("--weights", choices=("bf16", "mxfp8", "mxfp4"), default="bf16",
                    help="expert weight format of the named workload (the headline is bf16)")
    ap.add_argument("--hc", type=int, default=0,
                    help="also time the named workload wrapped by this many hyper-connection streams (bf16 only)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="budget of the headline's oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the device-ceiling microbenchmarks (HBM read, fp16 MFMA) reported as measured_peaks")
    ap.add_argument("--graph", action="store_true",
                    help="also time the L decode layers chained (each layer's output the next one's input) on one "
                         "workspace as one captured HIP graph against the same chain launched eagerly")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    if args.hc and (args.weights != "bf16" or not 1 <= args.hc <= 4):
        print("--hc takes 1 to 4 streams around bf16 expert weights", file=sys.stderr)
        sys.exit(2)

    import torch

    from mixture_experts_ffn_rmsnorm_amd import inputs as gen
    from mixture_experts_ffn_rmsnorm_amd import moe

    moe.lib()  # fail loudly if the HIP library is missing
    torch.cuda.set_device(0)
    cfg = gen.config(args.workload)
    subs = [] if (args.only or cfg.hidden != 4096 or args.weights != "bf16") else \
        [gen.config(n) for n in SUB_WORKLOADS if n != cfg.name]
    nl = lambda c: args.layers or (4 if c.rows <= 4 else 1)
    L = max([nl(cfg)] + [nl(c) for c in subs])
    log(f"workload {cfg.name} (+ {len(subs)} more): drawing {L} layers of weights on the GPU")
    big = draw_layers(cfg, L) if args.weights == "bf16" else draw_layers_mx(cfg, L, args.weights)
    layers = bind_layers(cfg, big, nl(cfg), args.weights)
    rec, gpu0 = time_workload(cfg, layers, args.steps, args.warmup, graph=args.graph and cfg.rows <= 4)
    R = cfg.rows
    res = {
        "metric": METRIC, "value": rec["rows_per_s"], "unit": "rows/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": rec["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32" if R <= 4 else "f16", "data": "synthetic",
        "config": {"workload": cfg.name, "rows": R, "hidden": cfg.hidden, "experts": cfg.experts,
                   "top_k": cfg.top_k, "inter": cfg.inter, "shared_experts": 1,
                   "layer_kind": "hash" if cfg.layer_kind == 1 else "score", "weights": args.weights,
                   "layers_cycled": rec["layers_cycled"],
                   "distinct_routed_experts": rec["distinct_routed_experts"]},
        "roofline": rec["roofline"],
    }
    for k in ("latency_us", "step_alg_bytes", "step_hbm_GBps", "step_hbm_frac", "step_alg_flops", "step_TFLOPs",
              "step_mfma_frac", "status_flags", "kernels", "graph"):
        if k in rec:
            res[k] = rec[k]
    if args.hc:
        res["hc"] = time_hc(cfg, layers, args.hc, args.steps, args.warmup, rec["ms_per_step"])
    sub_gpu = {}
    if subs:
        res["workloads"] = {}
    for c in subs:
        lay_c = bind_layers(c, big, nl(c))
        r_c, g_c = time_workload(c, lay_c, args.steps, args.warmup, graph=args.graph and c.rows <= 4)
        r_c["dtype"] = "f32" if c.rows <= 4 else "f16"
        r_c["layer_kind"] = "hash" if c.layer_kind == 1 else "score"
        res["workloads"][c.name] = r_c
        sub_gpu[c.name] = (lay_c[0], g_c)
        torch.cuda.empty_cache()
    if subs:
        for name in HC_WORKLOADS:
            c = gen.config(name)
            lay_c = bind_layers(c, big, nl(c))
            base_ms = rec["ms_per_step"] if c.name == cfg.name else res["workloads"][c.name]["ms_per_step"]
            res["workloads"][f"{c.name}-hc{HC_STREAMS}"] = time_hc(c, lay_c, HC_STREAMS, args.steps, args.warmup,
                                                                    base_ms)
    mx_gpu = {}
    if subs:
        for fmt, names in (("mxfp8", MX_WORKLOADS), ("mxfp4", MX4_WORKLOADS)):
            mx_cfgs = [gen.config(n) for n in names]
            big_mx = draw_layers_mx(cfg, max(nl(c) for c in mx_cfgs), fmt)
            for c in mx_cfgs:
                lay_c = bind_layers(c, big_mx, nl(c), fmt)
                r_c, g_c = time_workload(c, lay_c, args.steps, args.warmup, graph=args.graph and c.rows <= 4)
                r_c["dtype"] = "f32" if c.rows <= 4 else "f16"
                r_c["layer_kind"] = "hash" if c.layer_kind == 1 else "score"
                res["workloads"][f"{c.name}-{fmt}"] = r_c
                mx_gpu[f"{c.name}-{fmt}"] = (c, lay_c[0], g_c)
            del big_mx
            torch.cuda.empty_cache()
    if not args.no_peaks:
        # the published peaks above are the roofline's; these are the same
        # two ceilings measured on this device, after the timed passes
        from mixture_experts_ffn_rmsnorm_amd import device_peaks

        log("measuring device ceilings")
        pk = device_peaks.measure(read_sequence=rec["launch_bytes"])
        if "read_floor_us" in pk:
            # the step's event-timed latency against plain reads of its launches' bytes
            pk["step_latency_over_read_floor"] = rec["latency_us"]["median"] / pk["read_floor_us"]
        roof = res["roofline"]
        top = pk["hbm_read_GBps"] if roof["unit"] == "GB/s" else pk["mfma_f16_TFLOPs"]
        pk["roofline_frac_of_measured"] = roof["achieved"] / top
        res["measured_peaks"] = pk
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, layers[0], args.cpu_seconds, gpu0)
        for c in subs:
            lay0, g_c = sub_gpu[c.name]
            res["workloads"][c.name]["cpu_baseline"] = oracle_full_batch(c, lay0, g_c)
        for name, (c, lay0, g_c) in mx_gpu.items():
            res["workloads"][name]["cpu_baseline"] = oracle_full_batch(c, lay0, g_c)
    print(json.dumps(res), flush=True)


def graph_chain(dims, cfg, layers, x, tok, ws, reps, eager_ms):
    """The L layers back to back as a model runs them (layer l's output is
    layer l+1's input), every layer on the one workspace `ws`: launched
    eagerly, then captured once as a HIP graph and replayed.  Per-layer
    times of both."""
    import torch

    from mixture_experts_ffn_rmsnorm_amd import moe

    L = len(layers)
    bufs = [x] + [torch.empty_like(x) for _ in range(L)]

    fwd = forward_fn(layers[0][3])

    def chain():
        for l in range(L):
            fwd(dims, bufs[l], tok, cfg.layer_kind, layers[l][2], bufs[l + 1], ws)

    for _ in range(3):
        chain()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        chain()
    torch.cuda.synchronize()
    eager = (time.perf_counter() - t0) * 1e3 / (reps * L)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        chain()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    log(f"graph: {L} layers on one workspace, {reps} replays")
    t0 = time.perf_counter()
    for _ in range(reps):
        g.replay()
    torch.cuda.synchronize()
    ms_layer = (time.perf_counter() - t0) * 1e3 / (reps * L)
    return {"layers": L, "replays": reps, "workspaces": 1, "us_per_layer_graph": ms_layer * 1e3,
            "us_per_layer_eager_chain": eager * 1e3, "us_per_step_independent": eager_ms * 1e3,
            "rows_per_s_graph": cfg.rows / (ms_layer / 1e3)}


def _oracle_weights(cfg, layer):
    """The oracle's view of one bench layer: small parameters from the host
    inputs, expert matrices copied from the device when first needed."""
    from mixture_experts_ffn_rmsnorm_amd import inputs as gen
    from oracle import moe_ref as ref

    hi, keep, _, fmt = layer
    g, u, d, gs, us, ds = keep[4:]
    cache = {}
    if fmt == "bf16":
        host = gen.bf16_tensor_bits
        pick = lambda m, e: m[e]
    else:  # MXFP8 / MXFP4: (codes, scales) pairs, MXFP4 tagged for the oracle
        tag = (ref.MXFP4,) if fmt == "mxfp4" else ()
        host = lambda pair: gen.mx_host(pair) + tag
        pick = lambda m, e: (m[0][e], m[1][e])

    def expert(e):
        if e not in cache:
            cache[e] = tuple(host(pick(m, e)) for m in (g, u, d))
        return cache[e]

    return ref.Weights(hi.norm_w, hi.router, hi.sel_bias, hi.tid2eid, expert,
                       tuple(host(m) for m in (gs, us, ds))), cache


def _threads():
    """(threads the oracle's BLAS runs on, cores this process may use)."""
    try:
        from threadpoolctl import threadpool_info

        blas = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:
        blas = 1
    return blas, len(os.sched_getaffinity(0))


def _parity(cfg, hi, res, out_g, idx_g):
    """Agreement of the GPU's output and expert sets with the oracle's on the
    rows of `res`: relL2 (whole batch and worst row), max-abs ratio, rows
    whose expert set matches, and
    rows whose oracle 6th and 7th selection keys lie within 1e-6 (where a
    set mismatch would be a float32 tie, not an error; hash layers select
    from the table and have none)."""
    import numpy as np

    from oracle import moe_ref as ref

    n = res["out"].shape[0]
    ref_out = res["out"]
    same = sum(set(idx_g[r].tolist()) == set(res["idx"][r].tolist()) for r in range(n))
    gap_tol = 1e-6
    near = 0
    if cfg.layer_kind == ref.LAYER_SCORE and cfg.experts > cfg.top_k:
        keys = ref.sigmoid(res["logits"]) + np.asarray(hi.sel_bias, dtype=np.float64)
        top = -np.sort(-keys, axis=1)
        near = int(np.sum(top[:, cfg.top_k - 1] - top[:, cfg.top_k] < gap_tol))
    row_rel = np.linalg.norm(out_g - ref_out, axis=1) / np.maximum(np.linalg.norm(ref_out, axis=1), 1e-300)
    return {"rows": n, "relL2": float(np.linalg.norm(out_g - ref_out) / max(np.linalg.norm(ref_out), 1e-300)),
            "worst_row_relL2": float(row_rel.max()),
            "maxabs_ratio": float(np.abs(out_g - ref_out).max() / max(np.abs(ref_out).max(), 1e-300)),
            "index_match_rows": int(same), "near_tie_rows": near, "near_tie_gap": gap_tol}


def cpu_baseline(cfg, layer, budget_s, gpu):
    """The float64 oracle on a bounded sample of the headline workload (its
    first <= 4 rows, repeated for ~budget_s), with the GPU's agreement on
    those rows."""
    from oracle import moe_ref as ref

    hi = layer[0]
    W, _ = _oracle_weights(cfg, layer)
    per = min(cfg.rows, 4)
    xs, ts = hi.x[:per], hi.token_ids[:per]
    res = ref.forward(xs, ts, cfg.layer_kind, W, cfg.top_k, cfg.eps)  # fetches the experts before timing
    log(f"cpu baseline: timing the oracle on {per}-row samples for ~{budget_s:.0f}s")
    t0 = time.perf_counter()
    done = 0
    while True:
        ref.forward(xs, ts, cfg.layer_kind, W, cfg.top_k, cfg.eps)
        done += per
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    blas, host = _threads()
    out_g, idx_g = gpu
    return {"value": done / el, "unit": "rows/s", "cores": blas, "host_cores": host, "kind": "oracle",
            "sample": f"the first {per} row(s) of the workload through the float64 oracle, repeated "
                      f"{done // per}x in {el:.1f}s on {blas} BLAS threads ({host} cores available)",
            "parity": _parity(cfg, hi, res, out_g[:per], idx_g[:per])}


def oracle_full_batch(cfg, layer, gpu, min_s=3.0):
    """The float64 oracle over the workload's whole batch (repeated until
    min_s when one pass is shorter), timed after the experts it needs have
    been copied to the host, and the GPU's agreement on every row."""
    from oracle import moe_ref as ref

    hi = layer[0]
    W, cache = _oracle_weights(cfg, layer)
    R = cfg.rows
    log(f"{cfg.name}: oracle over all {R} rows")
    idx = ref.forward(hi.x, hi.token_ids, cfg.layer_kind, W, cfg.top_k, cfg.eps)["idx"] if R <= 4 else gpu[1]
    for e in set(int(v) for v in idx.reshape(-1) if 0 <= v < cfg.experts):
        W.expert(e)  # host copies outside the timed region
    t0 = time.perf_counter()
    passes = 0
    while True:
        res = ref.forward(hi.x, hi.token_ids, cfg.layer_kind, W, cfg.top_k, cfg.eps)
        passes += 1
        if time.perf_counter() - t0 >= min_s:
            break
    el = (time.perf_counter() - t0) / passes
    blas, host = _threads()
    rec = {"value": R / el, "unit": "rows/s", "cores": blas, "host_cores": host, "kind": "oracle",
           "oracle_s_per_batch": el,
           "sample": f"all {R} rows of the workload through the float64 oracle, {passes} pass(es) of {el:.2f}s "
                     f"on {blas} BLAS threads ({host} cores available); expert copies to the host not timed",
           "parity": _parity(cfg, hi, res, gpu[0], gpu[1])}
    cache.clear()
    return rec


if __name__ == "__main__":
    main()
