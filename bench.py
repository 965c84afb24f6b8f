#!/usr/bin/env python3
"""Throughput of the routed MoE FFN layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--layers L]

A step is one moe_ffn_forward call (RMSNorm, router, routing, sort, gate/up +
SwiGLU, down, weighted reduce + shared expert) over one batch of synthetic
rows with every input already in HBM.  Steps cycle over L independently drawn
layers of weights so that a step never finds the previous step's experts in
the 256 MB Infinity Cache.  Kernel durations come from HIP start/stop events
the library records at each kernel's own start and end during the timed
steps; the dominant kernel is reported against the MI355X roofline.  The
float64 CPU oracle is timed on a bounded sample beside it.

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
EXPERT_BYTES = lambda H, I: 3 * H * I * 2  # gate + up + down, bf16


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def alg_bytes(kernel, cfg, U, R):
    """Algorithmic HBM bytes of one launch: every touched weight once, plus
    activations in and out (U = distinct routed experts of the step; a
    routed (expert, row) pair per slot, R*K of them)."""
    H, I, E, K = cfg.hidden, cfg.inter, cfg.experts, cfg.top_k
    x = R * H * 4
    S = R * K
    if kernel == "dec_head":         # router + routing plan + shared gate/up
        return E * H * 2 + 2 * I * H * 2 + 2 * x + H * 4 + R * E * 12 + R * (H + I) * 4
    if kernel == "dec_gateup":       # shared down + routed gate/up
        return H * I * 2 + U * 2 * I * H * 2 + R * (I + H) * 4 + R * K * (H + I) * 4
    if kernel == "dec_down_reduce":  # routed down + weighted reduce
        return U * H * I * 2 + R * K * (I + 2 * H) * 4 + R * H * 4 + x
    if kernel == "dec1_router":      # one-row path: router, logits + xn out
        return E * H * 2 + x + H * 4 + R * E * 4 + R * H * 4
    if kernel == "dec1_gateup":      # shared + routed gate/up, routing from the logits
        return (U + 1) * 2 * I * H * 2 + R * E * 4 + R * H * 4 + (R * K + R) * I * 4 + R * K * 12
    if kernel == "dec1_down_reduce":  # routed + shared down + weighted reduce
        return (U + 1) * H * I * 2 + (R * K + R) * I * 4 + (R * K + R) * 2 * H * 4 + R * H * 4
    if kernel == "pre_norm":         # x in, xn16 + xlo16 out
        return x + 2 * R * H * 2
    if kernel == "pre_router":       # xn16 + xlo16 in, logits + routing out, router weights once
        return E * H * 2 + 2 * R * H * 2 + R * E * 4 + S * 12
    if kernel == "pre_sort":         # row masks in; row lists, slot ranks and counts out
        return E * ((R + 31) // 32) * 4 + S * 4 * 2 + (E + 1) * 4
    if kernel == "gemm_gateup_swiglu":
        return (U + 1) * 2 * I * H * 2 + (S + R) * H * 2 + (S + R) * I * 2
    if kernel == "gemm_down":        # routed experts: h16 in, d16 out
        return U * H * I * 2 + S * I * 2 + S * H * 2
    if kernel == "gemm_down_shared_reduce":  # shared expert + weighted reduce of d16
        return H * I * 2 + R * I * 2 + S * H * 2 + R * H * 4 + S * 12
    return None


def alg_flops(kernel, cfg, R):
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


def step_bytes(cfg, U, R):
    H, I, E = cfg.hidden, cfg.inter, cfg.experts
    return (U + 1) * EXPERT_BYTES(H, I) + E * H * 2 + 2 * R * H * 4 + H * 4 + E * 4


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode-r1-score")
    ap.add_argument("--layers", type=int, default=None, help="distinct weight sets cycled (default 4 decode, 1 prefill)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="budget of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the device-ceiling microbenchmarks (HBM read, fp16 MFMA) reported as measured_peaks")
    ap.add_argument("--graph", action="store_true",
                    help="also time the L layers chained (each layer's output the next one's input) "
                         "as one captured HIP graph, replayed --steps times; reported under 'graph'")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from mixture_experts_ffn_rmsnorm_amd import inputs as gen
    from mixture_experts_ffn_rmsnorm_amd import moe

    moe.lib()  # fail loudly if the HIP library is missing
    cfg = gen.config(args.workload)
    R = cfg.rows
    decode = R <= 4
    L = args.layers or (4 if decode else 1)
    log(f"workload {cfg.name}: rows={R} layers={L}; drawing weights on the GPU")
    torch.cuda.set_device(0)
    dims = moe.dims_of(cfg)
    layers = []
    for l in range(L):
        hi = gen.host_inputs(cfg, layer=l)
        (g, u, d), (gs, us, ds) = gen.expert_weights_device(cfg, "cuda", layer=l)
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        keep = [t(hi.norm_w), t(hi.router.view(np.int16)).view(torch.bfloat16), t(hi.sel_bias),
                t(hi.tid2eid) if hi.tid2eid is not None else None, g, u, d, gs, us, ds]
        layers.append((hi, keep, moe.make_weights(*keep)))
        log(f"layer {l} ready")
    hi0 = layers[0][0]
    x = torch.from_numpy(hi0.x).cuda()
    tok = torch.from_numpy(hi0.token_ids).cuda()
    out = torch.empty_like(x)
    ws = [moe.alloc_workspace(dims, R) for _ in range(L)]
    torch.cuda.synchronize()

    def step(i):
        l = i % L
        moe.forward(dims, x, tok, cfg.layer_kind, layers[l][2], out, ws[l])

    log(f"warmup {args.warmup}")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # distinct routed experts of each layer's step, from its routing
    U = []
    for l in range(L):
        step(l)
        torch.cuda.synchronize()
        idx = moe.routing_view(dims, R, ws[l])[1].cpu().numpy()
        U.append(len(np.unique(idx[(idx >= 0) & (idx < cfg.experts)])))
    log(f"distinct routed experts per layer: {U}")

    # throughput pass: the timed region, plain launches
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    value = R / (ms_per_step / 1e3)
    u_mean = float(np.mean([U[i % L] for i in range(args.steps)]))
    # kernel pass: the same steps again, each kernel bracketed by HIP
    # start/stop events taken at the kernel's own start and end
    log("timing kernels")
    moe.stage_timing_begin()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    stages = moe.stage_timing_end()
    # latency pass: each step bracketed by events on the stream the kernels use
    lat = []
    for i in range(args.steps):
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
    # the kernel's roofline: whichever of HBM and the matrix cores bounds it
    if flops is not None and flops / (MFMA_F16_PEAK_TFLOPS * 1e12) > b / (HBM_PEAK_GBPS * 1e9):
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

    measured = profiling.read_traffic(cfg.name)
    if measured and dom in measured:
        roof["traffic"] = measured[dom]
    for name, k in kernels.items():
        kb, kf = alg_bytes(name, cfg, u_mean, R), alg_flops(name, cfg, R)
        secs = k["avg_us"] * 1e-6
        if kb is not None:
            k["hbm_frac"] = kb / secs / 1e9 / HBM_PEAK_GBPS
        if kf is not None:
            k["mfma_frac"] = kf / secs / 1e12 / MFMA_F16_PEAK_TFLOPS
    sb = step_bytes(cfg, u_mean, R)
    sf = step_flops(cfg, R)
    # one call of layer 0 for the parity sample and the status word
    step(0)
    torch.cuda.synchronize()
    per = min(R, 4)
    gpu0 = (out[:per].cpu().numpy().copy(), moe.routing_view(dims, R, ws[0])[1][:per].cpu().numpy().copy())
    status_flags = moe.status(ws[0])
    res = {
        "metric": METRIC, "value": value, "unit": "rows/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32" if decode else "f16", "data": "synthetic",
        "config": {"workload": cfg.name, "rows": R, "hidden": cfg.hidden, "experts": cfg.experts,
                   "top_k": cfg.top_k, "inter": cfg.inter, "shared_experts": 1,
                   "layer_kind": "hash" if cfg.layer_kind == 1 else "score", "layers_cycled": L,
                   "distinct_routed_experts": u_mean},
        "roofline": roof,
        "latency_us": {"median": float(np.median(lat_us)), "p10": float(np.percentile(lat_us, 10)),
                       "p90": float(np.percentile(lat_us, 90))},
        "step_alg_bytes": sb,
        "step_hbm_GBps": sb / (ms_per_step / 1e3) / 1e9,
        "step_hbm_frac": sb / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBPS,
        "step_alg_flops": sf,
        "step_TFLOPs": sf / (ms_per_step / 1e3) / 1e12,
        "step_mfma_frac": sf / (ms_per_step / 1e3) / 1e12 / MFMA_F16_PEAK_TFLOPS,
        "status_flags": status_flags,
        "kernels": kernels,
    }

    if args.graph:
        res["graph"] = graph_chain(dims, cfg, layers, x, tok, ws, args.steps, log)
    if not args.no_peaks:
        # the published peaks above are the roofline's; these are the same
        # two ceilings measured on this device, after the timed passes
        from mixture_experts_ffn_rmsnorm_amd import device_peaks

        log("measuring device ceilings")
        pk = device_peaks.measure()
        top = pk["hbm_read_GBps"] if roof["unit"] == "GB/s" else pk["mfma_f16_TFLOPs"]
        pk["roofline_frac_of_measured"] = roof["achieved"] / top
        res["measured_peaks"] = pk
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, layers[0], args.cpu_seconds, log, gpu0)
    print(json.dumps(res), flush=True)


def graph_chain(dims, cfg, layers, x, tok, ws, reps, log):
    """The L layers back to back as a model runs them (layer l's output is
    layer l+1's input), captured once as a HIP graph and replayed: per-layer
    time without host launches between the kernels."""
    import torch

    from mixture_experts_ffn_rmsnorm_amd import moe

    L = len(layers)
    bufs = [x] + [torch.empty_like(x) for _ in range(L)]

    def chain():
        for l in range(L):
            moe.forward(dims, bufs[l], tok, cfg.layer_kind, layers[l][2], bufs[l + 1], ws[l])

    chain()  # outside the graph first
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        chain()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    log(f"graph: {L} layers, {reps} replays")
    t0 = time.perf_counter()
    for _ in range(reps):
        g.replay()
    torch.cuda.synchronize()
    ms_layer = (time.perf_counter() - t0) * 1e3 / (reps * L)
    return {"layers": L, "replays": reps, "ms_per_layer": ms_layer, "rows_per_s": cfg.rows / (ms_layer / 1e3)}


def cpu_baseline(cfg, layer, budget_s, log, gpu=None):
    """The float64 oracle on a bounded sample of the same workload; with the
    GPU's output and expert indices for the same rows (`gpu`), also their
    agreement with the oracle on that sample."""
    import numpy as np

    from mixture_experts_ffn_rmsnorm_amd import inputs as gen
    from oracle import moe_ref as ref

    hi, keep, _ = layer
    g, u, d, gs, us, ds = keep[4:]
    cache = {}

    def expert(e):
        if e not in cache:
            cache[e] = tuple(gen.bf16_tensor_bits(m[e]) for m in (g, u, d))
        return cache[e]

    W = ref.Weights(hi.norm_w, hi.router, hi.sel_bias, hi.tid2eid, expert,
                    tuple(gen.bf16_tensor_bits(m) for m in (gs, us, ds)))
    per = min(cfg.rows, 4)
    # fetch the experts of the sample rows before timing
    xs, ts = hi.x[:per], hi.token_ids[:per]
    res = ref.forward(xs, ts, cfg.layer_kind, W, cfg.top_k, cfg.eps)
    log(f"cpu baseline: timing the oracle on {per}-row samples for ~{budget_s:.0f}s")
    t0 = time.perf_counter()
    done = 0
    while True:
        ref.forward(xs, ts, cfg.layer_kind, W, cfg.top_k, cfg.eps)
        done += per
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    try:
        from threadpoolctl import threadpool_info

        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        cores = 1
    base = {"value": done / el, "unit": "rows/s", "cores": cores, "kind": "oracle",
            "sample": f"the first {per} row(s) of the workload through the float64 oracle, repeated "
                      f"{done // per}x in {el:.1f}s (BLAS threads = cores)"}
    if gpu is not None:
        out_g, idx_g = gpu
        ref_out = res["out"]
        same = [set(idx_g[r].tolist()) == set(res["idx"][r].tolist()) for r in range(per)]
        base["parity"] = {
            "rows": per,
            "relL2": float(np.linalg.norm(out_g - ref_out) / max(np.linalg.norm(ref_out), 1e-300)),
            "maxabs_ratio": float(np.abs(out_g - ref_out).max() / max(np.abs(ref_out).max(), 1e-300)),
            "index_match_rows": int(sum(same)),
        }
        # rows whose K-th and (K+1)-th selection keys (oracle, float64) lie
        # closer than float32 rounding of the logits could reorder: there an
        # index mismatch is a legitimate tie, not an error (hash layers select
        # from the table and have none)
        gap_tol = 1e-6
        near = 0
        if cfg.layer_kind == ref.LAYER_SCORE and cfg.experts > cfg.top_k:
            keys = ref.sigmoid(res["logits"]) + np.asarray(hi.sel_bias, dtype=np.float64)
            top = -np.sort(-keys, axis=1)
            near = int(np.sum(top[:, cfg.top_k - 1] - top[:, cfg.top_k] < gap_tol))
        base["parity"]["near_tie_rows"] = near
        base["parity"]["near_tie_gap"] = gap_tol
    return base


if __name__ == "__main__":
    main()
