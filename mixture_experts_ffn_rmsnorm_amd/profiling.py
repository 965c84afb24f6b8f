"""rocprofv3 summaries of the library's kernels, written under profiles/.

    python3 -m mixture_experts_ffn_rmsnorm_amd.profiling stats   --workload W [bench args...]
    python3 -m mixture_experts_ffn_rmsnorm_amd.profiling traffic --workload W

`stats` runs bench.py under ``rocprofv3 --kernel-trace --stats`` and writes
profiles/kernels-<W>.md: per-kernel call counts and durations plus the JSON
line the bench printed.

`traffic` measures HBM bytes per dispatch with two counter passes over the
same bench command (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch) and
calibrates each counter on a device-to-device copy of known size: the
factor is copy bytes / counter reading.  It writes profiles/traffic-<W>.txt
with the digest of the kernel sources it measured; bench.py reports the
dominant kernel's traffic from that file only while the digest matches.

Every run is a child process started with rocprofv3 in front of it; this
process itself never touches the GPU.  Raw profiler output stays in a
scratch directory (default /tmp/moe_prof).
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import shlex
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")
OUTDIR = PROFILES  # where summaries are written (--outdir)
COPY_BYTES = 1 << 30  # calibration copy: 1 GiB read, 1 GiB written


def sources_digest() -> str:
    """sha256 over the HIP sources and the public header (names and contents)."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "mixture_experts_ffn_rmsnorm_amd", "csrc", "*.hip")) +
                   glob.glob(os.path.join(ROOT, "mixture_experts_ffn_rmsnorm_amd", "csrc", "*.h")) +
                   glob.glob(os.path.join(ROOT, "include", "*.h")))
    for f in files:
        h.update(os.path.relpath(f, ROOT).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


PROFILED_NOTE = ("Under kernel tracing the bench's own per-kernel event timings (`kernels`, and the roofline "
                 "figure derived from them) include the tracer's per-dispatch overhead; the rocprofv3 durations in "
                 "the table are the reference, and the unprofiled bench's event timings agree with them.")


def short_name(kernel: str) -> str:
    """k_dec_gateup<4096, 2048> style names for this library's kernels."""
    s = re.sub(r"\(moe::\w+\)", "", kernel)
    s = s.replace("void ", "").replace("moe::(anonymous namespace)::", "").replace("moe::", "")
    return s.strip()


def _template(kernel: str):
    """(function name, top-level template arguments) of a demangled name."""
    k = short_name(kernel)
    k = k.split("(")[0] if "<" not in k.split("(")[0] else k
    lt = k.find("<")
    if lt < 0:
        return k.split("(")[0].strip(), []
    name, args, depth, cur = k[:lt].strip(), [], 0, ""
    for ch in k[lt + 1:]:
        if ch == "<":
            depth += 1
        elif ch == ">":
            if depth == 0:
                break
            depth -= 1
        if ch == "," and depth == 0:
            args.append(cur.strip())
            cur = ""
        else:
            cur += ch
    args.append(cur.strip())
    return name, args


def launch_name(kernel: str) -> str | None:
    """The launch name the stage timer and bench.py use for a kernel, by its
    template: block-scaled (MX) instances end in "_mx"; the one-row decode
    path's router-only head and shared-expert down are dec1_*."""
    name, args = _template(kernel)
    fmt = {"true": "_mx", "1": "_mx", "2": "_mx4"}.get(args[-1], "") if args else ""
    mx = fmt != ""
    base = None
    if name == "k_dec_head" and len(args) == 4:
        base = "dec1_router" if args[2] == "true" else "dec_head"
    elif name == "k_dec_gateup" and len(args) == 3:
        base = "dec_gateup"
    elif name == "k_dec1_gateup" and len(args) == 3:
        base = "dec1_gateup"
    elif name == "k_dec_down" and len(args) == 3:
        base = "dec_down"
    elif name == "k_dec1_down" and len(args) == 3:
        base = "dec1_down_reduce"
    elif name == "k_gemm" and len(args) == 5:
        base = {"0": "gemm_gateup_swiglu", "1": "gemm_down", "2": "gemm_down_shared_reduce"}.get(args[0])
    else:
        mx = False
        base = {"k_pre_norm": "pre_norm", "k_pre_router": "pre_router", "k_pre_sort": "pre_sort",
                "k_route": "route", "k_dec_reduce": "dec_reduce", "k_hc_mix": "hc_mix", "k_hc_mix_mfma": "hc_mix", "k_hc_pre": "hc_pre", "k_hc_post": "hc_post"}.get(name)
    if base is None:
        return None
    return base + fmt if mx else base


def _run(cmd, log):
    """Run `cmd`; its stderr goes to `log` and, line by line, to ours (the
    bench's progress lines); returns (returncode, stdout)."""
    print("[profiling] " + " ".join(shlex.quote(c) for c in cmd), file=sys.stderr, flush=True)
    with open(log, "w") as fh, open(log + ".stdout", "w") as fo:
        p = subprocess.Popen(cmd, stdout=fo, stderr=subprocess.PIPE, text=True, cwd=ROOT)
        for line in p.stderr:
            fh.write(line)
            if line.startswith("[bench]"):
                sys.stderr.write(line)
                sys.stderr.flush()
        rc = p.wait()
    return rc, open(log + ".stdout").read()


def _bench_cmd(workload, extra, weights="bf16", hc=0):
    return ([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", workload, "--only", "--weights", weights]
            + (["--hc", str(hc)] if hc else []) + list(extra))


def profile_key(workload: str, weights: str = "bf16", hc: int = 0) -> str:
    """File-name key of a workload's summaries: block-scaled weights add
    "-mxfp8" / "-mxfp4", the wrapped layer "-hc<streams>"."""
    key = workload if weights == "bf16" else f"{workload}-{weights}"
    return key + (f"-hc{hc}" if hc else "")


def _opts(args) -> str:
    """The format and wrapper options of a command line, as typed."""
    return ("" if args.weights == "bf16" else f" --weights {args.weights}") + (f" --hc {args.hc}" if args.hc else "")


def cmd_stats(args, extra):
    key = profile_key(args.workload, args.weights, args.hc)
    out_dir = os.path.join(args.scratch, f"stats_{key}")
    os.makedirs(out_dir, exist_ok=True)
    prof = ["rocprofv3", "--kernel-trace", "--stats", "--output-format", "csv", "-d", out_dir, "-o", "run", "--"]
    bench = _bench_cmd(args.workload, extra, args.weights, args.hc)
    rc, stdout = _run(prof + bench, os.path.join(out_dir, "log.txt"))
    json_line = next((l for l in stdout.splitlines() if l.startswith("{")), None)
    if rc != 0 and json_line is None:
        print(f"profiled command failed ({rc}); see {out_dir}/log.txt", file=sys.stderr)
        return rc
    stats = glob.glob(os.path.join(out_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not stats:
        print("no kernel_stats.csv produced", file=sys.stderr)
        return 1
    rows = []
    for row in csv.DictReader(open(stats[0])):
        if launch_name(row["Name"]) is None:
            continue
        rows.append((short_name(row["Name"]), launch_name(row["Name"]), int(row["Calls"]),
                     float(row["AverageNs"]) / 1e3, float(row["MinNs"]) / 1e3, float(row["MaxNs"]) / 1e3))
    rows.sort(key=lambda t: -t[2] * t[3])
    cmdline = "python3 -m mixture_experts_ffn_rmsnorm_amd.profiling stats --workload " + args.workload + _opts(args)
    if extra:
        cmdline += " -- " + " ".join(shlex.quote(e) for e in extra)
    path = os.path.join(OUTDIR, f"kernels-{key}.md")
    with open(path, "w") as f:
        f.write(f"# Kernel durations, workload {args.workload}, {args.weights} expert weights"
                + (f", wrapped by {args.hc} hyper-connection streams" if args.hc else "") + "\n\n")
        f.write("Command (from the repository root, on one MI355X):\n\n")
        f.write(f"    {cmdline}\n\nwhich runs\n\n    rocprofv3 --kernel-trace --stats --output-format csv "
                f"-d <scratch> -o run -- python3 bench.py --workload {args.workload} --only --weights {args.weights}"
                + (f" --hc {args.hc}" if args.hc else "") + ("" if not extra else " " + " ".join(extra)) + "\n\n")
        f.write(f"Kernel sources digest: `{sources_digest()}`\n\n")
        f.write("rocprofv3 kernel statistics for this library's kernels (every call of the run: warm-up, "
                "timed steps and the per-kernel event pass):\n\n")
        f.write("| kernel | launch name | calls | avg us | min us | max us |\n|---|---|---|---|---|---|\n")
        for s, ln, c, a, mn, mx in rows:
            f.write(f"| {s} | {ln} | {c} | {a:.1f} | {mn:.1f} | {mx:.1f} |\n")
        if json_line:
            f.write("\nbench.py output of the same run:\n\n```\n" + json_line + "\n```\n")
            f.write("\n" + PROFILED_NOTE + "\n")
    print(open(path).read())
    return 0


# counters are collected on this library's kernels only (the weight
# generation's torch kernels run unprofiled)
KERNEL_REGEX = "k_(dec|pre|gemm|route|hc)"


def _pmc_pass(counter, cmd, out_dir, include=None):
    os.makedirs(out_dir, exist_ok=True)
    prof = ["rocprofv3", "--pmc", counter, "--output-format", "csv", "-d", out_dir, "-o", "run"]
    prof += (["--kernel-include-regex", include] if include else []) + ["--"]
    rc, _ = _run(prof + cmd, os.path.join(out_dir, "log.txt"))
    files = glob.glob(os.path.join(out_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise RuntimeError(f"{counter}: no counter_collection.csv (rc {rc}); see {out_dir}/log.txt")
    per = {}
    for f in files:
        for row in csv.DictReader(open(f)):
            if row.get("Counter_Name") != counter:
                continue
            k = row["Kernel_Name"]
            d = row.get("Dispatch_Id", "")
            per.setdefault(k, {}).setdefault(d, 0.0)
            per[k][d] += float(row["Counter_Value"])
    return {k: sum(v.values()) / len(v) for k, v in per.items()}  # mean KiB per dispatch


def cmd_traffic(args, extra):
    copy_cmd = [sys.executable, "-m", "mixture_experts_ffn_rmsnorm_amd.profiling", "child-copy"]
    key = profile_key(args.workload, args.weights, args.hc)
    bench_args = ["--steps", "5", "--warmup", "2", "--layers", "1", "--no-cpu-baseline", "--no-peaks"]
    bench = _bench_cmd(args.workload, bench_args, args.weights, args.hc)
    res = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        copy = _pmc_pass(counter, copy_cmd, os.path.join(args.scratch, f"copy_{counter}"))
        big = max(copy.items(), key=lambda kv: kv[1])  # the 1 GiB copy
        kern = _pmc_pass(counter, bench, os.path.join(args.scratch, f"{key}_{counter}"), KERNEL_REGEX)
        res[counter] = (big, kern)
    (cf_name, cf), _ = res["FETCH_SIZE"]
    (cw_name, cw), _ = res["WRITE_SIZE"]
    ffac, wfac = COPY_BYTES / (cf * 1024.0), COPY_BYTES / (cw * 1024.0)
    names = sorted(set(res["FETCH_SIZE"][1]) | set(res["WRITE_SIZE"][1]))
    path = os.path.join(OUTDIR, f"traffic-{key}.txt")
    wopt = _opts(args)
    with open(path, "w") as f:
        f.write(f"# HBM traffic per dispatch, workload {args.workload}, {args.weights} expert weights, "
                + (f"wrapped by {args.hc} hyper-connection streams, " if args.hc else "")
                + "from rocprofv3 counters\n")
        f.write(f"# command: python3 -m mixture_experts_ffn_rmsnorm_amd.profiling traffic --workload {args.workload}"
                f"{wopt}\n")
        f.write(f"# passes: rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE, with --kernel-include-regex "
                f"'{KERNEL_REGEX}', each over\n")
        f.write(f"#   python3 bench.py --workload {args.workload} --only --weights {args.weights} "
                + (f"--hc {args.hc} " if args.hc else "") + " ".join(bench_args) + "\n")
        f.write("#   and over a 1 GiB device-to-device copy (calibration: factor = bytes / counter bytes)\n")
        f.write(f"sources_sha256: {sources_digest()}\n")
        f.write(f"copy_kernel: {short_name(cf_name)}\n")
        f.write(f"copy_fetch_kib: {cf:.1f}\ncopy_write_kib: {cw:.1f}\n")
        f.write(f"fetch_factor: {ffac:.4f}\nwrite_factor: {wfac:.4f}\n")
        for k in names:
            ln = launch_name(k)
            if ln is None:
                continue
            fk = res["FETCH_SIZE"][1].get(k, 0.0)
            wk = res["WRITE_SIZE"][1].get(k, 0.0)
            b = fk * 1024.0 * ffac + wk * 1024.0 * wfac
            f.write(f"kernel: {ln} fetch_kib {fk:.1f} write_kib {wk:.1f} bytes {b:.0f}\n")
    print(open(path).read())
    return 0


def read_traffic(workload: str):
    """{launch name: HBM bytes per dispatch} from profiles/traffic-<workload>.txt,
    or None if the file is absent or was measured on other kernel sources."""
    path = os.path.join(PROFILES, f"traffic-{workload}.txt")
    if not os.path.exists(path):
        return None
    out, digest = {}, None
    for line in open(path):
        if line.startswith("sources_sha256:"):
            digest = line.split(":", 1)[1].strip()
        elif line.startswith("kernel:"):
            p = line.split()
            out[p[1]] = float(p[p.index("bytes") + 1])
    if digest != sources_digest():
        return None
    return out


def child_copy():
    import torch

    n = COPY_BYTES // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print("copy done", flush=True)


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "child-copy":
        child_copy()
        return 0
    ap = argparse.ArgumentParser()
    ap.add_argument("what", choices=["stats", "traffic"])
    ap.add_argument("--workload", default="decode-r1-score")
    ap.add_argument("--weights", choices=["bf16", "mxfp8", "mxfp4"], default="bf16")
    ap.add_argument("--hc", type=int, default=0, help="profile the layer wrapped by this many streams")
    ap.add_argument("--scratch", default="/tmp/moe_prof")
    ap.add_argument("--outdir", default=PROFILES, help="directory for the summaries (default profiles/)")
    argv = sys.argv[1:]
    extra = []
    if "--" in argv:
        i = argv.index("--")
        argv, extra = argv[:i], argv[i + 1:]
    args = ap.parse_args(argv)
    global OUTDIR
    OUTDIR = os.path.abspath(args.outdir)
    os.makedirs(OUTDIR, exist_ok=True)
    return cmd_stats(args, extra) if args.what == "stats" else cmd_traffic(args, extra)


if __name__ == "__main__":
    sys.exit(main())
