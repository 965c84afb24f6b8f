"""Build libmoeffn.so (and libmoepeaks.so) in-tree with hipcc for gfx950.

    python -m mixture_experts_ffn_rmsnorm_amd.build

Each ``csrc/*.hip`` compiles to an object under ``_build/`` in parallel, then
everything links into ``mixture_experts_ffn_rmsnorm_amd/libmoeffn.so``;
``peaks/peaks.hip`` (the device-ceiling microbenchmarks) becomes
``mixture_experts_ffn_rmsnorm_amd/libmoepeaks.so``; the same sources built
with ``-DMOE_CHECKED`` become ``libmoeffn_checked.so``, the checked build
(bounds tests on the indices the call itself produces, reported through
MOE_FLAG_CHECK).  The build always recompiles (it is the "does it build"
check); loading code never builds.
"""

from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoeffn.so")
CHECKED_LIB = os.path.join(PKG, "libmoeffn_checked.so")
PEAKS_SRC = os.path.join(PKG, "peaks", "peaks.hip")
PEAKS_LIB = os.path.join(PKG, "libmoepeaks.so")
ARCH = os.environ.get("MOEFFN_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed-FP32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I", INCLUDE, "-I", CSRC,
]


def _compile(src: str, checked: bool = False) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + (".checked.o" if checked else ".o"))
    cmd = [HIPCC, *CFLAGS, *(["-DMOE_CHECKED"] if checked else []), "-c", src, "-o", obj]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{p.stderr}")
    warn = "\n".join(l for l in p.stderr.splitlines() if "packed-fp32-ops" not in l and "hip-link" not in l)
    if warn.strip():
        print(warn, file=sys.stderr)
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link of {lib} failed:\n{p.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = [(s, False) for s in srcs] + [(PEAKS_SRC, False)] + [(s, True) for s in srcs]
    with ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    n = len(srcs)
    _link(objs[n:n + 1], PEAKS_LIB)
    _link(objs[:n], LIB)
    _link(objs[n + 1:], CHECKED_LIB)
    if verbose:
        print(f"built {LIB}, {CHECKED_LIB} and {PEAKS_LIB}")
    return LIB


if __name__ == "__main__":
    build()
