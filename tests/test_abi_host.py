"""Host-side checks of the C ABI: the library loads, exports every function
include/moe_ffn.h declares, agrees with the header on struct layout, and
rejects every malformed call on the host with the documented code.  No call
here reaches a kernel launch, so no GPU is needed."""

from __future__ import annotations

import ctypes
import os
import re
import subprocess
import tempfile

import pytest

from mixture_experts_ffn_rmsnorm_amd import moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_ffn.h")
FULL = dict(hidden=4096, experts=256, top_k=6, inter=2048)
TINY = dict(hidden=512, experts=32, top_k=6, inter=256)
FAKE = 0x7F0000000000  # 256-aligned host-only placeholder address; never dereferenced
# Cases that fail only at the last host checks would launch kernels if a
# check regressed; keep them off machines that have a GPU.
no_gpu_here = pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="late-check cases run only without a GPU")


def header_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_\w+)\s*\(", txt)))


def test_exports_match_header():
    L = moe.lib()
    declared = header_functions()
    assert set(declared) == set(moe.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", moe.LIB_PATH], capture_output=True, text=True, check=True)
    syms = set(re.findall(r"\b(moe_\w+)\b", nm.stdout))
    assert set(declared) <= syms


def test_struct_layout_matches_header():
    src = r"""
    #include <stdio.h>
    #include <stddef.h>
    #include "moe_ffn.h"
    int main(void) {
      printf("%zu %zu %zu %zu %zu\n", sizeof(moe_dims_t), offsetof(moe_dims_t, table_rows),
             offsetof(moe_dims_t, eps), sizeof(moe_weights_t), offsetof(moe_weights_t, down_sh));
      return 0;
    }"""
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "t.c")
        open(c, "w").write(src)
        exe = os.path.join(d, "t")
        subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), c, "-o", exe], check=True)
        got = list(map(int, subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split()))
    assert got == [ctypes.sizeof(moe.Dims), moe.Dims.table_rows.offset, moe.Dims.eps.offset,
                   ctypes.sizeof(moe.WeightsC), moe.WeightsC.down_sh.offset]


def _weights(bias=True, table=True):
    return moe.WeightsC(FAKE, FAKE, FAKE if bias else None, FAKE if table else None, FAKE, FAKE, FAKE, FAKE, FAKE,
                        FAKE)


def _fwd(dims, x=FAKE, tok=FAKE, rows=4, kind=moe.LAYER_SCORE, w=None, out=FAKE + (1 << 30), ws=FAKE + (2 << 30),
         wsb=1 << 40):
    w = _weights() if w is None else w
    d = None if dims is None else ctypes.byref(dims)
    return moe.lib().moe_ffn_forward(d, x, tok, rows, kind, ctypes.byref(w), out, ws, wsb, None)


@pytest.mark.parametrize("case,code", [
    ("rows0", moe.MOE_EINVAL), ("rows_neg", moe.MOE_EINVAL), ("dims_null", moe.MOE_EINVAL),
    ("dims_other", moe.MOE_EUNSUPPORTED), ("topk8", moe.MOE_EUNSUPPORTED), ("two_shared", moe.MOE_EUNSUPPORTED),
    ("reserved", moe.MOE_EUNSUPPORTED), ("eps_nan", moe.MOE_EUNSUPPORTED), ("rows_huge", moe.MOE_EOVERFLOW),
    ("x_null", moe.MOE_EINVAL), ("x_misaligned", moe.MOE_EINVAL), ("out_null", moe.MOE_EINVAL),
    ("kind_bad", moe.MOE_EINVAL), ("score_no_bias", moe.MOE_EINVAL), ("hash_no_table", moe.MOE_EINVAL),
    ("hash_no_tokens", moe.MOE_EINVAL), ("hash_no_table_rows", moe.MOE_EINVAL), ("weights_null", moe.MOE_EINVAL),
    ("expert_null", moe.MOE_EINVAL), ("expert_misaligned", moe.MOE_EINVAL),
])
def test_forward_rejects_on_host(case, code):
    d = moe.make_dims(**FULL, table_rows=131072)
    kw = {}
    if case == "rows0":
        kw["rows"] = 0
    elif case == "rows_neg":
        kw["rows"] = -3
    elif case == "dims_null":
        d = None
    elif case == "dims_other":
        d = moe.make_dims(4096, 128, 6, 2048)
    elif case == "topk8":
        d = moe.make_dims(4096, 256, 8, 2048)
    elif case == "two_shared":
        d = moe.make_dims(**FULL, n_shared=2)
    elif case == "reserved":
        d.reserved0 = 1
    elif case == "eps_nan":
        d.eps = float("nan")
    elif case == "rows_huge":
        kw["rows"] = (1 << 24) + 1
    elif case == "x_null":
        kw["x"] = None
    elif case == "x_misaligned":
        kw["x"] = FAKE + 4
    elif case == "out_null":
        kw["out"] = None
    elif case == "kind_bad":
        kw["kind"] = 7
    elif case == "score_no_bias":
        kw["w"] = _weights(bias=False)
    elif case == "hash_no_table":
        kw.update(kind=moe.LAYER_HASH, w=_weights(table=False))
    elif case == "hash_no_tokens":
        kw.update(kind=moe.LAYER_HASH, tok=None)
    elif case == "hash_no_table_rows":
        d = moe.make_dims(**FULL, table_rows=0)
        kw["kind"] = moe.LAYER_HASH
    elif case == "weights_null":
        rc = moe.lib().moe_ffn_forward(ctypes.byref(d), FAKE, FAKE, 4, 0, None, FAKE + (1 << 30), FAKE, 1 << 40, None)
        assert rc == code
        return
    elif case == "expert_null":
        w = _weights()
        w.down_sh = None
        kw["w"] = w
    elif case == "expert_misaligned":
        w = _weights()
        w.up_exps = FAKE + 2
        kw["w"] = w
    assert _fwd(d, **kw) == code


@no_gpu_here
@pytest.mark.parametrize("case,code", [("ws_null", moe.MOE_EWORKSPACE), ("ws_small", moe.MOE_EWORKSPACE),
                                       ("ws_misaligned", moe.MOE_EWORKSPACE), ("overlap", moe.MOE_EOVERLAP),
                                       ("overlap_partial", moe.MOE_EOVERLAP)])
def test_forward_rejects_late_checks(case, code):
    d = moe.make_dims(**TINY)
    need = moe.workspace_bytes(d, 8)
    kw = dict(rows=8, wsb=need)
    if case == "ws_null":
        kw["ws"] = None
    elif case == "ws_small":
        kw["wsb"] = need - 1
    elif case == "ws_misaligned":
        kw["ws"] = FAKE + (2 << 30) + 16
    elif case == "overlap":
        kw["out"] = FAKE
    elif case == "overlap_partial":
        kw["out"] = FAKE + 8 * 512 * 4 - 16
    assert _fwd(d, **kw) == code


def test_workspace_bytes():
    d = moe.make_dims(**FULL)
    sizes = [moe.workspace_bytes(d, r) for r in (1, 2, 3, 4, 5, 512, 8192)]
    assert all(s % 256 == 0 and s > 0 for s in sizes)
    assert sizes[0] < sizes[1] < sizes[2] < sizes[3]
    assert sizes[4] < sizes[5] < sizes[6]
    # prefill at 8192 rows holds at least the grouped SwiGLU output and the
    # routed down output, both fp16
    assert sizes[6] >= (8192 * 6 + 8192) * 2048 * 2 + 8192 * 6 * 4096 * 2
    n = ctypes.c_size_t(0)
    assert moe.lib().moe_ffn_workspace_bytes(ctypes.byref(d), 0, ctypes.byref(n)) == moe.MOE_EINVAL
    assert moe.lib().moe_ffn_workspace_bytes(ctypes.byref(d), 4, None) == moe.MOE_EINVAL
    bad = moe.make_dims(1024, 256, 6, 2048)
    assert moe.lib().moe_ffn_workspace_bytes(ctypes.byref(bad), 4, ctypes.byref(n)) == moe.MOE_EUNSUPPORTED


def test_routing_view_is_host_arithmetic():
    d = moe.make_dims(**TINY)
    rows = 37
    need = moe.workspace_bytes(d, rows)
    lp, ip, wp = ctypes.c_void_p(), ctypes.c_void_p(), ctypes.c_void_p()
    rc = moe.lib().moe_ffn_routing_view(ctypes.byref(d), rows, FAKE, need, ctypes.byref(lp), ctypes.byref(ip),
                                        ctypes.byref(wp))
    assert rc == moe.MOE_OK
    offs = [p.value - FAKE for p in (lp, ip, wp)]
    assert all(o % 256 == 0 and 0 < o < need for o in offs)
    assert offs[1] - offs[0] >= rows * 32 * 4 and offs[2] - offs[1] >= rows * 6 * 4
    assert moe.lib().moe_ffn_routing_view(ctypes.byref(d), rows, FAKE, need - 1, None, None, None) == \
        moe.MOE_EWORKSPACE


def test_route_rejects_on_host():
    d = moe.make_dims(**FULL, table_rows=131072)
    L = moe.lib()
    w = _weights()
    assert L.moe_route(ctypes.byref(d), None, FAKE, 4, 0, ctypes.byref(w), FAKE, FAKE, None) == moe.MOE_EINVAL
    assert L.moe_route(ctypes.byref(d), FAKE, FAKE, 0, 0, ctypes.byref(w), FAKE, FAKE, None) == moe.MOE_EINVAL
    assert L.moe_route(ctypes.byref(d), FAKE, None, 4, 1, ctypes.byref(w), FAKE, FAKE, None) == moe.MOE_EINVAL
    nb = _weights(bias=False)
    assert L.moe_route(ctypes.byref(d), FAKE, FAKE, 4, 0, ctypes.byref(nb), FAKE, FAKE, None) == moe.MOE_EINVAL
    assert L.moe_route(ctypes.byref(d), FAKE, FAKE, 4, 0, ctypes.byref(w), None, FAKE, None) == moe.MOE_EINVAL


def test_status_and_timer_host_paths():
    L = moe.lib()
    f = ctypes.c_uint32()
    assert L.moe_ffn_status(None, None, ctypes.byref(f)) == moe.MOE_EINVAL
    assert L.moe_ffn_status(FAKE, None, None) == moe.MOE_EINVAL
    # an empty timing window touches no HIP state
    assert L.moe_ffn_stage_timing_begin() == moe.MOE_OK
    n = ctypes.c_int(-1)
    assert L.moe_ffn_stage_timing_end(0, None, None, None, ctypes.byref(n)) == moe.MOE_OK
    assert n.value == 0
    assert L.moe_ffn_stage_timing_end(-1, None, None, None, ctypes.byref(n)) == moe.MOE_EINVAL


def test_strerror():
    for c in range(8):
        assert moe.strerror(c) and moe.strerror(c) != "unknown status"
    assert moe.strerror(99) == "unknown status"


def test_peaks_library_exports_and_rejects_bad_arguments():
    """The device-ceiling microbenchmarks (libmoepeaks.so) load, export their
    functions, and reject malformed arguments before any launch."""
    from mixture_experts_ffn_rmsnorm_amd import device_peaks

    L = device_peaks.lib()
    nm = subprocess.run(["nm", "-D", "--defined-only", device_peaks.LIB_PATH], capture_output=True, text=True,
                        check=True)
    syms = set(re.findall(r"\b(moe_\w+)\b", nm.stdout))
    assert set(device_peaks.EXPORTS) <= syms
    assert L.moe_peaks_mfma_chains() >= 1 and L.moe_peaks_mfma_threads() % 64 == 0
    invalid = 1  # hipErrorInvalidValue
    sink = ctypes.c_void_p(FAKE)
    assert L.moe_peaks_read(None, 1 << 20, sink, 16, None) == invalid
    assert L.moe_peaks_read(ctypes.c_void_p(FAKE), (1 << 20) + 4, sink, 16, None) == invalid  # not whole 16-B chunks
    assert L.moe_peaks_read(ctypes.c_void_p(FAKE + 8), 1 << 20, sink, 16, None) == invalid  # misaligned
    assert L.moe_peaks_read(ctypes.c_void_p(FAKE), 1 << 20, sink, 0, None) == invalid
    assert L.moe_peaks_mfma(0, 16, sink, None) == invalid
    assert L.moe_peaks_mfma(16, 0, sink, None) == invalid
    assert L.moe_peaks_mfma(16, 16, None, None) == invalid


def _noalloc(dims, x=FAKE, tok=FAKE, rows=4, kind=moe.LAYER_SCORE, w=None, out=FAKE + (1 << 30)):
    w = _weights() if w is None else w
    d = None if dims is None else ctypes.byref(dims)
    return moe.lib().moe_ffn_forward_noalloc(d, x, tok, rows, kind, ctypes.byref(w), out, None)


def test_noalloc_rejects_on_host():
    """The allocation-free entry point checks its arguments like
    moe_ffn_forward, and a call whose intermediates exceed the built-in
    scratch is rejected with MOE_ESCRATCH -- all before any HIP call."""
    d = moe.make_dims(**FULL, table_rows=131072)
    assert _noalloc(None) == moe.MOE_EINVAL
    assert _noalloc(d, rows=0) == moe.MOE_EINVAL
    assert _noalloc(d, x=None) == moe.MOE_EINVAL
    assert _noalloc(d, out=None) == moe.MOE_EINVAL
    assert _noalloc(d, kind=5) == moe.MOE_EINVAL
    assert _noalloc(d, kind=moe.LAYER_HASH, tok=None) == moe.MOE_EINVAL
    assert _noalloc(moe.make_dims(4096, 128, 6, 2048)) == moe.MOE_EUNSUPPORTED
    assert _noalloc(d, rows=(1 << 24) + 1) == moe.MOE_EOVERFLOW
    assert _noalloc(d, rows=8, out=FAKE + 64) == moe.MOE_EOVERLAP
    # the size limit: 696 full-shape rows fit in 64 MiB, 697 do not
    assert moe.workspace_bytes(d, 696) <= moe.NOALLOC_SCRATCH_BYTES < moe.workspace_bytes(d, 697)
    assert _noalloc(d, rows=697) == moe.MOE_ESCRATCH
    assert _noalloc(d, rows=8192) == moe.MOE_ESCRATCH
    t = moe.make_dims(**TINY)
    assert moe.workspace_bytes(t, 5540) <= moe.NOALLOC_SCRATCH_BYTES < moe.workspace_bytes(t, 5541)
    assert _noalloc(t, rows=5541) == moe.MOE_ESCRATCH
    assert "scratch" in moe.strerror(moe.MOE_ESCRATCH)


def test_mx_struct_layout_matches_header():
    src = r"""
    #include <stdio.h>
    #include <stddef.h>
    #include "moe_ffn.h"
    int main(void) {
      printf("%zu %zu %zu %zu %d\n", sizeof(moe_mx_weights_t), offsetof(moe_mx_weights_t, gate_exps),
             offsetof(moe_mx_weights_t, down_sh), offsetof(moe_mx_matrix_t, scales), MOE_MX_BLOCK);
      return 0;
    }"""
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "t.c")
        open(c, "w").write(src)
        exe = os.path.join(d, "t")
        subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), c, "-o", exe], check=True)
        got = list(map(int, subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split()))
    assert got == [ctypes.sizeof(moe.MxWeightsC), moe.MxWeightsC.gate_exps.offset, moe.MxWeightsC.down_sh.offset,
                   moe.MxMatrixC.scales.offset, moe.MX_BLOCK]


def _mx_weights(drop=None, misalign=None):
    mats = {n: moe.MxMatrixC(FAKE, FAKE + (1 << 32)) for n in
            ("gate_exps", "up_exps", "down_exps", "gate_sh", "up_sh", "down_sh")}
    if drop:
        setattr(mats[drop[0]], drop[1], None)
    if misalign:
        setattr(mats[misalign[0]], misalign[1], getattr(mats[misalign[0]], misalign[1]) + 4)
    return moe.MxWeightsC(FAKE, FAKE, FAKE, FAKE, *mats.values())


def test_mxfp8_forward_rejects_on_host():
    """The MXFP8 entry point checks its weights (every code and scale array
    present and 16-byte aligned) and the shared arguments before any HIP
    call."""
    d = moe.make_dims(**FULL, table_rows=131072)
    L = moe.lib()

    def call(w, rows=4, dims=d, x=FAKE, kind=moe.LAYER_SCORE):
        return L.moe_ffn_forward_mxfp8(None if dims is None else ctypes.byref(dims), x, FAKE, rows, kind,
                                       None if w is None else ctypes.byref(w), FAKE + (1 << 30), FAKE + (2 << 30),
                                       1 << 40, None)

    assert call(None) == moe.MOE_EINVAL
    assert call(_mx_weights(), dims=None) == moe.MOE_EINVAL
    assert call(_mx_weights(drop=("down_sh", "scales"))) == moe.MOE_EINVAL
    assert call(_mx_weights(drop=("gate_exps", "codes"))) == moe.MOE_EINVAL
    assert call(_mx_weights(misalign=("up_exps", "codes"))) == moe.MOE_EINVAL
    assert call(_mx_weights(misalign=("gate_sh", "scales"))) == moe.MOE_EINVAL
    assert call(_mx_weights(), rows=0) == moe.MOE_EINVAL
    assert call(_mx_weights(), x=None) == moe.MOE_EINVAL
    assert call(_mx_weights(), kind=9) == moe.MOE_EINVAL
    assert call(_mx_weights(), dims=moe.make_dims(4096, 128, 6, 2048)) == moe.MOE_EUNSUPPORTED
    assert call(_mx_weights(), rows=(1 << 24) + 1) == moe.MOE_EOVERFLOW


def test_hc_struct_layout_matches_header():
    src = r"""
    #include <stdio.h>
    #include <stddef.h>
    #include "moe_ffn.h"
    int main(void) {
      printf("%zu %zu %zu %d %d\n", sizeof(moe_hc_weights_t), offsetof(moe_hc_weights_t, hc),
             offsetof(moe_hc_weights_t, sinkhorn_iters), MOE_HC_MAX, MOE_HC_MAX_ITERS);
      return 0;
    }"""
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "t.c")
        open(c, "w").write(src)
        exe = os.path.join(d, "t")
        subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), c, "-o", exe], check=True)
        got = list(map(int, subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split()))
    assert got == [ctypes.sizeof(moe.HcWeightsC), moe.HcWeightsC.hc.offset, moe.HcWeightsC.sinkhorn_iters.offset,
                   moe.HC_MAX, moe.HC_MAX_ITERS]


def test_hc_workspace_bytes_and_view():
    """The wrapper's workspace holds the FFN's layout at offset 0 plus the
    mixes, maps, FFN input and output; the view points inside it."""
    L = moe.lib()
    for dims, rows in ((moe.make_dims(**FULL, table_rows=131072), 1), (moe.make_dims(**TINY), 37)):
        n = ctypes.c_size_t(0)
        for hc in (0, 5):
            assert L.moe_ffn_hc_workspace_bytes(ctypes.byref(dims), hc, rows, ctypes.byref(n)) == \
                moe.MOE_EUNSUPPORTED
        assert L.moe_ffn_hc_workspace_bytes(ctypes.byref(dims), 4, rows, None) == moe.MOE_EINVAL
        base = moe.workspace_bytes(dims, rows)
        for hc in (1, 4):
            total = moe.hc_workspace_bytes(dims, hc, rows)
            mw, H = (2 + hc) * hc, dims.hidden
            assert total >= base + rows * (2 * mw + 2 * H) * 4
            ps = [ctypes.c_void_p() for _ in range(4)]
            assert L.moe_ffn_hc_view(ctypes.byref(dims), hc, rows, FAKE, total, *[ctypes.byref(p) for p in ps]) == 0
            offs = [p.value - FAKE for p in ps]
            assert offs[0] >= base and offs == sorted(offs) and all(o % 256 == 0 for o in offs)
            assert offs[1] - offs[0] >= rows * mw * 4 and offs[3] - offs[2] >= rows * H * 4
            assert offs[3] + rows * H * 4 <= total
            assert L.moe_ffn_hc_view(ctypes.byref(dims), hc, rows, FAKE, total - 1,
                                     *[ctypes.byref(p) for p in ps]) == moe.MOE_EWORKSPACE


def test_hc_forward_rejects_on_host():
    """Every malformed wrapper call fails on the host with its documented
    code before any HIP call."""
    d = moe.make_dims(**FULL, table_rows=131072)
    L = moe.lib()
    good = moe.HcWeightsC(FAKE, FAKE + 256, FAKE + 512, 4, 20)
    S = FAKE + (4 << 30)  # state_out, clear of state_in (FAKE) and the workspace

    def call(hw=good, rows=4, state=FAKE, out=S, ws=FAKE + (8 << 30), wsb=1 << 40, kind=moe.LAYER_SCORE, w=None):
        w = _weights() if w is None else w
        return L.moe_ffn_forward_hc(ctypes.byref(d), state, FAKE, rows, kind, ctypes.byref(w),
                                    None if hw is None else ctypes.byref(hw), out, ws, wsb, None)

    def hw(**kw):
        f = dict(hc_fn=FAKE, hc_scale=FAKE + 256, hc_base=FAKE + 512, hc=4, sinkhorn_iters=20)
        f.update(kw)
        return moe.HcWeightsC(f["hc_fn"], f["hc_scale"], f["hc_base"], f["hc"], f["sinkhorn_iters"])

    assert call(hw=None) == moe.MOE_EINVAL
    assert call(hw=hw(hc=0)) == moe.MOE_EUNSUPPORTED
    assert call(hw=hw(hc=5)) == moe.MOE_EUNSUPPORTED
    assert call(hw=hw(sinkhorn_iters=0)) == moe.MOE_EINVAL
    assert call(hw=hw(sinkhorn_iters=moe.HC_MAX_ITERS + 1)) == moe.MOE_EINVAL
    assert call(hw=hw(hc_fn=None)) == moe.MOE_EINVAL
    assert call(hw=hw(hc_fn=FAKE + 8)) == moe.MOE_EINVAL
    assert call(hw=hw(hc_base=None)) == moe.MOE_EINVAL
    assert call(hw=hw(hc_scale=FAKE + 2)) == moe.MOE_EINVAL
    assert call(state=None) == moe.MOE_EINVAL
    assert call(out=S + 4) == moe.MOE_EINVAL
    assert call(rows=0) == moe.MOE_EINVAL
    assert call(kind=moe.LAYER_HASH, w=_weights(table=False)) == moe.MOE_EINVAL
    assert call(out=FAKE + 4096 * 4) == moe.MOE_EOVERLAP              # inside state_in
    assert call(ws=S + 64 * 1024) == moe.MOE_EOVERLAP                 # workspace inside state_out
    assert call(wsb=1024) == moe.MOE_EWORKSPACE
    assert call(ws=FAKE + (8 << 30) + 16) == moe.MOE_EWORKSPACE
    assert call(rows=(1 << 24) + 1) == moe.MOE_EOVERFLOW


def test_checked_build_exports_the_same_functions():
    """The checked build (bounds tests reported through MOE_FLAG_CHECK) is the
    same C ABI."""
    syms = []
    for path in (moe.LIB_PATH, moe.CHECKED_LIB_PATH):
        nm = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True, check=True)
        syms.append(set(re.findall(r"\b(moe_\w+)\b", nm.stdout)))
    assert syms[0] == syms[1] and set(moe.EXPORTS) <= syms[1]
    L = moe.load(moe.CHECKED_LIB_PATH)
    assert L.moe_strerror(moe.MOE_EINVAL) == moe.lib().moe_strerror(moe.MOE_EINVAL)
