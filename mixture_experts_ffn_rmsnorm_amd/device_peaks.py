"""Device ceilings measured on the GPU itself (libmoepeaks.so), reported
beside MI355X's published figures (8 TB/s HBM, 2.5 PFLOP/s dense fp16/bf16
matrix) that the roofline fractions are taken against.

    hbm_read_GBps    -- 16-byte non-temporal loads over a 2 GiB buffer (8x
                        the 256 MB last-level cache), each workgroup reading
                        contiguous 32 KiB chunks
    mfma_f16_TFLOPs  -- v_mfma_f32_32x32x16_f16 from registers, 4
                        independent accumulators per wave, 4 waves per
                        workgroup, 4 workgroups per compute unit

Each launch is timed with its own pair of HIP events on the current stream,
after two untimed launches; a ceiling is the best launch.

    read_floor_us    -- (optional) plain reads of a given list of byte
                        counts, one launch each, back to back on one stream:
                        the time the same reads take when every launch only
                        reads (a launch's fixed ramp and tail included), the
                        floor of a step that makes launches of those sizes.
                        The windows rotate over the 2 GiB buffer, so no
                        launch finds its bytes in the last-level cache; the
                        median of the sequences.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoepeaks.so")
EXPORTS = ("moe_peaks_read", "moe_peaks_mfma", "moe_peaks_mfma_chains", "moe_peaks_mfma_threads")
MFMA_FLOPS = 2 * 32 * 32 * 16  # one v_mfma_f32_32x32x16_f16

_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m mixture_experts_ffn_rmsnorm_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.moe_peaks_read.argtypes = [P, SZ, P, I32, P]
        L.moe_peaks_mfma.argtypes = [I32, I32, P, P]
        L.moe_peaks_mfma_chains.argtypes = []
        L.moe_peaks_mfma_threads.argtypes = []
        _lib = L
    return _lib


def _timed(launch, reps: int) -> float:
    """Milliseconds of the fastest of `reps` launches (after 2 untimed)."""
    import torch

    for _ in range(2):
        launch()
    torch.cuda.synchronize()
    ev = []
    for _ in range(reps):
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        launch()
        t1.record()
        ev.append((t0, t1))
    torch.cuda.synchronize()
    return min(a.elapsed_time(b) for a, b in ev)


def _read_floor(L, buf, read_bytes, sizes, sink, stream, reps=30):
    """Median microseconds of plain reads of `sizes` bytes (one launch each,
    back to back), or None if the windows do not fit the buffer often enough
    to leave the last-level cache behind."""
    import torch

    sizes = [int(s) // 4096 * 4096 for s in sizes if s >= 4096]
    total = sum(sizes)
    nwin = read_bytes // total if total else 0
    if nwin < 2 or nwin * total < (1 << 30):
        return None
    base = buf.data_ptr()
    ev = []
    for rep in range(reps + 2):
        o = base + (rep % nwin) * total
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for s in sizes:
            rc = L.moe_peaks_read(ctypes.c_void_p(o), s, ctypes.c_void_p(sink.data_ptr()), 2048, stream)
            if rc != 0:
                raise RuntimeError(f"moe_peaks_read: hip error {rc}")
            o += s
        e1.record()
        ev.append((e0, e1))
    torch.cuda.synchronize()
    us = sorted(a.elapsed_time(b) * 1e3 for a, b in ev[2:])
    return us[len(us) // 2]


def measure(read_bytes: int = 2 << 30, reps: int = 10, mfma_iters: int = 8192, read_sequence=None) -> dict:
    import torch

    L = lib()
    dev = torch.cuda.current_device()
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    buf = torch.ones(read_bytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(max(1, 4 * cus), dtype=torch.float32, device="cuda")
    rblocks = 8 * cus

    def read():
        rc = L.moe_peaks_read(ctypes.c_void_p(buf.data_ptr()), read_bytes, ctypes.c_void_p(sink.data_ptr()), rblocks,
                              stream)
        if rc != 0:
            raise RuntimeError(f"moe_peaks_read: hip error {rc}")

    mblocks = 4 * cus

    def mfma():
        rc = L.moe_peaks_mfma(mblocks, mfma_iters, ctypes.c_void_p(sink.data_ptr()), stream)
        if rc != 0:
            raise RuntimeError(f"moe_peaks_mfma: hip error {rc}")

    ms_read = _timed(read, reps)
    ms_mfma = _timed(mfma, reps)
    floor = _read_floor(L, buf, read_bytes, read_sequence, sink, stream) if read_sequence else None
    waves = mblocks * L.moe_peaks_mfma_threads() // 64
    flops = waves * mfma_iters * L.moe_peaks_mfma_chains() * MFMA_FLOPS
    del buf
    out = {}
    if floor is not None:
        out = {"read_floor_us": floor, "read_floor_launch_bytes": [int(b) for b in read_sequence]}
    return {
        **out,
        "hbm_read_GBps": read_bytes / (ms_read * 1e-3) / 1e9,
        "mfma_f16_TFLOPs": flops / (ms_mfma * 1e-3) / 1e12,
        "compute_units": cus,
        "method": (f"read: {read_bytes >> 20} MiB of 16-B non-temporal loads, {rblocks} workgroups; "
                   f"mfma: v_mfma_f32_32x32x16_f16 from registers, {mblocks} workgroups x 4 waves x "
                   f"{L.moe_peaks_mfma_chains()} accumulators x {mfma_iters} iterations; "
                   f"HIP events per launch, best of {reps} after 2"),
    }


if __name__ == "__main__":
    import json

    print(json.dumps(measure()))
