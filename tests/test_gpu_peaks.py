"""The device-ceiling microbenchmarks on the GPU: both measured rates are
positive and below MI355X's published peaks plus a small margin (a reading
above them would mean the kernels skip work or the caches serve the read)."""

from __future__ import annotations

import pytest

pytestmark = pytest.mark.gpu


def test_measured_peaks_are_plausible():
    from mixture_experts_ffn_rmsnorm_amd import device_peaks

    pk = device_peaks.measure(read_bytes=1 << 30, reps=3, mfma_iters=2048)
    print(pk)
    assert 1000.0 < pk["hbm_read_GBps"] < 8000.0 * 1.05
    assert 200.0 < pk["mfma_f16_TFLOPs"] < 2516.6 * 1.05
