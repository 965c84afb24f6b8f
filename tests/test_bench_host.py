"""Host checks of bench.py's algorithmic accounting (no GPU): over each
launch sequence the per-kernel weight bytes add up to the step's -- every
touched expert and the router counted exactly once -- and one more
distinct routed expert adds exactly one expert's three matrices."""

from __future__ import annotations

import pytest

import bench
from mixture_experts_ffn_rmsnorm_amd import inputs as gen

PATHS = {
    "decode, 2 to 4 rows": ("dec_head", "dec_gateup", "dec_down_reduce"),
    "decode, 1 row": ("dec1_router", "dec1_gateup", "dec1_down_reduce"),
    "prefill": ("pre_norm", "pre_router", "pre_sort", "gemm_gateup_swiglu", "gemm_down",
                "gemm_down_shared_reduce"),
}


def _sum(kernels, cfg, U, R):
    return sum(bench.alg_bytes(k, cfg, U, R) or 0 for k in kernels)


@pytest.mark.parametrize("path", sorted(PATHS))
@pytest.mark.parametrize("cfg_i", [0, 1])
def test_weight_bytes_add_up(path, cfg_i):
    cfg = gen.config(cfg_i)
    H, I, E = cfg.hidden, cfg.inter, cfg.experts
    expert = 3 * H * I * 2
    for U in (0, 1, 6, 23):
        # with no rows only weights remain (plus the f32 norm weight and bias)
        w = _sum(PATHS[path], cfg, U, 0)
        assert (U + 1) * expert + E * H * 2 <= w <= (U + 1) * expert + E * H * 2 + H * 4 + E * 4, (path, U)
        for R in (1, 4, 512):
            assert _sum(PATHS[path], cfg, U + 1, R) - _sum(PATHS[path], cfg, U, R) == expert, (path, U, R)


def test_step_bytes_match_the_paths():
    cfg = gen.config(1)
    for U in (6, 23):
        for path in PATHS.values():
            assert abs(_sum(path, cfg, U, 0) - bench.step_bytes(cfg, U, 0)) <= cfg.hidden * 4 + cfg.experts * 4
