"""Host checks of bench.py's algorithmic accounting (no GPU): over each
launch sequence the per-kernel weight bytes add up to the step's -- every
touched expert and the router counted exactly once -- and one more
distinct routed expert adds exactly one expert's three matrices."""

from __future__ import annotations

import pytest

import bench
from mixture_experts_ffn_rmsnorm_amd import inputs as gen

PATHS = {
    "decode, 2 to 4 rows": ("dec_head", "dec_gateup", "dec_down", "dec_reduce"),
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


def test_profiled_kernel_names_map_to_launch_names():
    """rocprofv3 reports demangled template names; each of the library's
    kernels maps to the launch name the stage timer and bench.py use."""
    from mixture_experts_ffn_rmsnorm_amd import profiling

    ns = "void moe::(anonymous namespace)::"
    cases = {
        "k_dec_head<4096, 2048, false, 0>(moe::FwdArgs)": "dec_head",
        "k_dec_head<4096, 2048, true, 0>(moe::FwdArgs)": "dec1_router",
        "k_dec_head<4096, 2048, true, 1>(moe::FwdArgs)": "dec1_router_mx",
        "k_dec_head<4096, 2048, true, 2>(moe::FwdArgs)": "dec1_router_mx4",
        "k_dec_gateup<4096, 2048, 0>(moe::FwdArgs)": "dec_gateup",
        "k_dec_gateup<4096, 2048, 1>(moe::FwdArgs)": "dec_gateup_mx",
        "k_dec1_gateup<512, 256, 0>(moe::FwdArgs)": "dec1_gateup",
        "k_dec1_gateup<4096, 2048, 2>(moe::FwdArgs)": "dec1_gateup_mx4",
        "k_dec_down<4096, 2048, 0>(moe::FwdArgs)": "dec_down",
        "k_dec_reduce<4096>(moe::FwdArgs)": "dec_reduce",
        "k_dec1_down<512, 256, 0>(moe::FwdArgs)": "dec1_down_reduce",
        "k_dec1_down<4096, 2048, 1>(moe::FwdArgs)": "dec1_down_reduce_mx",
        "k_dec1_down<4096, 2048, 2>(moe::FwdArgs)": "dec1_down_reduce_mx4",
        "k_dec_down<512, 256, 2>(moe::FwdArgs)": "dec_down_mx4",
        "k_pre_norm<4096>(moe::FwdArgs)": "pre_norm",
        "k_pre_router<4096, 256, 8>(moe::FwdArgs)": "pre_router",
        "k_pre_sort(moe::FwdArgs)": "pre_sort",
        "k_gemm<0, 4096, 2048, moe::(anonymous namespace)::GemmCfg<64, 1, 128, 1, 128, 3, 4, 512>, 0>(moe::FwdArgs)":
            "gemm_gateup_swiglu",
        "k_gemm<0, 4096, 2048, moe::(anonymous namespace)::GemmCfg<64, 1, 128, 1, 128, 3, 4, 512>, 1>(moe::FwdArgs)":
            "gemm_gateup_swiglu_mx",
        "k_gemm<1, 2048, 4096, moe::(anonymous namespace)::GemmCfg<256, 4, 256, 2, 64, 2, 4, 512>, 0>(moe::FwdArgs)":
            "gemm_down",
        "k_gemm<2, 2048, 4096, moe::(anonymous namespace)::GemmCfg<256, 4, 256, 2, 64, 2, 4, 512>, 1>(moe::FwdArgs)":
            "gemm_down_shared_reduce_mx",
        "k_route(moe::RouteArgs)": "route",
        "k_hc_mix<4>(moe::HcArgs)": "hc_mix",
        "k_hc_mix_mfma<3>(moe::HcArgs)": "hc_mix",
        "k_hc_pre<4>(moe::HcArgs)": "hc_pre",
        "k_hc_post<2>(moe::HcArgs)": "hc_post",
    }
    for kernel, name in cases.items():
        assert profiling.launch_name(ns + kernel) == name, kernel
    assert profiling.launch_name("__amd_rocclr_copyBuffer") is None
    # every launch name has an algorithmic byte count in bench.py (route aside)
    cfg = gen.config(1)
    for name in set(cases.values()) - {"route"}:
        assert bench.alg_bytes(name, cfg, 6, 4) is not None, name
