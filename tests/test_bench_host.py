"""Host logic of bench.py (no GPU): algorithmic work per stage, the stage
roofline arithmetic, and the one-GPU guard."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from token_routing_shuffle_amd import workload as wl  # noqa: E402


def test_algorithmic_work_of_the_bench_layer():
    cfg = wl.CONFIGS["dsv2lite"]
    A = cfg.T * cfg.k
    alg = bench.algorithmic(cfg, A)
    T, H, I, Ish = cfg.T, cfg.H, cfg.I, cfg.n_shared * cfg.I_shared
    # GEMM1: gate and up projections of every routed row and of the shared FFN
    assert alg["ffn_up_flops"] == 2 * A * H * 2 * I + 2 * T * H * 2 * Ish == 377957122048
    assert alg["ffn_down_flops"] == alg["ffn_up_flops"] / 2
    assert alg["dispatch_bytes"] == T * H * 2 + A * H * 2 + 8 * T + 12 * A
    assert alg["combine_bytes"] == A * H * 2 + 8 * A + 2 * T * H * 2


def test_stage_rooflines_fractions():
    cfg = wl.CONFIGS["dsv2lite"]
    A = cfg.T * cfg.k
    alg = bench.algorithmic(cfg, A)
    ms = {"route": 0.02, "shuffle": 0.025, "gather": 0.0, "ffn_up": 0.4, "ffn_down": 0.2, "combine": 0.025}
    r = bench.stage_rooflines(cfg, A, alg, ms, 0.378)
    up = r["ffn_up"]
    assert up["bound"] == "mfma"
    assert up["achieved_tflops"] == pytest.approx(alg["ffn_up_flops"] / 0.378e-3 / 1e12, rel=1e-3)
    assert up["frac"] == pytest.approx(up["achieved_tflops"] / bench.BF16_MFMA_PEAK_TFLOPS, rel=1e-3)
    comb = r["combine"]
    assert comb["achieved_gbs"] == pytest.approx(alg["combine_bytes"] / 0.025e-3 / 1e9, rel=1e-3)
    assert comb["frac"] == pytest.approx(comb["achieved_gbs"] / bench.HBM_PEAK_GBS, rel=1e-3)
    # the combine's 134 MB fit in the 256 MB Infinity Cache
    assert comb["mall_resident"]
    assert 0 < r["route"]["mfma_frac"] < r["route"]["frac"] < 1


def test_binding_roofline_of_the_headline_layer():
    """DeepSeek-V3-shaped prefill GEMM1: 15.5 GB of algorithmic bytes (all
    256 experts' W1/W3, the shared W1/W3, x once, the SwiGLU outputs) take
    1.94 ms at 8 TB/s, longer than its 4.33 TFLOP at 2.5 PFLOP/s (1.73 ms):
    HBM is the binding roof."""
    cfg = wl.CONFIGS["dsv3_prefill"]
    A = cfg.T * cfg.k
    alg = bench.algorithmic(cfg, A)
    T, H, I, Ish, E = cfg.T, cfg.H, cfg.I, cfg.I_shared, cfg.E
    assert alg["ffn_up_bytes"] == 2 * (E * 2 * I * H + 2 * Ish * H + T * H + A * I + T * Ish)
    r = bench.binding_roofline(alg["ffn_up_flops"], alg["ffn_up_bytes"], 4.9)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == bench.HBM_PEAK_GBS
    assert r["roof_ms"] == pytest.approx(alg["ffn_up_bytes"] / 8e12 * 1e3, rel=1e-3)
    assert r["frac"] == pytest.approx(r["roof_ms"] / 4.9, rel=1e-3)
    assert r["mfma_frac"] < r["frac"]
    # fewer touched experts, fewer weight bytes
    assert bench.algorithmic(cfg, A, 200)["ffn_up_bytes"] < alg["ffn_up_bytes"]
    # the DeepSeek-V2-Lite-shaped layer's GEMM1 is MFMA-bound
    c2 = wl.CONFIGS["dsv2lite"]
    a2 = bench.algorithmic(c2, c2.T * c2.k)
    assert bench.binding_roofline(a2["ffn_up_flops"], a2["ffn_up_bytes"], 0.37)["bound"] == "mfma"


def test_default_workload_is_the_largest_layer():
    assert bench.parse([]).workload == "dsv3_prefill"
    big = max(wl.CONFIGS.values(), key=lambda c: bench.algorithmic(c, c.T * c.k)["ffn_up_flops"])
    assert big.name == bench.WORKLOAD
    assert "DeepSeek-V3-shaped" in bench.describe(big) and "T=8192" in bench.describe(big)
    assert set(bench.OTHER_LAYERS) | {bench.WORKLOAD} == set(wl.CONFIGS)


def test_cpu_info():
    n, model = bench.cpu_info()
    assert n >= 1 and isinstance(model, str) and model


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout == ""
