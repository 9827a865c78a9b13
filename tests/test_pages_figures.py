"""The host-side roofline arithmetic reproduces the figures the pages print
(tests/golden/pages_figures.json, each entry citing where it is printed)."""
import json
import math
import os

import pytest

from dense_gemm_epilogue_tiled_amd import roofline as rl

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")))


def check(name, got):
    g = GOLDEN[name]
    rel = g.get("rel")
    if rel is None:
        # integer figures: the printed value is the rounded result
        assert round(got) == g["value"], (name, got)
    else:
        assert abs(got - g["value"]) <= rel * abs(g["value"]), (name, got)


def test_shared_memory_bill():
    check("smem_bill_128x128x32_3stages_bytes", rl.pipelined_tile_smem_bytes(128, 128, 32, 3))
    check("smem_bill_128x128x32_8stages_bytes", rl.pipelined_tile_smem_bytes(128, 128, 32, 8))


def test_tile_intensity():
    check("tile_intensity_128x128", rl.tile_step_intensity(128, 128))
    check("tile_intensity_256x256", rl.tile_step_intensity(256, 256))
    assert math.floor(rl.tile_step_intensity(128, 256)) == GOLDEN["tile_intensity_128x256"]["value"]


def test_ridge_point():
    check("a100_ridge_flop_per_byte", rl.ridge_flop_per_byte(312, 2))


def test_gemm4096_case():
    n = 4096
    check("gemm4096_flops", rl.algorithmic_flops(n, n, n))
    check("gemm4096_time_at_312tflops_ms", rl.time_at_peak_s(n, n, n, 312) * 1e3)
    check("gemm4096_whole_problem_intensity", rl.whole_problem_intensity(n, n, n))
    check("gemm4096_ideal_traffic_bytes", rl.ideal_traffic_bytes(n, n, n))
    per_tile = rl.per_tile_traffic_bytes(n, n, n, 128, 128)
    check("gemm4096_per_tile_traffic_128x128_bytes", per_tile)
    check("gemm4096_traffic_ratio", per_tile / rl.ideal_traffic_bytes(n, n, n))
    need = rl.ridge_flop_per_byte(312, 2) / rl.tile_step_intensity(128, 128)
    check("reuse_needed_to_pass_ridge", need)
    # fraction of 32 readers that must hit: 1 - 1/need
    check("l2_readers_hitting_of_32", 32 * (1 - 1 / need))


def test_mi355x_denominators():
    assert rl.MI355X_MFMA_F16_TFLOPS == pytest.approx(256 * 4096 * 2.4e9 / 1e12, rel=1e-4)
    assert rl.MI355X_HBM_GBS == 8000.0
