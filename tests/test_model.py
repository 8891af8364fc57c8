"""The FLOP / traffic model the benchmark reports with, pinned to the figures
the pages print (tests/golden/paper_figures.txt, each line cited)."""
import os

import pytest

from fp32_sgemm_tuning_amd import model

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "paper_figures.txt")


def _load():
    vals, text = {}, {}
    for line in open(GOLDEN):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        k, v = (s.strip() for s in line.split("=", 1))
        vals[k] = float(v)
        text[k] = v
    return vals, text


G, GTEXT = _load()


def _half_ulp(key):
    """Half a unit in the last printed digit of a golden figure."""
    t = GTEXT[key]
    d = len(t.split(".", 1)[1]) if "." in t else 0
    return 0.5 * 10.0 ** (-d)


N4 = 4096


def test_flop_count_4096():
    f = model.flops(N4, N4, N4)
    assert f == 137_438_953_472
    assert f / 1e9 == pytest.approx(G["flops_4096_gflop"], abs=0.005)
    assert round(f / 1e9) == G["flops_4096_gflop_course"]
    # 137 GFLOP at the course card's 30.9 TFLOP/s peak is about 4.4 ms
    assert f / (G["course_peak_tflops"] * 1e12) * 1e3 == pytest.approx(G["course_peak_time_ms"], abs=0.05)


def test_tile_traffic_model():
    assert model.tile_loads_per_output(N4, 128, 128) == G["tile128_loads_per_output"]
    total = model.tile_global_bytes(N4, N4, N4, 128, 128)
    assert total / 1e9 == pytest.approx(G["tile128_total_gb"], abs=0.005)
    ai = model.arithmetic_intensity(model.flops(N4, N4, N4), total)
    assert ai == pytest.approx(G["tile128_intensity"], rel=1e-12)
    assert model.register_tile_loads_per_output(N4, 8, 8) == G["regtile8_loads_per_output"]
    # square tiles minimise traffic at fixed area
    assert model.tile_loads_per_output(N4, 128, 128) < model.tile_loads_per_output(N4, 256, 64)


def test_intensity_figures():
    # naive: 2 FLOP per two 4-byte loads
    assert model.arithmetic_intensity(2, 2 * model.FP32_BYTES) == G["naive_intensity"]
    # T x T tiles: 2K/T loads per output of 2K FLOP -> T/4 FLOP/B
    for T, key in [(16, "tiled16_intensity"), (32, "tiled32_intensity")]:
        K = 4096
        loads = model.tile_loads_per_output(K, T, T)
        assert model.arithmetic_intensity(2 * K, loads * model.FP32_BYTES) == G[key]


def test_c_read_bytes():
    assert model.c_read_bytes(N4, N4) / 1e6 == pytest.approx(G["c_read_mb"], abs=0.5)
    assert model.min_hbm_bytes(N4, N4, N4, True) - model.min_hbm_bytes(N4, N4, N4, False) == \
        model.c_read_bytes(N4, N4)


@pytest.mark.parametrize("ms,thr,scale", [
    ("rtx3060_cublas_ms", "rtx3060_cublas_tflops", 1.0),
    ("rtx3060_staged_ms", "rtx3060_staged_tflops", 1.0),
    ("regtile_kernel_ms", "regtile_kernel_gflops", 1e3),
    ("final_kernel_ms", "final_kernel_gflops", 1e3),
])
def test_printed_time_throughput_pairs(ms, thr, scale):
    got = model.tflops(N4, N4, N4, G[ms] * 1e-3) * scale
    # the printed time and the printed rate are each rounded to their last digit
    tol = _half_ulp(thr) + got * _half_ulp(ms) / G[ms]
    assert abs(got - G[thr]) <= tol


def test_bench_quotes_the_pages_figures():
    """The context figures on the bench line are the ones the pages print."""
    import bench
    c = bench.PAGES_CONTEXT
    assert c["rtx3060_vendor_library_tflops"] == G["rtx3060_cublas_tflops"]
    assert c["rtx3060_pipelined_kernel_tflops"] == G["rtx3060_staged_tflops"]
    assert c["rtx3060_locked_clock_mhz"] == G["rtx3060_locked_clock_mhz"]
    assert c["t4_shared_memory_tile32_tflops"] == pytest.approx(G["t4_tile32_4096_gflops"] / 1000.0)
