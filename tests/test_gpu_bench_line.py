"""The benchmark's JSON line on the GPU: exactly one line on stdout, the
contract's fields, and figures that agree with one another (algbw = S / T,
busbw = algbw * 2(N-1)/N, HBM rate = 2*N*S / T, the roofline fraction, the
ring steps' moved bytes, the counter traffic only from a summary of the same
sources)."""
import json
import os
import subprocess
import sys

import pytest

import bench

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                       timeout=300, cwd=ROOT)
    assert p.returncode == 0, p.stderr[-3000:]
    lines = [ln for ln in p.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, p.stdout
    return json.loads(lines[0])


def check_common(j, steps, warmup, workload):
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
              "vs_baseline", "dtype", "data", "config", "busbw", "hbm_gbps", "roofline", "copy_ceiling"):
        assert k in j, k
    assert j["unit"] == "GB/s" and j["n_gpus"] == 1
    assert j["steps"] == steps and j["warmup"] == warmup
    assert j["higher_is_better"] is True and j["scaling"] == "weak" and j["vs_baseline"] is None
    assert j["data"] == "synthetic"
    cfg = j["config"]
    assert isinstance(cfg["workload"], str) and cfg["workload"].startswith(workload)
    n, S = cfg["nranks"], cfg["bytes_per_rank"]
    assert S == cfg["count_per_rank"] * bench.ESIZE[j["dtype"]]
    T = j["ms_per_step"] * 1e-3
    assert T > 0
    # the printed figures are rounded to 6 significant digits
    assert j["value"] == pytest.approx(S / T / 1e9, rel=2e-3)
    assert j["busbw"] == pytest.approx(j["value"] * 2 * (n - 1) / n, rel=1e-4)
    assert j["hbm_gbps"] == pytest.approx(2 * n * S / T / 1e9, rel=2e-3)
    rf = j["roofline"]
    assert set(rf) >= {"bound", "achieved", "peak", "unit", "frac", "traffic"}
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert rf["achieved"] == pytest.approx(j["hbm_gbps"], rel=1e-6)
    assert rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"], abs=1e-4)
    assert 0 < rf["frac"] < 1
    cc = j["copy_ceiling"]
    assert 0 < cc["hbm_frac"] < 1
    assert cc["achieved_over_copy"] == pytest.approx(rf["frac"] / cc["hbm_frac"], rel=2e-3)
    return n, S, T


@pytest.mark.parametrize("mode", ["fused", "stepwise"])
def test_bench_line_sweep_point(mode):
    j = run_bench("--workload", "sweep256m", "--mode", mode, "--steps", "3", "--warmup", "1", "--no-cpu-baseline")
    n, S, T = check_common(j, 3, 1, "sweep point")
    assert j["dtype"] == "f32" and j["config"]["mode"] == mode
    # the counter traffic appears only while the sources match its summary
    assert j["roofline"]["traffic"] == bench.load_traffic("sweep256m", mode)
    sb = j["same_buffer_copy"]
    assert sb["achieved_over_copy"] == pytest.approx(sb["ms"] / j["ms_per_step"], rel=1e-3)
    if mode == "stepwise":
        mv = j["moved"]
        assert mv["bytes"] == bench.ring_moved_bytes(n, j["config"]["count_per_rank"], "f32")
        assert mv["gbps"] == pytest.approx(mv["bytes"] / T / 1e9, rel=2e-3)
    else:
        assert "moved" not in j


def test_bench_line_multi_tensor_bucket():
    j = run_bench("--workload", "bucket8", "--multi", "--steps", "3", "--warmup", "1", "--no-cpu-baseline")
    check_common(j, 3, 1, "bucket8")
    assert "ar_all_reduce_multi" in j["config"]["workload"]
    assert j["roofline"]["traffic"] is None  # counters are summarized for the flat call only


def test_bench_line_small_stepwise_steps():
    """The handbook's 4-rank shape defaults to the stepwise ring and reports
    each launch's device time and the per-step alpha."""
    j = run_bench("--workload", "small", "--steps", "5", "--warmup", "2", "--no-cpu-baseline")
    n, S, T = check_common(j, 5, 2, "small")
    assert n == 4 and S == 4096 * 4 and j["config"]["mode"] == "stepwise"
    rs = j["ring_steps"]
    assert rs["launches"] == 2 * (n - 1) and len(rs["step_us_median"]) == 2 * (n - 1)
    assert all(t > 0 for t in rs["step_us_median"])
    assert rs["alpha_device_us"] == pytest.approx(sum(rs["step_us_median"]) / (2 * (n - 1)), rel=1e-2, abs=0.01)
    assert rs["alpha_call_us"] == pytest.approx(j["ms_per_step"] * 1e3 / (2 * (n - 1)), rel=1e-3, abs=1e-3)


def test_bench_line_op_override():
    """--op replaces the workload's reduction op; the line names it, and
    reports no HBM-counter traffic (the committed counters are for the
    workload's own op)."""
    j = run_bench("--workload", "small", "--op", "prod", "--steps", "3", "--warmup", "1", "--no-cpu-baseline")
    assert j["config"]["op"] == "prod" and "PROD" in j["config"]["workload"]
    assert j["roofline"]["traffic"] is None


def test_range_point_fields():
    """One point of the metric-range block the default line carries."""
    import torch

    import ring_all_reduce_ar_amd as ar
    import synthetic
    p = bench.range_point(torch, ar, synthetic, "bucket25", 3, 1, copy_gbps=4000.0)
    n, S = p["nranks"], p["bytes_per_rank"]
    assert n == 8 and S == 6_553_600 * 4 and p["rotating_buffer_sets"] >= 6
    T = p["ms_per_step"] * 1e-3
    assert p["algbw_gbps"] == pytest.approx(S / T / 1e9, rel=2e-3)
    assert p["hbm_gbps"] == pytest.approx(2 * n * S / T / 1e9, rel=2e-3)
    assert p["hbm_frac"] == pytest.approx(p["hbm_gbps"] / 8000.0, abs=1e-4)
    assert p["achieved_over_copy"] == pytest.approx(p["hbm_gbps"] / 4000.0, rel=1e-3)
    assert p["first_allocation_ms_per_step"] > 0
    sb = p["same_buffer_copy"]
    assert sb["ms"] > 0 and sb["achieved_over_copy"] == pytest.approx(sb["ms"] / p["ms_per_step"], rel=1e-3)
    assert sb["hbm_frac"] == pytest.approx(2 * n * S / (sb["ms"] * 1e-3) / 8e12, rel=2e-3)
