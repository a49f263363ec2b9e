"""bench.py's output line on the GPU: the fields the benchmark contract names,
for the headline workload and for an HBM-bound small one."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
pytestmark = pytest.mark.gpu


def run_bench(*args):
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), *args],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    return json.loads(lines[0])


def test_headline_line_has_the_contract_fields():
    rec = run_bench("--steps", "5", "--warmup", "5", "--cpu-budget", "0.5")
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in rec, key
    assert rec["n_gpus"] == 1 and rec["steps"] == 5 and rec["warmup"] == 5
    assert rec["unit"] == "TFLOP/s" and rec["dtype"] == "bf16" and rec["higher_is_better"]
    assert rec["config"]["workload"] == "prefill_h32_s4096_d128"
    assert rec["value"] > 0
    ro = rec["roofline"]
    assert ro["bound"] == "mfma" and ro["unit"] == "TFLOP/s" and ro["peak"] == 2516.6
    assert 0 < ro["frac"] < 1 and abs(ro["frac"] - ro["achieved"] / ro["peak"]) < 1e-3
    assert ro["flops_per_launch"] == 4 * 32 * 4096 * 4096 * 128 / 2
    assert ro["traffic"] is None or ro["traffic"] > ro["compulsory_bytes_per_launch"] * 0.9
    cb = rec["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["unit"] == "TFLOP/s" and cb["value"] > 0
    assert cb["cores"] >= 1 and cb["sample"]


def test_hbm_bound_workload_reports_bandwidth():
    rec = run_bench("--workload", "stress_b3h2_d32_skv1000", "--splits", "0",
                    "--steps", "5", "--warmup", "5", "--cpu-budget", "0")
    ro = rec["roofline"]
    assert ro["bound"] == "hbm" and ro["unit"] == "GB/s" and ro["peak"] == 8000.0
    assert rec["config"]["key_chunks"] > 1
    assert "cpu_baseline" not in rec


def test_mfma_probe_line():
    # the matrix-core rate probe: constant operands must run at least as fast
    # as random ones, and nothing may beat the published peak
    rec = run_bench("--mfma-probe", "400")
    for name in ("mfma_zero", "mfma_random", "mfma_lds_zero", "mfma_lds_random"):
        r = rec[name]
        assert 0 < r["frac_of_peak"] <= 1.0, (name, r)
    assert rec["mfma_zero"]["tflops"] >= 0.9 * rec["mfma_random"]["tflops"]


def test_launch_series_line():
    # the cold-start series: one positive time per launch, window means that
    # agree with the times
    rec = run_bench("--launch-series", "12", "--workload", "single_head_s64_d32")
    us = rec["us"]
    assert rec["launch_series"] == 12 and len(us) == 12 and all(t > 0 for t in us)
    assert rec["us_mean"]["6-25"] == round(sum(us[5:]) / len(us[5:]), 2)
