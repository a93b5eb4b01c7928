"""The benchmark's output contract.

CPU: more than one GPU is refused with a message (exit status 2), before
anything touches a GPU.  GPU: a short run prints one JSON line whose fields
agree with each other: the whole-job rate is the step FLOPs over the wall time
per step, the roofline fraction is achieved over peak, the kernel time from
events fits inside the wall time per step, the MFMA-loop fraction is the
kernel rate over the measured loop rate, and a decoding workload (HBM-bound)
is reported in GB/s against 8 TB/s.
"""
import json
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]


def run_bench(*args, timeout=300):
    return subprocess.run([sys.executable, str(ROOT / "bench.py"), *args], capture_output=True,
                          text=True, timeout=timeout, cwd=str(ROOT))


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2", timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def last_json(stdout):
    lines = [l for l in stdout.splitlines() if l.startswith("{")]
    assert lines, stdout
    return json.loads(lines[-1])


@pytest.mark.gpu
def test_headline_line_is_consistent():
    r = run_bench("--steps", "5", "--warmup", "2", "--cold-steps", "2", "--no-cpu-baseline")
    assert r.returncode == 0, r.stderr[-2000:]
    d = last_json(r.stdout)
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config", "roofline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 2
    assert d["unit"] == "TFLOP/s" and d["dtype"] == "bf16" and d["higher_is_better"] is True
    assert d["config"]["workload"].startswith("C4")
    flops = d["config"]["flops_per_step"]
    assert flops == 4.0 * 16 * 16384 * 16384 * 64
    assert abs(d["value"] - flops / (d["ms_per_step"] * 1e-3) / 1e12) <= 0.01 * d["value"]
    rf = d["roofline"]
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s" and rf["peak"] == 2500.0
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert rf["kernel_ms_avg"] <= d["ms_per_step"] * 1.05
    assert abs(rf["achieved"] - flops / (rf["kernel_ms_avg"] * 1e-3) / 1e12) <= 0.01 * rf["achieved"]
    assert rf["kernel_ms_cold_median"] is not None
    assert 1000.0 < rf["mfma_loop_tflops"] <= 2516.6 * 1.02
    assert abs(rf["frac_of_mfma_loop"] - rf["achieved"] / rf["mfma_loop_tflops"]) < 1e-3


@pytest.mark.gpu
def test_decoding_line_is_hbm_bound():
    r = run_bench("--workload", "D1", "--steps", "5", "--warmup", "2", "--cold-steps", "0",
                  "--no-cpu-baseline")
    assert r.returncode == 0, r.stderr[-2000:]
    d = last_json(r.stdout)
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert "mfma_loop_tflops" not in rf
