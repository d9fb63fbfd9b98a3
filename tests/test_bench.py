"""bench.py's contract: one GPU only, the oracle baseline's fields, and (on a GPU) one JSON line
carrying the metric, the roofline of the dominant kernel and the workload's configuration."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "measures one GPU" in r.stderr and r.stdout == ""


def test_cpu_baseline_fields():
    sys.path.insert(0, ROOT)
    import bench
    from workloads import WORKLOADS, gen
    cb = bench.cpu_baseline(WORKLOADS["tiny_fp32_b1_k2"], gen, seconds_target=0.1, max_steps=2)
    assert cb["kind"] == "oracle" and cb["unit"] == "verified tokens/s"
    assert cb["value"] > 0 and cb["cores"] >= 1 and cb["blas_threads"] >= 1
    assert cb["cpu_model"] and "verify steps" in cb["sample"]


@pytest.mark.gpu
def test_bench_line_on_the_tiny_workload():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload",
                        "tiny_fp32_b1_k2", "--steps", "3", "--warmup", "1", "--no-cpu-baseline"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    d = json.loads(lines[-1])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "hbm_ceiling"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["dtype"] == "f32"
    assert d["config"]["workload"] == "tiny_fp32_b1_k2"
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert rf["achieved"] > 0 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
