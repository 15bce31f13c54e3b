"""The benchmark's output contract: one JSON line with the metric, the roofline
object and (unless switched off) the CPU baseline; one GPU only."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args, timeout=300):
    return subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=timeout)


def test_bench_refuses_several_gpus():
    r = _run("--gpus", "2", timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.gpu
def test_bench_json_line():
    r = _run("--workload", "bf16_n256_d64_short", "--steps", "2", "--warmup", "1", "--no-cpu-baseline")
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout
    out = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
                "vs_baseline", "dtype", "data", "config", "roofline"):
        assert key in out, key
    assert out["n_gpus"] == 1 and out["steps"] == 2 and out["warmup"] == 1
    assert out["value"] > 0 and out["ms_per_step"] > 0 and out["higher_is_better"] is True
    assert out["config"]["workload"] == "bf16_n256_d64_short"
    roof = out["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert 0 < roof["frac"] < 1 and abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert "cpu_baseline" not in out
    host = out["host"]
    for key in ("cpu_model", "cpu_count", "affinity_cpus", "gpu_clock_mhz_avg", "gpu_clock_samples",
                "gpu_clock_source"):
        assert key in host, key
    assert host["cpu_count"] >= host["affinity_cpus"] >= 1
