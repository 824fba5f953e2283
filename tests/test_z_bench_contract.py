"""The one-line JSON contract of bench.py.

On the CPU: more than one GPU is refused with a message and a non-zero exit,
before anything touches a GPU.  On the GPU: a short default run prints one
JSON line with the metric, the roofline of the attention kernel and the CPU
oracle baseline, with consistent values.
"""
import json
import math
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, timeout=600):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=timeout, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _bench("--gpus", "2", timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.gpu
def test_default_run_prints_the_contract_line():
    r = _bench("--steps", "5", "--warmup", "2", "--cpu-seconds", "2", timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 2
    assert d["unit"] == "steps/s" and d["higher_is_better"] is True
    assert d["vs_baseline"] is None and d["data"] == "synthetic" and d["dtype"] == "bf16"
    assert d["config"]["workload"].startswith("cfg2")
    assert math.isclose(d["value"], 1e3 / d["ms_per_step"], rel_tol=1e-9)
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert 0.0 < rf["frac"] < 1.0
    assert math.isclose(rf["frac"], rf["achieved"] / rf["peak"], rel_tol=1e-9)
    assert math.isclose(rf["achieved"],
                        rf["algorithmic_bytes_per_launch"] / rf["avg_launch_us"] / 1e3,
                        rel_tol=1e-9)
    assert rf["traffic"] is None or rf["traffic"] > 0
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
