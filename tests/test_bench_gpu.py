"""bench.py's output line on the GPU: one JSON line with the fields the
measurement contract asks for, a roofline whose fraction is its achieved rate
over the peak, the oracle timed as the CPU baseline, and the other workloads'
figures.  A short run (few steps, one other workload)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.gpu
def test_bench_line_fields():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "5", "--warmup", "2",
                        "--instances", "1", "--cpu-budget", "1", "--others", "tiny"],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, lines
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline", "kernels"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 2
    assert d["data"] == "synthetic" and d["config"]["workload"] == "llama32k"
    assert d["value"] > 0 and d["ms_per_step"] > 0
    roof = d["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert abs(roof["achieved"] - roof["bytes_per_launch"] / (roof["us_per_launch"] * 1e-6) / 1e9) < 0.01 * roof["achieved"]
    if roof["traffic"] is not None:   # counted bytes of the current sources: at most a few % above the algorithmic
        assert roof["bytes_per_launch"] <= roof["traffic"] <= 1.05 * roof["bytes_per_launch"]
    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1 and cpu["sample"]
    others = d["other_workloads"]
    assert [o["workload"] for o in others] == ["tiny"]
    assert others[0]["ms_per_step"] > 0 and others[0]["kernels"]
