"""bench.py's contract: the one-GPU refusal (CPU) and, on a GPU, one JSON line
per workload with every field the measurement needs (value, step time,
roofline object with its peak and fraction, cpu_baseline key)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


_KEYS = ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
         "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config", "roofline",
         "cpu_baseline")


@pytest.mark.gpu
@pytest.mark.parametrize("args", [
    ["--steps", "2", "--warmup", "1", "--no-cpu-baseline"],
    ["--workload", "block_L8192", "--steps", "2", "--warmup", "1", "--no-cpu-baseline"],
    ["--workload", "io_L8192", "--steps", "3", "--warmup", "1"],
])
def test_bench_prints_one_complete_json_line(args):
    print("bench", " ".join(args), flush=True)
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), *args],
                       capture_output=True, text=True, timeout=280)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    j = json.loads(lines[0])
    for k in _KEYS:
        assert k in j, k
    assert j["value"] > 0 and j["ms_per_step"] > 0 and j["n_gpus"] == 1
    assert j["steps"] == int(args[args.index("--steps") + 1])
    assert "workload" in j["config"]
    rf = j["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in rf, k
    assert rf["peak"] > 0 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
