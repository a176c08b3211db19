"""bench.py's output contract: one JSON line with the fields the benchmark
runner reads, and a clear refusal of more than one GPU.

The GPU cases run bench.py as a child process on small workloads."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""


def _run(*args):
    print(f"[bench-contract] {' '.join(args)}", flush=True)
    r = subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout
    return json.loads(lines[0])


@pytest.mark.gpu
@pytest.mark.timeout(600)
@pytest.mark.parametrize("workload", ["flux_512", "tiny_fp32"])
def test_bench_json_line(workload):
    d = _run("--workload", workload, "--steps", "3", "--warmup", "1", "--no-cpu-baseline", "--settle-ms", "20")
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
              "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["unit"] == "tokens/s" and d["higher_is_better"] is True and d["scaling"] == "weak"
    assert d["vs_baseline"] is None and d["cpu_baseline"] is None and d["data"] == "synthetic"
    assert d["config"]["workload"] == workload
    assert d["value"] > 0 and d["ms_per_step"] > 0
    w = d["config"]
    assert abs(d["value"] - w["B"] * w["N"] / (d["ms_per_step"] * 1e-3)) <= 1e-6 * d["value"]
    rl = d["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in rl, k
    assert rl["bound"] in ("hbm", "mfma") and rl["peak"] > 0
    assert abs(rl["frac"] - rl["achieved"] / rl["peak"]) < 1e-9
    assert d["dtype"] == ("f32" if workload == "tiny_fp32" else "bf16")
