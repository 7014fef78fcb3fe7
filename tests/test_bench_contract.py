"""bench.py's output contract: one JSON line on stdout with the metric, the timed steps, the roofline block of the
dominant kernel and the per-kernel figures, from a short run (few steps, no prefill, no oracle leg) in a child
process on the GPU; and the refusal of a run on more than one GPU (host only)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_bench_refuses_more_than_one_gpu():
    p = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    out = json.loads(p.stdout.strip().splitlines()[-1])
    assert out["n_gpus"] == 2 and "one GPU" in out["error"]


@pytest.mark.gpu
def test_bench_json_line():
    cmd = [sys.executable, "-u", BENCH, "--steps", "40", "--warmup", "5", "--no-prefill", "--no-q4k",
           "--no-cpu-baseline", "--verify-steps", "5", "--no-sweep", "--kernel-reps", "40"]
    print("[bench-contract] " + " ".join(cmd[2:]), flush=True)
    p = subprocess.run(cmd, capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert p.returncode == 0, p.stderr[-3000:]
    lines = [ln for ln in p.stdout.strip().splitlines() if ln.strip()]
    assert len(lines) == 1, p.stdout[-2000:]
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
                "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline", "decode_kernels",
                "decode_latency", "verify"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 40 and d["warmup"] == 5
    assert d["unit"] == "tokens/s" and d["higher_is_better"] is True and d["value"] > 0
    assert abs(d["value"] - 1e3 / d["ms_per_step"]) <= 0.01 * d["value"]
    assert d["config"]["timed_tokens"] == 40 and "workload" in d["config"]
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    # achieved = the algorithmic bytes of one launch over its measured duration
    assert abs(r["achieved"] - r["bytes_per_launch"] / r["avg_launch_us"] / 1e3) <= 0.002 * r["achieved"]
    assert r["traffic"] is None or r["traffic"] >= r["bytes_per_launch"]
    assert d["cpu_baseline"] is None                         # --no-cpu-baseline
    lat = d["decode_latency"]
    assert 0 < lat["p50_us"] <= lat["p99_us"] <= lat["max_us"]
