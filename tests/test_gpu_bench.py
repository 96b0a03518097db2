"""bench.py's command line on the GPU: the JSON line it prints keeps the
contract fields for the fwd+bwd workloads (with the HIP-graph timing) and
for the decode workload."""

import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CONTRACT = ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
            "scaling", "vs_baseline", "dtype", "data", "config", "roofline")


def run_bench(*args):
    print(f"[case] bench.py {' '.join(args)}", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1",
                        "--no-cpu-baseline", *args], capture_output=True, text=True, timeout=110, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    line = [l for l in r.stdout.splitlines() if l.startswith("{")][-1]
    d = json.loads(line)
    for k in CONTRACT:
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1 and d["value"] > 0
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in d["roofline"], k
    return d


def test_bench_fwd_bwd_line_with_graph_timing():
    d = run_bench("--workload", "gpt2", "--graph")
    assert d["unit"] == "TFLOP/s" and d["graph_ms_per_step"] > 0 and d["graph_tflops"] > 0


def test_bench_decode_line():
    d = run_bench("--workload", "decode")
    assert d["unit"] == "GB/s" and d["roofline"]["bound"] == "hbm"
