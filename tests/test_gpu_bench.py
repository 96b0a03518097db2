"""bench.py's output contract on the GPU: one JSON line with the metric, the
whole-step throughput, the roofline object of the dominant kernel (achieved
over peak, measured on the kernel's own stream) and the oracle's CPU
baseline on a bounded sample; the decode line in GB/s; and the HIP-graph
replay timing of --graph."""

import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, timeout=240):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                       timeout=timeout, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [json.loads(l) for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    return lines[0]


def _roofline_consistent(d):
    rf = d["roofline"]
    assert rf["bound"] in ("mfma", "hbm") and rf["peak"] > 0 and rf["achieved"] > 0
    assert rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"], rel=2e-3)
    assert 0.0 < rf["frac"] < 1.0
    assert rf["traffic"] is None or rf["traffic"] > 0


@pytest.mark.timeout(300)
def test_default_line_contract():
    """The default workload (long causal, d = 128): the fields the contract
    names, a positive throughput, and a CPU baseline from a small sample."""
    print("[case] bench.py default workload, 3 steps, 512-row CPU sample", flush=True)
    d = _bench("--steps", "3", "--warmup", "1", "--cpu-rows", "512")
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1 and d["higher_is_better"] is True
    assert d["unit"] == "TFLOP/s" and d["dtype"] == "bf16" and d["value"] > 0 and d["ms_per_step"] > 0
    assert d["config"]["workload"].startswith("long")
    assert d["roofline"]["unit"] == "TFLOP/s" and d["roofline"]["kernel"] == "bwd_kv_kernel"
    _roofline_consistent(d)
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["unit"] == "TFLOP/s" and cb["value"] > 0 and cb["cores"] >= 1
    assert "512" in cb["sample"]
    print(f"[ok] {d['value']} TFLOP/s, frac {d['roofline']['frac']}, cpu {cb['value']}", flush=True)


@pytest.mark.timeout(300)
def test_decode_line_contract():
    """The decode workload reports HBM GB/s against the 8 TB/s roofline."""
    print("[case] bench.py --workload decode, 5 steps", flush=True)
    d = _bench("--workload", "decode", "--steps", "5", "--warmup", "1", "--no-cpu-baseline")
    assert d["unit"] == "GB/s" and d["value"] > 0 and d["config"]["workload"].startswith("decode")
    assert d["roofline"]["bound"] == "hbm" and d["roofline"]["unit"] == "GB/s"
    _roofline_consistent(d)
    print(f"[ok] decode {d['value']} GB/s, frac {d['roofline']['frac']}", flush=True)


@pytest.mark.timeout(300)
def test_graph_timing_line():
    """--graph: the same step captured once in a HIP graph and replayed, its
    time and throughput reported beside the eager ones (GPT-2 shape)."""
    print("[case] bench.py --workload gpt2 --graph, 3 steps", flush=True)
    d = _bench("--workload", "gpt2", "--graph", "--steps", "3", "--warmup", "1", "--no-cpu-baseline")
    assert d["unit"] == "TFLOP/s" and d["value"] > 0
    assert d["graph_ms_per_step"] > 0 and d["graph_tflops"] > 0
    _roofline_consistent(d)
    print(f"[ok] eager {d['ms_per_step']} ms, graph {d['graph_ms_per_step']} ms", flush=True)
