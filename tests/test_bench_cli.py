"""bench.py's command line on the CPU: it measures one GPU and says so when
asked for more, before touching the GPU."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60, cwd=ROOT)
    assert r.returncode == 2
    assert r.stdout == ""
    assert "one GPU" in r.stderr and "--gpus 1" in r.stderr


def test_help_lists_the_measurement_options():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"],
                       capture_output=True, text=True, timeout=60, cwd=ROOT)
    assert r.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup", "--workload", "--graph", "--sweep", "--io-ablation",
                 "--compare-standard", "--calibrate-copy", "--no-cpu-baseline"):
        assert flag in r.stdout, flag
