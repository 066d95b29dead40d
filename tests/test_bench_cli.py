"""The benchmark's command line (CPU only: nothing here touches a GPU)."""
from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in r.stdout + r.stderr


def test_help_lists_the_workload_switches():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0
    for flag in ("--steps", "--warmup", "--gpus", "--no-cpu-baseline", "--no-prefill", "--no-workloads", "--counters"):
        assert flag in r.stdout
