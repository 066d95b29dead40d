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


def test_traffic_figure_is_tied_to_the_kernel_and_its_headers(tmp_path):
    # the committed counter summary counts only while the scoring kernel's
    # source and the headers it includes are unchanged
    sys.path.insert(0, ROOT)
    import bench
    (tmp_path / "k.hip").write_text('#include "a.hpp"\n#include <stdint.h>\nint k;\n')
    (tmp_path / "a.hpp").write_text('#include "b.hpp"\n')
    (tmp_path / "b.hpp").write_text("int b;\n")
    (tmp_path / "unused.hpp").write_text("int u;\n")
    src = str(tmp_path / "k.hip")
    d0 = bench.source_digest(src)
    summary = tmp_path / "s.md"
    summary.write_text(f"text\n\n- source_digest: `{d0}`\n- traffic_bytes_per_launch: 1234\n")
    assert bench.measured_traffic(str(summary), src) == 1234
    (tmp_path / "unused.hpp").write_text("int v;\n")
    assert bench.source_digest(src) == d0
    (tmp_path / "b.hpp").write_text("int c;\n")  # a header two includes deep
    assert bench.source_digest(src) != d0
    assert bench.measured_traffic(str(summary), src) is None
