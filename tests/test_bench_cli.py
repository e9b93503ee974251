"""bench.py's command-line contract, checked on the host (no GPU touched)."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_exits_with_a_message(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert r.stdout == ""
    assert "one GPU only" in r.stderr and f"--gpus {n}" in r.stderr


def test_defaults_are_one_gpu_and_a_short_run(monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    a = bench.parse()
    assert (a.gpus, a.steps, a.warmup, a.workload, a.weights) == (1, 20, 5, "16b", "packed")
    assert 0 < bench.WARMUP_MIN_S <= 1.0
