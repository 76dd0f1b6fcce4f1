"""The benchmark's command line, checked without a GPU: more than one GPU is
refused with a message (this path measures one GPU), before any device work."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "exactly one GPU" in res.stderr
    assert res.stdout == ""  # no metric line


def test_unknown_workload_is_rejected():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "nope"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode != 0 and "invalid choice" in res.stderr
