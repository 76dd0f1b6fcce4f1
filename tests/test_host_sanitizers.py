"""The host side of the library under AddressSanitizer and
UndefinedBehaviorSanitizer: node-table validation, the planner, the
prefix-tree builder and the C ABI's argument checks, exercised by the host
test files (planner, prefix compression, linear-attention plans) against a
build of the host sources with both sanitizers (prefix_shared_tree_attn_amd/
build.py, build_host_sanitized).  Any report fails the run.  No GPU code is
instrumented and no GPU is used."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_paths_are_clean_under_sanitizers():
    if shutil.which("g++") is None:
        pytest.skip("no host C++ compiler")
    from prefix_shared_tree_attn_amd import build as libbuild
    lib = libbuild.build_host_sanitized()
    asan = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    assert os.path.isabs(asan), "compiler has no AddressSanitizer runtime"
    env = dict(os.environ)
    env.update(TREE_ATTN_LIBRARY=lib, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    files = [os.path.join(ROOT, "tests", f)
             for f in ("test_planner.py", "test_prefix_host.py", "test_linear_host.py")]
    # -s: a sanitizer report goes to the process's stderr, which the inner
    # run must not capture
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p",
                          "no:cacheprovider", *files], cwd=ROOT, env=env, capture_output=True,
                         text=True, timeout=900)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " passed" in out
