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


def test_cpu_baseline_is_bounded_and_labelled():
    """The host baseline times the oracle on a bounded sample (whole paths,
    one query head), reports the cores it may use and the BLAS library, and
    says that it is scaled."""
    sys.path.insert(0, ROOT)
    import bench
    from tree_inputs import config_spec, config_tree, make_inputs, tree_stats
    # the long trunk: whole paths within about 1e12 fp64 FLOP of one head
    t5 = config_tree(5)
    paths = bench._sample_paths(t5, 128)
    work = sum(12.0 * 128 * len(p) * (len(p) + 1) / 2 for p in paths)
    assert len(paths) >= 1 and work <= 1.0e12
    # a small tree: all of its paths fit; the sample's scale factor is the
    # query-head count times the dense work over the sampled paths' work
    t = config_tree(1)
    sp = config_spec(1)
    x = make_inputs(t.num_tokens, 1, 1, 64, dtype="fp32", do_std=1.0)
    rec = bench.cpu_baseline(t, sp, bench._baseline_sample(t, x, 64))
    assert rec["kind"] == "oracle" and rec["scaled"] is True and rec["value"] > 0
    assert rec["cores"] == len(os.sched_getaffinity(0))
    assert rec["blas"] != "none found"
    assert abs(rec["scale_factor"] - 1.0) < 1e-12  # every path, the only head
    assert tree_stats(t)["dense_pairs"] == 25920
