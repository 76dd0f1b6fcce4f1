"""Host-side tests of tree_attn_build_tree (C++ prefix compression, no GPU):
exact agreement with the oracle on every output, the inverse map, edge cases
and argument errors."""

import ctypes

import numpy as np
import pytest

import prefix_shared_tree_attn_amd as ta
from prefix_shared_tree_attn_amd import _ffi
from oracle import prefix_tree as opt
import oracle
from tree_inputs import config_tree


def _random_trajectories(seed, n_traj=20, vocab=5, max_len=30):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n_traj):
        if out and rng.random() < 0.6:
            base = out[int(rng.integers(len(out)))]
            cut = int(rng.integers(0, len(base) + 1))
            out.append(base[:cut] + rng.integers(0, vocab, int(rng.integers(0, max_len))).tolist())
        else:
            out.append(rng.integers(0, vocab, int(rng.integers(0, max_len + 1))).tolist())
    return out


def _compare(trajs):
    got = ta.build_tree(trajs)
    ref = opt.build_tree(trajs)
    for k in ("parent", "seg_start", "seg_len", "unique_tokens", "traj_index", "mult"):
        np.testing.assert_array_equal(getattr(got, k), ref[k], err_msg=k)
    # inverse map: positions of each unique row, ascending, consistent with
    # the forward map
    n = got.num_tokens
    assert got.inv_offsets[0] == 0 and got.inv_offsets[n] == len(got.traj_index)
    for u in range(n):
        pos = got.inv_positions[got.inv_offsets[u]:got.inv_offsets[u + 1]]
        assert np.all(np.diff(pos) > 0)
        assert np.all(got.traj_index[pos] == u)
    return got


@pytest.mark.parametrize("seed", range(10))
def test_matches_oracle_random(seed):
    _compare(_random_trajectories(seed))


@pytest.mark.parametrize("trajs", [
    [], [[]], [[], []], [[5]], [[1, 2, 3], [1, 2, 3]], [[1, 2, 3], [1, 2]],
    [[1], [2], [3]], [[0] * 50, [0] * 20 + [1]],
])
def test_matches_oracle_edge_cases(trajs):
    _compare(trajs)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_workload_paths_give_a_valid_plan(cfg):
    """The trajectories of a workload tree (token id = unique row) compress
    to a node table that the planner accepts, with the same pair count; nodes
    with a single child are merged into it."""
    t = config_tree(cfg)
    paths = oracle.root_to_leaf_paths(t.parent, t.seg_start, t.seg_len)
    got = _compare([p.tolist() for p in paths]) if cfg <= 2 else ta.build_tree([p.tolist() for p in paths])
    # radix compression merges every node that has exactly one child into it
    kids = np.bincount(t.parent[t.parent >= 0], minlength=t.num_nodes)
    assert got.num_tokens == t.num_tokens
    assert got.num_nodes == t.num_nodes - int((kids == 1).sum())
    p = ta.plan_host(got.parent, got.seg_start, got.seg_len, got.num_tokens, 8, 8, 128)
    from tree_inputs import tree_stats
    assert p.stats()["pairs"] == tree_stats(t)["pairs"]


def test_argument_errors():
    lib = _ffi.lib()
    one = (ctypes.c_int32 * 4)(0, 0, 0, 0)
    m, n = ctypes.c_int32(0), ctypes.c_int32(0)
    bad = (ctypes.c_int64 * 2)(1, 3)  # offsets must start at 0
    st = lib.tree_attn_build_tree(one, bad, 1, one, one, one, one, one, None, None, None,
                                  ctypes.byref(m), ctypes.byref(n))
    assert _ffi.STATUS[st] == "INVALID_ARG"
    dec = (ctypes.c_int64 * 3)(0, 2, 1)  # decreasing
    st = lib.tree_attn_build_tree(one, dec, 2, one, one, one, one, one, None, None, None,
                                  ctypes.byref(m), ctypes.byref(n))
    assert _ffi.STATUS[st] == "INVALID_ARG"
    neg = (ctypes.c_int32 * 2)(1, -4)
    ok = (ctypes.c_int64 * 2)(0, 2)
    st = lib.tree_attn_build_tree(neg, ok, 1, one, one, one, one, one, None, None, None,
                                  ctypes.byref(m), ctypes.byref(n))
    assert _ffi.STATUS[st] == "INVALID_ARG"
    with pytest.raises(ta.TreeAttnError):
        ta.build_tree([[3, -1]])


def test_device_ops_reject_bad_arguments_without_a_gpu():
    lib = _ffi.lib()
    assert _ffi.STATUS[lib.tree_attn_gather_rows(None, None, None, -1, 4, None)] == "INVALID_ARG"
    assert _ffi.STATUS[lib.tree_attn_gather_rows(None, None, None, 0, 4, None)] == "OK"
    assert _ffi.STATUS[lib.tree_attn_scatter_sum_rows(None, None, None, None, 3, 4, 9, None)] == "UNSUPPORTED"
    assert _ffi.STATUS[lib.tree_attn_rope(None, None, 4, 2, 7, ctypes.c_float(1e4), 0, 0, None)] == "UNSUPPORTED"
    assert _ffi.STATUS[lib.tree_attn_rope(None, None, 4, 2, 8, ctypes.c_float(0.5), 0, 0, None)] == "INVALID_ARG"
    assert _ffi.STATUS[lib.tree_attn_rope(None, None, 4, 2, 8, ctypes.c_float(1e4), 0, 0, None)] == "INVALID_ARG"
