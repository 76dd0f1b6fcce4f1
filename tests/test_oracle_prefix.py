"""Pins for the prefix-tree oracle (oracle/prefix_tree.py), independent of it.

* prefix compression against brute force: the unique rows are exactly the
  distinct prefixes of the trajectories, and a row's multiplicity is the
  number of trajectories that start with its prefix;
* round trip: the unique tokens indexed by the trajectory map give back
  every trajectory;
* radix compression: siblings start with different tokens and every inner
  node has at least two children;
* a workload tree is recovered from its own root-to-leaf paths;
* gather / scatter-sum: the adjoint identity and the multiplicity count;
* rotary embedding: the complex-number form of the rotation, norm
  preservation, inverse, position 0, and the relative-position property.
"""

import numpy as np
import pytest

import oracle
from oracle import prefix_tree as opt
from tree_inputs import config_tree


def _random_trajectories(seed, n_traj=12, vocab=4, max_len=9):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n_traj):
        if out and rng.random() < 0.5:  # share a prefix with an earlier one
            base = out[int(rng.integers(len(out)))]
            cut = int(rng.integers(0, len(base) + 1))
            tail = rng.integers(0, vocab, int(rng.integers(0, max_len))).tolist()
            out.append(base[:cut] + tail)
        else:
            out.append(rng.integers(0, vocab, int(rng.integers(0, max_len + 1))).tolist())
    return out


def _row_prefixes(r):
    """Prefix (tuple of token ids) of every unique row, from the node table."""
    n = r["unique_tokens"].shape[0]
    node_of = np.empty(n, np.int64)
    for i, (s, l) in enumerate(zip(r["seg_start"], r["seg_len"])):
        node_of[s:s + l] = i
    pref = []
    for row in range(n):
        node = node_of[row]
        toks = list(r["unique_tokens"][r["seg_start"][node]:row + 1])
        p = r["parent"][node]
        while p >= 0:
            toks = list(r["unique_tokens"][r["seg_start"][p]:r["seg_start"][p] + r["seg_len"][p]]) + toks
            p = r["parent"][p]
        pref.append(tuple(int(t) for t in toks))
    return pref


@pytest.mark.parametrize("seed", range(8))
def test_unique_rows_are_the_distinct_prefixes(seed):
    trajs = _random_trajectories(seed)
    r = opt.build_tree(trajs)
    brute = {}
    for t in trajs:
        for k in range(1, len(t) + 1):
            brute[tuple(t[:k])] = brute.get(tuple(t[:k]), 0) + 1
    pref = _row_prefixes(r)
    assert sorted(pref) == sorted(brute)
    assert [brute[p] for p in pref] == r["mult"].tolist()


@pytest.mark.parametrize("seed", range(8))
def test_round_trip_and_radix_shape(seed):
    trajs = _random_trajectories(seed + 50)
    r = opt.build_tree(trajs)
    flat = [tok for t in trajs for tok in t]
    assert r["unique_tokens"][r["traj_index"]].tolist() == flat
    # every position maps to the row of its own prefix
    pref = _row_prefixes(r)
    i = 0
    for t in trajs:
        for k in range(1, len(t) + 1):
            assert pref[r["traj_index"][i]] == tuple(t[:k])
            i += 1
    # segments partition [0, N); siblings differ in their first token; inner
    # nodes branch
    m = r["parent"].shape[0]
    order = np.argsort(r["seg_start"])
    pos = 0
    for j in order:
        assert r["seg_start"][j] == pos and r["seg_len"][j] >= 1
        pos += r["seg_len"][j]
    assert pos == r["unique_tokens"].shape[0]
    kids = {}
    for j in range(m):
        kids.setdefault(int(r["parent"][j]), []).append(j)
    for p, ch in kids.items():
        firsts = [int(r["unique_tokens"][r["seg_start"][c]]) for c in ch]
        assert len(set(firsts)) == len(firsts)
        if p >= 0:
            assert len(ch) >= 2


def test_edge_cases():
    r = opt.build_tree([])
    assert r["parent"].shape == (0,) and r["unique_tokens"].shape == (0,)
    r = opt.build_tree([[], [7], [], [7]])
    assert r["parent"].tolist() == [-1] and r["mult"].tolist() == [2]
    r = opt.build_tree([[1, 2, 3], [1, 2]])  # a prefix of another adds nothing
    assert r["seg_len"].tolist() == [3] and r["traj_index"].tolist() == [0, 1, 2, 0, 1]


@pytest.mark.parametrize("cfg", [1, 2, 4])
def test_workload_tree_recovered_from_its_paths(cfg):
    """Token id = unique row: the trie of a tree's root-to-leaf paths is the
    tree again (same node count, depth offsets and segment lengths)."""
    t = config_tree(cfg)
    paths = oracle.root_to_leaf_paths(t.parent, t.seg_start, t.seg_len)
    r = opt.build_tree([p.tolist() for p in paths])
    assert r["parent"].shape[0] == t.num_nodes
    assert r["unique_tokens"].shape[0] == t.num_tokens
    assert sorted(r["unique_tokens"].tolist()) == list(range(t.num_tokens))
    _, pos = oracle.token_positions(t.parent, t.seg_start, t.seg_len, t.num_tokens)
    _, pos_r = oracle.token_positions(r["parent"], r["seg_start"], r["seg_len"], t.num_tokens)
    # the unique row holding original token u sits at the same depth
    np.testing.assert_array_equal(pos_r[np.argsort(r["unique_tokens"])], pos)


def test_gather_scatter_adjoint():
    rng = np.random.default_rng(3)
    idx = rng.integers(0, 9, 40)
    x = rng.standard_normal((9, 5))
    y = rng.standard_normal((40, 5))
    lhs = float((opt.gather_rows(x, idx) * y).sum())
    rhs = float((x * opt.scatter_sum_rows(y, idx, 9)).sum())
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))
    ones = opt.scatter_sum_rows(np.ones((40, 1)), idx, 9)[:, 0]
    np.testing.assert_array_equal(ones, np.bincount(idx, minlength=9))


def test_rope_complex_form_and_invariants():
    rng = np.random.default_rng(4)
    n, h, d = 7, 3, 16
    x = rng.standard_normal((n, h, d))
    pos = rng.integers(0, 50000, n)
    y = opt.rope(x, pos, theta=10000.0)
    # complex form: z = a + i b multiplied by exp(i pos theta^(-2j/d))
    half = d // 2
    z = x[..., :half] + 1j * x[..., half:]
    w = np.exp(1j * pos[:, None, None] * (10000.0 ** (-np.arange(half) * 2.0 / d))[None, None, :])
    zz = z * w
    np.testing.assert_allclose(y, np.concatenate([zz.real, zz.imag], -1), atol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-12)
    np.testing.assert_allclose(opt.rope(y, pos, inverse=True), x, atol=1e-10)
    np.testing.assert_array_equal(opt.rope(x, np.zeros(n, np.int64)), x)
    # scores depend on the position difference only
    q = rng.standard_normal((1, 1, d))
    k = rng.standard_normal((1, 1, d))
    s1 = float((opt.rope(q, [100]) * opt.rope(k, [37])).sum())
    s2 = float((opt.rope(q, [1163]) * opt.rope(k, [1100])).sum())
    assert abs(s1 - s2) <= 1e-9


def test_rope_at_depth_equals_rope_on_every_path():
    """Rotating a unique token at its depth equals rotating each trajectory
    copy at its index in the trajectory."""
    t = config_tree(1)
    rng = np.random.default_rng(5)
    x = rng.standard_normal((t.num_tokens, 2, 8))
    _, pos = oracle.token_positions(t.parent, t.seg_start, t.seg_len, t.num_tokens)
    y = opt.rope(x, pos)
    for p in oracle.root_to_leaf_paths(t.parent, t.seg_start, t.seg_len):
        np.testing.assert_allclose(opt.rope(x[p], np.arange(p.shape[0])), y[p], atol=1e-12)
