"""Pins for the oracle of the depth-first schedule (query-subset calls).

AReaL-DTA (abstract) walks the prefix tree depth first, one root-to-leaf path
resident at a time, and still computes each shared prefix once.  One call of
that walk takes the queries of some nodes; ``oracle.tree_attention_subset``
gives its outputs and its gradients, those of the loss summed over its query
rows only.  Pinned here against:
* a brute-force dense softmax over all unique tokens (mask from the
  transitive closure of the parent relation) whose autograd loss sums over
  the query rows only -- a different algorithm and a direct statement of the
  restricted loss;
* the whole-tree oracle: over the nodes of a depth-first walk, one node per
  call, the forward rows and dQ rows are the whole-tree ones and the K/V
  gradients sum to the whole-tree ones (the unique-token loss is the sum of
  the per-node losses);
* special cases: no query node gives zero K/V gradients; every node at once
  is the whole tree.
"""

import numpy as np
import pytest
import torch

import oracle
from tree_inputs import binary_tree, dfs_preorder, random_tree, star_tree
from test_oracle import _rand_qkvdo, _rel, visibility_mask


def _brute_force_rows(t, q, k, v, do, scale, rows):
    """Dense masked attention over all unique tokens, torch fp64 autograd,
    loss = sum over the rows in ``rows`` of <dO_t, O_t>."""
    mask_t = torch.from_numpy(visibility_mask(t))
    hq, hkv = q.shape[1], k.shape[1]
    gs = hq // hkv
    Q = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    K = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    V = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    dO = torch.tensor(do, dtype=torch.float64)
    outs, lses = [], []
    for h in range(hq):
        g = h // gs
        s = (scale * (Q[:, h] @ K[:, g].T)).masked_fill(~mask_t, float("-inf"))
        lses.append(torch.logsumexp(s, dim=1))
        outs.append(torch.softmax(s, dim=1) @ V[:, g])
    O = torch.stack(outs, dim=1)
    sel = torch.from_numpy(np.flatnonzero(rows))
    (O[sel] * dO[sel]).sum().backward()
    return {"o": O.detach().numpy(), "lse": torch.stack(lses).detach().numpy(),
            "dq": Q.grad.numpy(), "dk": K.grad.numpy(), "dv": V.grad.numpy()}


def _row_mask(t, nodes):
    rows = np.zeros(t.num_tokens, bool)
    for i in nodes:
        rows[t.seg_start[i]:t.seg_start[i] + t.seg_len[i]] = True
    return rows


@pytest.mark.parametrize("seed,nodes,roots,hq,hkv,d", [
    (0, 6, 1, 2, 1, 8), (1, 11, 2, 4, 2, 8), (2, 15, 1, 3, 3, 4), (3, 9, 3, 6, 2, 8),
])
def test_subset_equals_bruteforce_restricted_loss(seed, nodes, roots, hq, hkv, d):
    rng = np.random.default_rng(100 + seed)
    t = random_tree(rng, nodes, max_len=10, n_roots=roots)
    q, k, v, do = _rand_qkvdo(rng, t.num_tokens, hq, hkv, d)
    scale = 1.0 / np.sqrt(d)
    for trial in range(3):
        qn = rng.choice(t.num_nodes, size=int(rng.integers(1, t.num_nodes + 1)), replace=False)
        rows = _row_mask(t, qn)
        r = oracle.tree_attention_subset(q, k, v, do, t.parent, t.seg_start, t.seg_len, scale, qn)
        b = _brute_force_rows(t, q, k, v, do, scale, rows)
        assert np.array_equal(r["rows"], rows)
        assert _rel(r["o"][rows], b["o"][rows]) < 1e-12
        assert _rel(r["lse"][:, rows], b["lse"][:, rows]) < 1e-12
        assert _rel(r["dq"][rows], b["dq"][rows]) < 1e-12
        for key in ("dk", "dv"):
            assert _rel(r[key], b[key]) < 1e-12, (key, trial)
        # rows outside the subset are not computed by one call
        assert np.isnan(r["o"][~rows]).all() and np.isnan(r["dq"][~rows]).all()


def test_depth_first_walk_sums_to_whole_tree():
    rng = np.random.default_rng(5)
    for t in (binary_tree(7, 5, 3), star_tree(9, 4, 6), random_tree(rng, 12, max_len=9,
                                                                     n_roots=2)):
        q, k, v, do = _rand_qkvdo(rng, t.num_tokens, 4, 2, 8)
        scale = 0.3
        full = oracle.tree_attention(q, k, v, do, t.parent, t.seg_start, t.seg_len, scale)
        dk = np.zeros_like(full["dk"])
        dv = np.zeros_like(full["dv"])
        seen = np.zeros(t.num_tokens, bool)
        order = dfs_preorder(t.parent)
        assert sorted(order) == list(range(t.num_nodes))
        for node in reversed(order):
            r = oracle.tree_attention_subset(q, k, v, do, t.parent, t.seg_start, t.seg_len,
                                             scale, [node])
            rows = r["rows"]
            assert not (seen & rows).any()
            seen |= rows
            assert _rel(r["o"][rows], full["o"][rows]) < 1e-13
            assert _rel(r["lse"][:, rows], full["lse"][:, rows]) < 1e-13
            assert _rel(r["dq"][rows], full["dq"][rows]) < 1e-12
            dk += r["dk"]
            dv += r["dv"]
        assert seen.all()
        assert _rel(dk, full["dk"]) < 1e-12 and _rel(dv, full["dv"]) < 1e-12


def test_dfs_preorder_visits_parents_first():
    rng = np.random.default_rng(9)
    t = random_tree(rng, 30, max_len=3, n_roots=3)
    order = dfs_preorder(t.parent)
    at = {n: i for i, n in enumerate(order)}
    for i, p in enumerate(t.parent):
        if p >= 0:
            assert at[p] < at[i]
    # depth first: each node's subtree is one contiguous run of the order
    for i in range(t.num_nodes):
        sub = {i}
        for j in order[at[i] + 1:]:
            if t.parent[j] in sub:
                sub.add(j)
            else:
                break
        desc = {j for j in range(t.num_nodes) if _is_desc(t.parent, j, i)}
        assert sub == desc | {i}


def _is_desc(parent, j, i):
    a = int(parent[j])
    while a >= 0:
        if a == i:
            return True
        a = int(parent[a])
    return False


def test_special_subsets():
    rng = np.random.default_rng(3)
    t = random_tree(rng, 8, max_len=7)
    q, k, v, do = _rand_qkvdo(rng, t.num_tokens, 2, 1, 4)
    full = oracle.tree_attention(q, k, v, do, t.parent, t.seg_start, t.seg_len, 0.5)
    none = oracle.tree_attention_subset(q, k, v, do, t.parent, t.seg_start, t.seg_len, 0.5, [])
    assert not none["rows"].any()
    assert np.all(none["dk"] == 0) and np.all(none["dv"] == 0)
    every = oracle.tree_attention_subset(q, k, v, do, t.parent, t.seg_start, t.seg_len, 0.5,
                                         range(t.num_nodes))
    for key in ("o", "lse", "dq", "dk", "dv"):
        assert _rel(every[key], full[key]) == 0.0, key
    # a leaf alone: its K/V gradients differ from the whole tree's (a dropped
    # restriction of the loss would make them equal)
    leaf = [i for i in range(t.num_nodes) if i not in set(t.parent.tolist())][0]
    one = oracle.tree_attention_subset(q, k, v, do, t.parent, t.seg_start, t.seg_len, 0.5,
                                       [leaf])
    assert _rel(one["dk"], full["dk"]) > 1e-3
