"""Host checks of the linear-attention piece table (no GPU).

The table must cut every node exactly where the trajectory depth of its
tokens is a multiple of the chunk, cover every token once, and link each
piece to the piece whose end state it starts from (predecessor) and to the
pieces that start from its end state (successors).  Depths are computed here
from the node table, independently of the library.
"""

import numpy as np
import pytest

import prefix_shared_tree_attn_amd as ta
from tree_inputs import binary_tree, chain_tree, config_tree, random_tree, star_tree


def _depths(t):
    m = t.num_nodes
    depth = np.zeros(m, np.int64)
    for i in range(m):
        a, d = int(t.parent[i]), 0
        while a >= 0:
            d += int(t.seg_len[a])
            a = int(t.parent[a])
        depth[i] = d
    return depth


def _check(t):
    p = ta.plan_host(t.parent, t.seg_start, t.seg_len, t.num_tokens, 2, 1, 64, "bf16")
    st = p.stats()
    e = p.lin_export()
    pcs, succ = e["pieces"], e["succ"]
    chunk = st["lin_chunk"]
    assert chunk == 64
    depth = _depths(t)
    covered = np.zeros(t.num_tokens, np.int64)
    first, last = {}, {}
    for j, (t0, ln, pred, sb, se, node, _, _) in enumerate(pcs):
        s, l = int(t.seg_start[node]), int(t.seg_len[node])
        assert 1 <= ln <= chunk and s <= t0 and t0 + ln <= s + l
        covered[t0:t0 + ln] += 1
        d0 = depth[node] + (t0 - s)  # trajectory depth of the first token
        # starts at a chunk boundary or at the node's start; never crosses one
        assert d0 % chunk == 0 or t0 == s
        assert (d0 % chunk) + ln <= chunk
        assert pred < j
        first.setdefault(int(node), j)
        last[int(node)] = j
    for j, pc in enumerate(pcs):
        node = int(pc[5])
        assert pc[6] == (1 if first[node] == j else 0) | (2 if last[node] == j else 0)
    assert np.all(covered == 1)
    for j, (t0, ln, pred, sb, se, node, _, _) in enumerate(pcs):
        node = int(node)
        if t0 == t.seg_start[node]:
            par = int(t.parent[node])
            assert pred == (last[par] if par >= 0 else -1)
        else:
            assert pred == j - 1 and pcs[j - 1][0] + pcs[j - 1][1] == t0
        want = sorted(c for c in range(len(pcs)) if pcs[c][2] == j)
        assert sorted(succ[sb:se].tolist()) == want
        assert all(c > j for c in want)
    return len(pcs)


@pytest.mark.parametrize("name", ["chain", "star", "binary", "random", "forest", "agent"])
def test_piece_table(name):
    rng = np.random.default_rng(3)
    t = {"chain": chain_tree([70, 1, 129, 64, 200]), "star": star_tree(100, 5, 70),
         "binary": binary_tree(32, 16, 3), "random": random_tree(rng, 30, max_len=150),
         "forest": random_tree(rng, 20, max_len=90, n_roots=4), "agent": config_tree(3)}[name]
    n = _check(t)
    assert n >= (t.num_tokens + 63) // 64


def test_workspace_sizes():
    t = star_tree(100, 3, 70)
    p = ta.plan_host(t.parent, t.seg_start, t.seg_len, t.num_tokens, 4, 2, 128, "bf16")
    f, b = p.lin_workspace_size()
    blk = p.stats()["lin_pieces"] * 2 * 128 * 128 * 2  # bf16 piece states
    ends = t.num_nodes * 2 * 128 * 128 * 4              # fp32 node states
    assert f >= 2 * blk + ends and b >= 3 * blk + ends and f % 256 == 0 and b % 256 == 0


def _scan_trees():
    rng = np.random.default_rng(5)
    return {"chain": chain_tree([70, 1, 129, 64, 200]), "star": star_tree(100, 5, 70),
            "binary": binary_tree(32, 16, 4), "random": random_tree(rng, 40, max_len=150),
            "forest": random_tree(rng, 25, max_len=90, n_roots=4), "agent": config_tree(3),
            "long-trunk": config_tree(5)}


TREES = _scan_trees()


@pytest.mark.parametrize("name", list(TREES))
def test_scan_chains(name):
    """The state scans walk heavy paths: every node in exactly one chain,
    each chain a run of parent -> child steps that always takes the child
    with the most pieces below it, a chain's head a root (phase 0) or a
    light child of a node on a chain of the previous phase, and the phases
    listed in order -- so a forward phase finds every head's parent done and
    a backward phase every node's light children done.  A root-to-leaf path
    crosses at most log2(pieces) + 1 phases."""
    t = TREES[name]
    p = ta.plan_host(t.parent, t.seg_start, t.seg_len, t.num_tokens, 4, 2, 64, "bf16")
    ex = p.lin_export()
    st = p.stats()
    pieces, chains, cn, phases = ex["pieces"], ex["chains"], ex["chain_nodes"], ex["phases"]
    m = t.num_nodes
    assert st["lin_nodes"] == m and sorted(cn.tolist()) == list(range(m))
    # the root-first node order of the scans: node index of each position
    first_piece = {}
    for j, pc in enumerate(pieces):
        first_piece.setdefault(int(pc[5]), j)
    order = sorted(first_piece, key=lambda n: first_piece[n])
    node_at = {k: n for k, n in enumerate(order)}
    count = np.bincount(pieces[:, 5], minlength=m)
    below = count.astype(np.int64).copy()
    for n in reversed(order):
        if t.parent[n] >= 0:
            below[t.parent[n]] += below[n]
    kids = [[] for _ in range(m)]
    for n in range(m):
        if t.parent[n] >= 0:
            kids[t.parent[n]].append(n)
    phase_of = {}
    for ci, (b, e, ph, _) in enumerate(chains):
        nodes = [node_at[int(k)] for k in cn[b:e]]
        for n in nodes:
            phase_of[n] = int(ph)
        head = nodes[0]
        if t.parent[head] < 0:
            assert ph == 0
        else:
            assert phase_of[int(t.parent[head])] == ph - 1
            assert max(below[c] for c in kids[t.parent[head]]) >= below[head]
        for a_, b_ in zip(nodes, nodes[1:]):
            assert t.parent[b_] == a_ and below[b_] == max(below[c] for c in kids[a_])
        assert kids[nodes[-1]] == [] or all(phase_of.get(c, ph + 1) == ph + 1 for c in kids[nodes[-1]])
    assert phases[0][0] == 0 and phases[-1][1] == len(chains)
    for k, (cb, ce, _, _) in enumerate(phases):
        assert (chains[cb:ce, 2] == k).all()
        if k + 1 < len(phases):
            assert phases[k + 1][0] == ce
    assert len(phases) <= int(np.log2(max(2, len(pieces)))) + 1
