"""Rollout prefix trees as node tables.

A tree (or a forest) is three int32 arrays of length M (number of nodes):

* ``parent[i]``    index of node i's parent, -1 for a root;
* ``seg_start[i]`` first packed row of node i's token segment;
* ``seg_len[i]``   number of tokens in node i's segment (>= 1).

The segments partition the packed rows ``[0, N)``.  Token ``t`` in node ``i``
at offset ``o`` has as its context every token of every proper ancestor of
``i`` plus tokens ``seg_start[i] .. seg_start[i]+o`` of its own node: that is
the root-to-leaf prefix structure the pages describe (AReaL-DTA, abstract:
prefix sharing induces a tree over rollouts; HARTS, abstract: irregular
rollout trees with shared histories).

Packing order is depth-first preorder with children in creation order unless
a builder says otherwise.  Nothing here computes attention.
"""

from __future__ import annotations

import dataclasses
from typing import List, Tuple

import numpy as np


@dataclasses.dataclass
class NodeTable:
    parent: np.ndarray     # int32 [M]
    seg_start: np.ndarray  # int32 [M]
    seg_len: np.ndarray    # int32 [M]
    num_tokens: int
    name: str = ""

    @property
    def num_nodes(self) -> int:
        return int(self.parent.shape[0])

    def copy(self) -> "NodeTable":
        return NodeTable(self.parent.copy(), self.seg_start.copy(),
                         self.seg_len.copy(), self.num_tokens, self.name)


def _from_lists(parents: List[int], lens: List[int], name: str,
                order: List[int] | None = None) -> NodeTable:
    """Pack nodes contiguously in ``order`` (default: node id order)."""
    m = len(parents)
    order = list(range(m)) if order is None else order
    seg_start = np.zeros(m, np.int64)
    pos = 0
    for i in order:
        seg_start[i] = pos
        pos += lens[i]
    return NodeTable(np.asarray(parents, np.int32), seg_start.astype(np.int32),
                     np.asarray(lens, np.int32), int(pos), name)


def chain_tree(lengths: List[int], name: str = "chain") -> NodeTable:
    """A single path split into consecutive nodes (one trajectory)."""
    parents = [-1] + list(range(len(lengths) - 1))
    return _from_lists(parents, list(lengths), name)


def star_tree(prompt: int, n_children: int, child_len: int,
              name: str = "star") -> NodeTable:
    """One prompt node with ``n_children`` response nodes (a GRPO group)."""
    parents = [-1] + [0] * n_children
    lens = [prompt] + [child_len] * n_children
    return _from_lists(parents, lens, name)


def binary_tree(root_len: int, seg_len: int, levels: int,
                name: str = "binary") -> NodeTable:
    """Full binary tree: a root of ``root_len`` tokens and ``levels`` levels of
    children of ``seg_len`` tokens each; packed in DFS preorder."""
    parents: List[int] = []
    lens: List[int] = []

    def rec(par: int, depth: int) -> None:
        me = len(parents)
        parents.append(par)
        lens.append(root_len if depth == 0 else seg_len)
        if depth < levels:
            rec(me, depth + 1)
            rec(me, depth + 1)

    rec(-1, 0)
    return _from_lists(parents, lens, name)


def agent_tree(seed: int = 0, levels: int = 8, branch: Tuple[int, int] = (1, 3),
               seg: Tuple[int, int] = (128, 1024), target: int = 32768,
               tol: int = 2048, max_path: int = 16384,
               name: str = "agent") -> NodeTable:
    """Irregular multi-turn agent tree.

    The root is level 1; every node above the last level gets U{branch}
    children, every segment length is U[seg].  Nodes are drawn depth-first
    from one PCG64 stream; whole trees are redrawn from the same stream until
    the unique-token count lies in ``[target - tol, target + tol]`` and the
    longest path is at most ``max_path``.
    """
    rng = np.random.default_rng(seed)
    while True:
        parents: List[int] = []
        lens: List[int] = []

        def rec(par: int, level: int) -> None:
            me = len(parents)
            parents.append(par)
            lens.append(int(rng.integers(seg[0], seg[1] + 1)))
            if level < levels:
                nch = int(rng.integers(branch[0], branch[1] + 1))
                for _ in range(nch):
                    rec(me, level + 1)

        rec(-1, 1)
        n = sum(lens)
        if target - tol <= n <= target + tol:
            t = _from_lists(parents, lens, name)
            if tree_stats(t)["max_path"] <= max_path:
                return t


def trunk_tree(seed: int = 0, trunk: int = 32768, n_branches: int = 64,
               branch_len: int = 2048, name: str = "trunk") -> NodeTable:
    """Long trunk chain with leaf branches attached at random trunk positions.

    Branch b attaches after trunk token p_b - 1 (it sees trunk[0:p_b]), with
    p_b ~ U{1..trunk} drawn from PCG64(seed).  The trunk is cut into chain
    nodes at every distinct p_b < trunk; branches with equal p_b are siblings.
    The trunk is packed first (contiguous, in order), then the branches in
    ascending p_b (ties in draw order).  The trunk's last chain node is a
    leaf unless some p_b == trunk.
    """
    rng = np.random.default_rng(seed)
    p = rng.integers(1, trunk + 1, size=n_branches)
    cuts = sorted(set(int(x) for x in p if x < trunk))
    bounds = [0] + cuts + [trunk]
    parents: List[int] = []
    lens: List[int] = []
    end_to_node = {}
    for i in range(len(bounds) - 1):
        parents.append(i - 1)
        lens.append(bounds[i + 1] - bounds[i])
        end_to_node[bounds[i + 1]] = i
    for b in sorted(range(n_branches), key=lambda b: (int(p[b]), b)):
        parents.append(end_to_node[int(p[b])])
        lens.append(branch_len)
    return _from_lists(parents, lens, name)


def random_tree(rng: np.random.Generator, n_nodes: int, max_len: int = 40,
                min_len: int = 1, n_roots: int = 1, shuffle: bool = True,
                name: str = "random") -> NodeTable:
    """Random small forest for tests: random parents, random segment lengths,
    and (optionally) random node ids and a random packing order."""
    n_roots = max(1, min(n_roots, n_nodes))
    parents = [-1] * n_roots
    for i in range(n_roots, n_nodes):
        parents.append(int(rng.integers(0, i)))
    lens = [int(rng.integers(min_len, max_len + 1)) for _ in range(n_nodes)]
    if not shuffle:
        return _from_lists(parents, lens, name)
    # relabel nodes with a random permutation and pack in another random order
    perm = rng.permutation(n_nodes)          # old id -> new id
    new_par = [0] * n_nodes
    new_len = [0] * n_nodes
    for old in range(n_nodes):
        new = int(perm[old])
        new_par[new] = -1 if parents[old] < 0 else int(perm[parents[old]])
        new_len[new] = lens[old]
    order = [int(x) for x in rng.permutation(n_nodes)]
    return _from_lists(new_par, new_len, name, order)


def caterpillar_tree(trunk_lens: List[int], leaf_len: int,
                     name: str = "caterpillar") -> NodeTable:
    """A trunk of nodes (each the first child of the previous) with one leaf
    child per trunk node, packed in depth-first preorder: the whole trunk is
    contiguous, then the leaves deepest first.  Many short trunk nodes share
    each 128-token tile, and each of their leaves sees only part of it."""
    n = len(trunk_lens)
    parents = [-1] + list(range(n - 1)) + list(range(n))
    lens = list(trunk_lens) + [leaf_len] * n
    order = list(range(n)) + [n + i for i in reversed(range(n))]
    return _from_lists(parents, lens, name, order)


def dfs_preorder(parent) -> List[int]:
    """Node indices in depth-first preorder (roots and children in index
    order): the order in which a depth-first walk of the tree visits each
    node's segment as the new part of the current root-to-leaf path
    (AReaL-DTA, abstract)."""
    parent = np.asarray(parent, np.int64)
    children: List[List[int]] = [[] for _ in range(parent.shape[0])]
    roots = []
    for i, p in enumerate(parent):
        (children[p] if p >= 0 else roots).append(i)
    order: List[int] = []
    stack = roots[::-1]
    while stack:
        i = stack.pop()
        order.append(i)
        stack.extend(children[i][::-1])
    return order


def tree_stats(t: NodeTable) -> dict:
    """Shape statistics of a tree: leaves, paths, pair counts.

    ``pairs`` = sum over unique tokens of (number of ancestor tokens + 1),
    ``dense_pairs`` = the same count with every root-to-leaf path expanded
    into its own causal sequence.  These count work; they compute nothing of
    the attention itself.
    """
    m = t.num_nodes
    par = t.parent.astype(np.int64)
    ln = t.seg_len.astype(np.int64)
    children = [[] for _ in range(m)]
    for i in range(m):
        if par[i] >= 0:
            children[par[i]].append(i)
    # depth offset (ancestor tokens before the node) via iterative DFS
    off = np.zeros(m, np.int64)
    roots = [i for i in range(m) if par[i] < 0]
    stack = list(roots)
    while stack:
        i = stack.pop()
        for c in children[i]:
            off[c] = off[i] + ln[i]
            stack.append(c)
    leaves = [i for i in range(m) if not children[i]]
    n_desc_leaves = np.zeros(m, np.int64)
    # post-order accumulation of leaf counts
    order = []
    stack = list(roots)
    while stack:
        i = stack.pop()
        order.append(i)
        stack.extend(children[i])
    for i in reversed(order):
        n_desc_leaves[i] = 1 if not children[i] else sum(n_desc_leaves[c] for c in children[i])
    # pairs: node i contributes sum_{o=0}^{len-1} (off + o + 1)
    pairs = int(np.sum(ln * off + ln * (ln + 1) // 2))
    path_len = off + ln
    dense_pairs = int(sum(int(path_len[l]) * (int(path_len[l]) + 1) // 2 for l in leaves))
    return {
        "nodes": m,
        "leaves": len(leaves),
        "tokens": int(t.num_tokens),
        "max_path": int(max(path_len[l] for l in leaves)),
        "sum_path": int(sum(int(path_len[l]) for l in leaves)),
        "pairs": pairs,
        "dense_pairs": dense_pairs,
        "dense_ratio": dense_pairs / pairs,
    }


# ---------------------------------------------------------------------------
# The five benchmark workloads.  Sizes and head shapes are the workload
# definitions; the tree shapes mirror the pages' rollout trees (see module
# docstring).  ``scale`` is the softmax scale 1/sqrt(head_dim).

CONFIGS = {
    1: dict(name="tiny-binary", heads_q=1, heads_kv=1, head_dim=64, dtype="fp32",
            do_std=1.0),
    2: dict(name="grpo-star", heads_q=32, heads_kv=8, head_dim=128, dtype="bf16",
            do_std=1e-2),
    3: dict(name="agent-irregular", heads_q=32, heads_kv=8, head_dim=128,
            dtype="bf16", do_std=1e-2),
    4: dict(name="segment-search", heads_q=28, heads_kv=4, head_dim=128,
            dtype="bf16", do_std=1e-2),
    5: dict(name="long-trunk", heads_q=64, heads_kv=8, head_dim=128, dtype="bf16",
            do_std=1e-2),
}


def config_tree(i: int, seed: int = 0) -> NodeTable:
    if i == 1:
        return binary_tree(32, 16, 3, name="tiny-binary")
    if i == 2:
        return star_tree(1024, 16, 2048, name="grpo-star")
    if i == 3:
        return agent_tree(seed=seed, name="agent-irregular")
    if i == 4:
        return binary_tree(512, 512, 6, name="segment-search")
    if i == 5:
        return trunk_tree(seed=seed, name="long-trunk")
    raise ValueError(f"unknown config {i}")


def config_spec(i: int) -> dict:
    spec = dict(CONFIGS[i])
    spec["scale"] = 1.0 / float(np.sqrt(spec["head_dim"]))
    return spec
