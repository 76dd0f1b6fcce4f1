"""Oracle for the passes either side of tree attention (test infrastructure).

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may use
it, and it shares no code with the HIP library.

Rollouts that share a prefix are stored once (AReaL-DTA, abstract: the
rollouts of one prompt form a prefix tree whose shared prefixes are computed
once; HARTS, abstract: arbitrary rollout trees processed in one packed call
while per-trajectory objectives keep their interface).  This module writes
out, plainly:

* ``build_tree``: prefix compression -- a dictionary trie of the token
  sequences, chains of single-child tokens merged into segments, nodes
  numbered in depth-first preorder with children in order of first
  appearance;
* ``gather_rows`` / ``scatter_sum_rows``: handing per-unique-token rows back
  to trajectory positions, and summing per-position rows onto unique tokens
  (the adjoint, used for gradients);
* ``rope``: rotary position embedding with rotate-half pairing, in fp64.
  The pages do not fix a positional scheme; a token's position on every path
  through it is its depth, and the plainest reading is to rotate each unique
  token at that position (the rotate-half convention and theta = 10000 are
  the common defaults and are recorded as a reading).

Pins live in ``tests/test_oracle_prefix.py``: brute-force prefix sets and
counts, round trips, the adjoint identity, the complex-number form of the
rotation, norm preservation, inverse, and the relative-position property of
rotary embeddings.
"""

from __future__ import annotations

from typing import List, Sequence

import numpy as np


def build_tree(trajectories: Sequence[Sequence[int]]):
    """Prefix tree of token sequences.

    Returns a dict with the node table (parent, seg_start, seg_len), the
    packed unique token ids, the unique row of every trajectory position
    (flattened in trajectory order), and the number of trajectories through
    each unique row.
    """
    # trie: node 0 is a virtual root; each other node is one distinct prefix
    token = [-1]
    children: List[List[int]] = [[]]
    child_of: List[dict] = [{}]
    pos_node = []
    for traj in trajectories:
        cur = 0
        for tok in traj:
            tok = int(tok)
            if tok not in child_of[cur]:
                token.append(tok)
                children.append([])
                child_of.append({})
                child_of[cur][tok] = len(token) - 1
                children[cur].append(len(token) - 1)
            cur = child_of[cur][tok]
            pos_node.append(cur)
    # merge single-child chains, number nodes in depth-first preorder
    parent, seg_start, seg_len, unique = [], [], [], []
    row_of = {}

    def visit(start: int, parent_node: int) -> None:
        node = len(parent)
        parent.append(parent_node)
        seg_start.append(len(unique))
        t = start
        length = 0
        while True:
            row_of[t] = len(unique)
            unique.append(token[t])
            length += 1
            if len(children[t]) != 1:
                break
            t = children[t][0]
        seg_len.append(length)
        for c in children[t]:
            visit(c, node)

    import sys
    old = sys.getrecursionlimit()
    sys.setrecursionlimit(max(old, 10000))
    try:
        for c in children[0]:
            visit(c, -1)
    finally:
        sys.setrecursionlimit(old)
    traj_index = np.array([row_of[p] for p in pos_node], np.int64)
    mult = np.bincount(traj_index, minlength=len(unique)).astype(np.int64)
    return {
        "parent": np.array(parent, np.int64),
        "seg_start": np.array(seg_start, np.int64),
        "seg_len": np.array(seg_len, np.int64),
        "unique_tokens": np.array(unique, np.int64),
        "traj_index": traj_index,
        "mult": mult,
    }


def gather_rows(src: np.ndarray, index: np.ndarray) -> np.ndarray:
    """out[i] = src[index[i]]."""
    return np.asarray(src)[np.asarray(index, np.int64)]


def scatter_sum_rows(src: np.ndarray, index: np.ndarray, num_rows: int) -> np.ndarray:
    """out[u] = sum of src[i] over the positions i with index[i] == u (fp64)."""
    src = np.asarray(src, np.float64)
    out = np.zeros((num_rows,) + src.shape[1:], np.float64)
    for i, u in enumerate(np.asarray(index, np.int64)):
        out[u] += src[i]
    return out


def rope(x: np.ndarray, pos: np.ndarray, theta: float = 10000.0, inverse: bool = False):
    """Rotary embedding of x [N, H, D] at positions pos [N], rotate-half
    pairing: (x_i, x_{i+D/2}) rotated by pos * theta^(-2i/D), in fp64."""
    x = np.asarray(x, np.float64)
    n, h, d = x.shape
    half = d // 2
    i = np.arange(half, dtype=np.float64)
    ang = np.asarray(pos, np.float64)[:, None] * theta ** (-2.0 * i / d)[None, :]
    if inverse:
        ang = -ang
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)
