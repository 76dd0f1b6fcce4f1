"""fp64 CPU oracle: causal linear attention over a rollout prefix tree.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
product path (the HIP library and its binding) never does; it shares no code
with this file.

What it computes.  HARTS (abstract) trains hybrid-attention models over
arbitrary rollout trees: besides full attention, their chunkwise
linear-attention layers run over the tree in one packed call, with state
handed from a prefix to its branches and gradients propagated back through
those handoffs, while keeping the results of trajectory-wise training.  The
pages name no gate, decay or normaliser, so the oracle takes the plainest
linear attention: causal, unnormalised, ungated,

    o_t = scale * sum_{s <= t on t's root-to-leaf path} (q_t . k_s) v_s
        = scale * S_t^T q_t,   S_t = sum_{s <= t} k_s v_s^T  (running state).

As for softmax tree attention, the oracle is the trajectory-wise computation
itself:

1. every root-to-leaf path is expanded into its own token sequence;
2. each path runs the dense quadratic form of causal linear attention,
   forward and backward, in fp64;
3. per-path outputs are written to the unique tokens (they agree on every
   path through a token) and per-path gradients are summed onto them, each of
   the ``mult(t)`` path copies of token t receiving ``dO_t / mult(t)``, so the
   sum is the gradient of the unique-token loss sum_t <dO_t, O_t>.

How a chunkwise kernel partitions a path (chunk size, where states are
materialised) changes only the rounding, not this result.

Readings where the pages are silent (each listed in the design notes): the
recurrence above; a token attends to itself and its ancestors; query head h
reads key/value head h // (Hq / Hkv).

Parity pins (tests/test_oracle_linear.py): brute force over all unique tokens
with an ancestor mask and torch fp64 autograd; the running-state recurrence
on chains, differentiated by torch autograd; central finite differences;
closed forms on a hand-solved three-node tree; the homogeneity identities
<dQ, Q> = <dK, K> = <dV, V> = sum_t <dO_t, O_t>; path consistency.
"""

from __future__ import annotations

from typing import Dict

import numpy as np

from .path_expansion import path_multiplicity, root_to_leaf_paths


def causal_linear_attention(q, k, v, do, scale: float):
    """Causal linear attention on one sequence, fp64, quadratic form.

    ``q, k, v, do``: [L, D].  Forward: A = scale * tril(Q K^T) (entry (t, s)
    kept for s <= t), O = A V.  Backward of the loss sum <dO, O>:
    dV = A^T dO; G = scale * tril(dO V^T) is the gradient with respect to
    Q K^T; dQ = G K; dK = G^T Q.  Returns (o, dq, dk, dv).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    a = scale * np.tril(q @ k.T)
    o = a @ v
    g = scale * np.tril(do @ v.T)
    return o, g @ k, g.T @ q, a.T @ do


def tree_linear_attention(q, k, v, do, parent, seg_start, seg_len, scale: float,
                          kv_heads=None) -> Dict[str, np.ndarray]:
    """Forward and backward of tree linear attention by path expansion, fp64.

    ``q, do``: [N, Hq, D]; ``k, v``: [N, Hkv, D]; node table as in the
    library.  ``kv_heads`` restricts the work to those kv-head groups (all
    query heads of each group); entries of other heads are NaN.  Returns
    ``o, dq [N,Hq,D]``, ``dk, dv [N,Hkv,D]``, ``mult [N]`` and
    ``path_spread``, the largest difference between two paths' outputs for
    the same token.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    if q.ndim != 3 or k.shape != v.shape or q.shape != do.shape:
        raise ValueError("expected q, do [N, Hq, D] and k, v [N, Hkv, D]")
    n, hq, d = q.shape
    hkv = k.shape[1]
    if k.shape[0] != n or k.shape[2] != d or hkv < 1 or hq % hkv:
        raise ValueError("head counts or sizes disagree")
    gs = hq // hkv
    paths = root_to_leaf_paths(parent, seg_start, seg_len)
    mult = path_multiplicity(paths, n)
    if n and mult.min() < 1:
        raise ValueError("some token lies on no root-to-leaf path")
    inv_mult = 1.0 / mult.astype(np.float64)
    groups = set(range(hkv) if kv_heads is None else kv_heads)
    o = np.full((n, hq, d), np.nan)
    dq = np.full((n, hq, d), np.nan)
    dk = np.full((n, hkv, d), np.nan)
    dv = np.full((n, hkv, d), np.nan)
    for g in groups:
        o[:, g * gs:(g + 1) * gs] = 0.0
        dq[:, g * gs:(g + 1) * gs] = 0.0
        dk[:, g] = 0.0
        dv[:, g] = 0.0
    seen = np.zeros((n, hq), bool)
    spread = 0.0
    for h in range(hq):
        g = h // gs
        if g not in groups:
            continue
        for p in paths:
            op, dqp, dkp, dvp = causal_linear_attention(
                q[p, h], k[p, g], v[p, g], do[p, h] * inv_mult[p][:, None], scale)
            old = seen[p, h]
            if old.any():
                spread = max(spread, float(np.abs(o[p[old], h] - op[old]).max()))
            o[p, h] = op
            seen[p, h] = True
            # indices inside one path are distinct, so += scatters exactly
            dq[p, h] += dqp
            dk[p, g] += dkp
            dv[p, g] += dvp
    return {"o": o, "dq": dq, "dk": dk, "dv": dv, "mult": mult, "path_spread": spread}


# --------------------------------------------------------------------------
# sampled outputs for workloads too large for the full expansion

def _ancestor_context(parent, seg_start, seg_len, row: int) -> np.ndarray:
    """Rows that token ``row`` attends to, root first: the segments of its
    node's proper ancestors, then its own node up to and including it."""
    seg_start = np.asarray(seg_start, np.int64)
    seg_len = np.asarray(seg_len, np.int64)
    node = int(np.nonzero((seg_start <= row) & (row < seg_start + seg_len))[0][0])
    chain = []
    a = int(parent[node])
    while a >= 0:
        chain.append(a)
        a = int(parent[a])
    parts = [np.arange(seg_start[c], seg_start[c] + seg_len[c]) for c in reversed(chain)]
    parts.append(np.arange(seg_start[node], row + 1))
    return np.concatenate(parts)


def linear_query_rows(q, k, v, do, parent, seg_start, seg_len, scale: float, rows, heads):
    """O and dQ of selected (row, head) pairs, fp64.

    A token's context (its path prefix) is the same on every path through
    it, so one row of ``causal_linear_attention`` gives O; its dQ row sums
    the ``mult`` path copies, each carrying dO / mult, which is the row for
    the full dO.  Returns ``o, dq`` of shape [R, H, D].
    """
    hq, hkv = q.shape[1], k.shape[1]
    gs = hq // hkv
    o = np.empty((len(rows), len(heads), q.shape[2]))
    dq = np.empty_like(o)
    for ri, t in enumerate(rows):
        ctx = _ancestor_context(parent, seg_start, seg_len, int(t))
        for hi, h in enumerate(heads):
            kc = np.asarray(k[ctx, h // gs], np.float64)
            vc = np.asarray(v[ctx, h // gs], np.float64)
            o[ri, hi] = scale * ((kc @ np.asarray(q[t, h], np.float64)) @ vc)
            dq[ri, hi] = scale * ((vc @ np.asarray(do[t, h], np.float64)) @ kc)
    return o, dq


def linear_key_rows(q, k, v, do, parent, seg_start, seg_len, scale: float, keys,
                    kv_head: int):
    """dK and dV of selected packed key rows of one kv head, fp64.

    Sums, over every path containing a selected key and every query head of
    the kv head's group, that key's column of the per-path gradients of
    ``causal_linear_attention`` (rows at or after the key, dO / mult per path
    copy).  Returns ``dk, dv`` of shape [K, D].
    """
    n, hq = q.shape[0], q.shape[1]
    gs = hq // k.shape[1]
    keys = np.asarray(keys, np.int64)
    paths = root_to_leaf_paths(parent, seg_start, seg_len)
    inv_mult = 1.0 / path_multiplicity(paths, n).astype(np.float64)
    d = q.shape[2]
    dk = np.zeros((len(keys), d))
    dv = np.zeros((len(keys), d))
    g = kv_head
    for p in paths:
        where = {int(t): i for i, t in enumerate(p)}
        sel = [(ki, where[int(t)]) for ki, t in enumerate(keys) if int(t) in where]
        if not sel:
            continue
        kidx = np.array([s[0] for s in sel])
        kpos = np.array([s[1] for s in sel])
        r0 = int(kpos.min())
        later = np.arange(r0, len(p))[:, None] >= kpos[None, :]  # row sees key
        ks_ = np.asarray(k[p[kpos], g], np.float64)
        vs_ = np.asarray(v[p[kpos], g], np.float64)
        for h in range(g * gs, (g + 1) * gs):
            qr = np.asarray(q[p[r0:], h], np.float64)
            dor = np.asarray(do[p[r0:], h], np.float64) * inv_mult[p[r0:]][:, None]
            gcol = scale * (dor @ vs_.T) * later  # dL / d(q_t . k_s)
            acol = scale * (qr @ ks_.T) * later   # A[t, s]
            np.add.at(dk, kidx, gcol.T @ qr)
            np.add.at(dv, kidx, acol.T @ dor)
    return dk, dv
