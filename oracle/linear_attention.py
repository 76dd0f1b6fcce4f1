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


def tree_linear_attention(q, k, v, do, parent, seg_start, seg_len,
                          scale: float) -> Dict[str, np.ndarray]:
    """Forward and backward of tree linear attention by path expansion, fp64.

    ``q, do``: [N, Hq, D]; ``k, v``: [N, Hkv, D]; node table as in the
    library.  Returns ``o, dq [N,Hq,D]``, ``dk, dv [N,Hkv,D]``, ``mult [N]``
    and ``path_spread``, the largest difference between two paths' outputs
    for the same token.
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
    o = np.zeros((n, hq, d))
    dq = np.zeros((n, hq, d))
    dk = np.zeros((n, hkv, d))
    dv = np.zeros((n, hkv, d))
    seen = np.zeros((n, hq), bool)
    spread = 0.0
    for h in range(hq):
        g = h // gs
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
