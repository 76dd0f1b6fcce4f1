"""fp64 CPU oracle: tree attention as trajectory-wise dense causal attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
product path (the HIP library and its binding) never does; it shares no code
with this file.

What it computes.  Rollouts that share prefixes form a tree, and training
each root-to-leaf trajectory on its own recomputes the shared prefixes in the
forward and the backward pass (AReaL-DTA, abstract; HARTS, abstract).  Tree
attention must give the results of that trajectory-wise computation while
computing each shared prefix once (Tree Training, in the HARTS page's related
list: compute each shared prefix once and reuse it in forward and backward;
HARTS, abstract: numerical differences comparable to self-rerun variation).
So the oracle is the trajectory-wise computation itself:

1. every root-to-leaf path is expanded into its own token sequence (the
   concatenation of its nodes' segments, root first);
2. each path runs ordinary dense causal scaled-dot-product attention,
   forward and backward, in fp64;
3. per-path outputs are written to the unique tokens (they agree on every
   path through a token) and per-path gradients are summed onto the unique
   tokens.

Readings where the pages are silent (each listed in the design notes):
* a token attends to itself and to its ancestors (causal attention);
* ``dO`` given for a unique token is the total upstream gradient of that
  token; each of the ``mult(t)`` path copies of token t receives
  ``dO_t / mult(t)``, which makes the summed per-path gradients the exact
  gradient of the unique-token loss sum_t <dO_t, O_t>;
* LSE is the natural log of sum_j exp(scale * q.k_j), shape [Hq, N];
* grouped-query heads map q head h to kv head h // (Hq / Hkv).

Parity pins (tests/test_oracle.py): brute-force ancestor-masked softmax over
all unique tokens with torch fp64 autograd on random forests; torch's
``scaled_dot_product_attention(is_causal=True)`` on chains; central finite
differences; closed forms and invariances (gradient sums, scale identity,
first-token values, path consistency, segmentation / permutation / forest /
GQA invariance); hand-derived golden values in ``tests/golden``.  Every
function below is pinned by at least one of them.
"""

from __future__ import annotations

from typing import Dict, Iterable, List, Sequence

import numpy as np


# --------------------------------------------------------------------------
# tree structure

def root_to_leaf_paths(parent, seg_start, seg_len) -> List[np.ndarray]:
    """Packed row indices of every root-to-leaf trajectory, leaves in node-id
    order.  A leaf is a node that is nobody's parent."""
    parent = np.asarray(parent, np.int64)
    seg_start = np.asarray(seg_start, np.int64)
    seg_len = np.asarray(seg_len, np.int64)
    m = parent.shape[0]
    has_child = np.zeros(m, bool)
    for i in range(m):
        if parent[i] >= 0:
            has_child[parent[i]] = True
    paths = []
    for leaf in range(m):
        if has_child[leaf]:
            continue
        chain = []
        node = leaf
        while node >= 0:
            chain.append(node)
            if len(chain) > m:
                raise ValueError("parent pointers contain a cycle")
            node = parent[node]
        chain.reverse()
        paths.append(np.concatenate(
            [np.arange(seg_start[n], seg_start[n] + seg_len[n]) for n in chain]))
    return paths


def path_multiplicity(paths: Sequence[np.ndarray], n_tokens: int) -> np.ndarray:
    """Number of root-to-leaf paths that contain each packed token."""
    mult = np.zeros(n_tokens, np.int64)
    for p in paths:
        mult[p] += 1
    return mult


# --------------------------------------------------------------------------
# one trajectory: dense causal attention, forward and backward

def token_positions(parent, seg_start, seg_len, n_tokens: int):
    """Node index and trajectory position of every unique token.

    Walks every root-to-leaf path (``root_to_leaf_paths``): token t at index
    i of a path gets position i, and the node whose segment holds it.  A
    shared-prefix token occupies the same index on every path through it (its
    ancestors' tokens and the earlier tokens of its node precede it); the
    walk checks that agreement.  Returns (node_id, pos_id), int64 [N].
    """
    seg_start = np.asarray(seg_start, np.int64)
    seg_len = np.asarray(seg_len, np.int64)
    node_id = np.full(n_tokens, -1, np.int64)
    for i in range(seg_start.shape[0]):
        node_id[seg_start[i]:seg_start[i] + seg_len[i]] = i
    pos_id = np.full(n_tokens, -1, np.int64)
    for path in root_to_leaf_paths(parent, seg_start, seg_len):
        idx = np.arange(path.shape[0])
        seen = pos_id[path]
        if np.any((seen >= 0) & (seen != idx)):
            raise AssertionError("a token sits at different positions on two paths")
        pos_id[path] = idx
    if np.any(pos_id < 0) or np.any(node_id < 0):
        raise ValueError("the segments do not cover every token with a path")
    return node_id, pos_id


def causal_attention(q, k, v, do, scale: float, row_block: int = 4096):
    """Scaled dot-product attention with a causal mask on one sequence.

    ``q, k, v, do``: [L, D].  Returns ``o, lse, dq, dk, dv`` in fp64 with

        S = scale q k^T,  S_ij = -inf for j > i
        P = row softmax of S,  lse_i = log sum_j exp S_ij,  O = P v
        dP = dO v^T,  dS_ij = P_ij (dP_ij - sum_l P_il dP_il)
        dq = scale dS k,  dk = scale dS^T q,  dv = P^T dO

    Softmax rows are independent, so rows are taken ``row_block`` at a time
    purely to bound memory for long paths.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    L, D = q.shape
    o = np.empty((L, D))
    lse = np.empty(L)
    dq = np.empty((L, D))
    dk = np.zeros((L, D))
    dv = np.zeros((L, D))
    for r0 in range(0, L, row_block):
        r1 = min(L, r0 + row_block)
        kk, vv = k[:r1], v[:r1]
        s = scale * (q[r0:r1] @ kk.T)
        future = np.arange(r1)[None, :] > np.arange(r0, r1)[:, None]
        s[future] = -np.inf
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        l = e.sum(axis=1, keepdims=True)
        p = e / l
        lse[r0:r1] = (m + np.log(l))[:, 0]
        o[r0:r1] = p @ vv
        dp = do[r0:r1] @ vv.T
        ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
        dq[r0:r1] = scale * (ds @ kk)
        dk[:r1] += scale * (ds.T @ q[r0:r1])
        dv[:r1] += p.T @ do[r0:r1]
    return o, lse, dq, dk, dv


# --------------------------------------------------------------------------
# the whole tree

def _check_shapes(q, k, v, do):
    n, hq, d = q.shape
    if k.shape[0] != n or k.shape[2] != d or v.shape != k.shape or do.shape != q.shape:
        raise ValueError("inconsistent tensor shapes")
    hkv = k.shape[1]
    if hq % hkv:
        raise ValueError("query heads must be a multiple of kv heads")
    return n, hq, hkv, d


def tree_attention(q, k, v, do, parent, seg_start, seg_len, scale: float,
                   kv_heads: Iterable[int] | None = None,
                   row_block: int = 4096) -> Dict[str, np.ndarray]:
    """Forward and backward of tree attention by path expansion, fp64.

    ``q, do``: [N, Hq, D]; ``k, v``: [N, Hkv, D]; node table as in the
    library.  ``kv_heads`` restricts the work to those kv-head groups (all
    query heads of each group); entries of other heads are NaN.

    Returns ``o [N,Hq,D]``, ``lse [Hq,N]``, ``dq [N,Hq,D]``, ``dk, dv
    [N,Hkv,D]``, ``mult [N]`` and ``path_spread``: the largest difference
    between two paths' forward results for the same token (zero up to
    rounding when outputs are path-independent, as tree attention requires).
    """
    n, hq, hkv, d = _check_shapes(q, k, v, do)
    g_size = hq // hkv
    paths = root_to_leaf_paths(parent, seg_start, seg_len)
    mult = path_multiplicity(paths, n)
    if n and mult.min() < 1:
        raise ValueError("some token lies on no root-to-leaf path")
    groups = range(hkv) if kv_heads is None else list(kv_heads)
    o = np.full((n, hq, d), np.nan)
    lse = np.full((hq, n), np.nan)
    dq = np.full((n, hq, d), np.nan)
    dk = np.full((n, hkv, d), np.nan)
    dv = np.full((n, hkv, d), np.nan)
    spread = 0.0
    inv_mult = 1.0 / mult.astype(np.float64)
    for g in groups:
        dk[:, g] = 0.0
        dv[:, g] = 0.0
        kg = np.asarray(k[:, g], np.float64)
        vg = np.asarray(v[:, g], np.float64)
        for h in range(g * g_size, (g + 1) * g_size):
            dq[:, h] = 0.0
            qh = np.asarray(q[:, h], np.float64)
            doh = np.asarray(do[:, h], np.float64)
            seen = np.zeros(n, bool)
            for p in paths:
                op, lp, dqp, dkp, dvp = causal_attention(
                    qh[p], kg[p], vg[p], doh[p] * inv_mult[p][:, None], scale,
                    row_block)
                old = seen[p]
                if old.any():
                    spread = max(spread,
                                 float(np.abs(o[p[old], h] - op[old]).max()),
                                 float(np.abs(lse[h, p[old]] - lp[old]).max()))
                o[p, h] = op
                lse[h, p] = lp
                seen[p] = True
                # indices inside one path are distinct, so += scatters exactly
                dq[p, h] += dqp
                dk[p, g] += dkp
                dv[p, g] += dvp
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv, "mult": mult,
            "path_spread": spread}


def tree_attention_subset(q, k, v, do, parent, seg_start, seg_len, scale: float,
                          query_nodes: Iterable[int], **kw) -> Dict[str, np.ndarray]:
    """One call of the depth-first schedule: tree attention whose queries are
    the tokens of ``query_nodes`` only, fp64.

    AReaL-DTA (abstract) walks the tree depth first, keeping one root-to-leaf
    path resident, and still computes every shared prefix once.  One step of
    that walk computes the outputs of the rows it visits and their share of
    the gradients; the loss of such a step is sum over its query rows t of
    <dO_t, O_t>.  That loss is the unique-token loss of ``tree_attention``
    with dO set to zero on every other row, so this is ``tree_attention`` on
    that dO.  Returned: ``o``, ``lse`` and ``dq`` on the query rows (NaN on
    the other rows, which one step does not compute), ``dk``, ``dv`` on every
    row (zero where no query row sees the key), and ``rows``, the bool [N]
    mask of query rows.
    """
    n = q.shape[0]
    rows = np.zeros(n, bool)
    for node in query_nodes:
        s = int(seg_start[node])
        rows[s:s + int(seg_len[node])] = True
    do_step = np.where(rows[:, None, None], np.asarray(do, np.float64), 0.0)
    ref = tree_attention(q, k, v, do_step, parent, seg_start, seg_len, scale, **kw)
    ref["o"][~rows] = np.nan
    ref["lse"][:, ~rows] = np.nan
    ref["dq"][~rows] = np.nan
    ref["rows"] = rows
    return ref


# --------------------------------------------------------------------------
# sampled outputs for workloads too large for the full expansion

def _node_of_rows(seg_start, seg_len, rows):
    seg_start = np.asarray(seg_start, np.int64)
    seg_len = np.asarray(seg_len, np.int64)
    order = np.argsort(seg_start)
    starts = seg_start[order]
    pos = np.searchsorted(starts, rows, side="right") - 1
    node = order[pos]
    assert np.all(rows < seg_start[node] + seg_len[node])
    return node


def _context(parent, seg_start, seg_len, node, row):
    """Rows that token ``row`` (in ``node``) attends to, in path order."""
    chain = []
    a = int(parent[node])
    while a >= 0:
        chain.append(a)
        a = int(parent[a])
    chain.reverse()
    parts = [np.arange(seg_start[c], seg_start[c] + seg_len[c]) for c in chain]
    parts.append(np.arange(seg_start[node], row + 1))
    return np.concatenate(parts)


def query_rows(q, k, v, do, parent, seg_start, seg_len, scale: float,
               rows: Sequence[int], heads: Sequence[int]):
    """O, LSE and dQ of selected (row, head) pairs, fp64.

    A token's row of attention is the same on every path through it, so one
    row of the per-path computation (``causal_attention``'s formulas applied
    to the token's context) gives O and LSE; dQ sums that row's gradient over
    the token's ``mult`` paths, each carrying ``dO / mult``.
    Returns arrays ``o [R,H,D]``, ``lse [H,R]``, ``dq [R,H,D]``.
    """
    n, hq, hkv, d = _check_shapes(q, k, v, do)
    g_size = hq // hkv
    rows = np.asarray(rows, np.int64)
    paths = root_to_leaf_paths(parent, seg_start, seg_len)
    mult = path_multiplicity(paths, n)
    nodes = _node_of_rows(seg_start, seg_len, rows)
    o = np.empty((len(rows), len(heads), d))
    lse = np.empty((len(heads), len(rows)))
    dq = np.empty((len(rows), len(heads), d))
    for ri, (t, node) in enumerate(zip(rows, nodes)):
        ctx = _context(parent, seg_start, seg_len, node, int(t))
        for hi, h in enumerate(heads):
            g = h // g_size
            kc = np.asarray(k[ctx, g], np.float64)
            vc = np.asarray(v[ctx, g], np.float64)
            s = scale * (kc @ np.asarray(q[t, h], np.float64))
            m = s.max()
            e = np.exp(s - m)
            l = e.sum()
            p = e / l
            o[ri, hi] = p @ vc
            lse[hi, ri] = m + np.log(l)
            do_copy = np.asarray(do[t, h], np.float64) / mult[t]
            dp = vc @ do_copy
            ds = p * (dp - p @ dp)
            dq[ri, hi] = mult[t] * (scale * (ds @ kc))
    return o, lse, dq


def key_rows(q, k, v, do, parent, seg_start, seg_len, scale: float,
             keys: Sequence[int], kv_head: int, row_block: int = 1024):
    """dK and dV of selected packed key rows of one kv head, fp64.

    Sums, over every path that contains a selected key and every query head
    of the kv head's group, that key's column of the per-path backward
    (``causal_attention``'s formulas, rows taken ``row_block`` at a time from
    the first selected key onward; earlier rows cannot attend to it).
    Returns ``dk, dv`` of shape [K, D].
    """
    n, hq, hkv, d = _check_shapes(q, k, v, do)
    g_size = hq // hkv
    keys = np.asarray(keys, np.int64)
    paths = root_to_leaf_paths(parent, seg_start, seg_len)
    mult = path_multiplicity(paths, n)
    inv_mult = 1.0 / mult.astype(np.float64)
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
        L = len(p)
        kp = np.asarray(k[p, g], np.float64)
        vp = np.asarray(v[p, g], np.float64)
        for h in range(g * g_size, (g + 1) * g_size):
            qp = np.asarray(q[p, h], np.float64)
            dop = np.asarray(do[p, h], np.float64) * inv_mult[p][:, None]
            for r0 in range(int(kpos.min()), L, row_block):
                r1 = min(L, r0 + row_block)
                s = scale * (qp[r0:r1] @ kp[:r1].T)
                future = np.arange(r1)[None, :] > np.arange(r0, r1)[:, None]
                s[future] = -np.inf
                m = s.max(axis=1, keepdims=True)
                e = np.exp(s - m)
                pr = e / e.sum(axis=1, keepdims=True)
                dp = dop[r0:r1] @ vp[:r1].T
                ds = pr * (dp - (pr * dp).sum(axis=1, keepdims=True))
                # keys at path positions >= r1 are not seen by these rows
                live = kpos < r1
                kl, pl = kidx[live], kpos[live]
                dk[kl] += scale * (ds[:, pl].T @ qp[r0:r1])
                dv[kl] += pr[:, pl].T @ dop[r0:r1]
    return dk, dv


def key_rows_by_row(q, k, v, do, parent, seg_start, seg_len, scale: float,
                    keys: Sequence[int], kv_head: int, row_block: int = 1024):
    """dK and dV of selected packed key rows of one kv head, fp64, taken over
    unique query rows rather than over paths.

    The sums are those of ``key_rows``.  A unique row t lies on ``mult(t)``
    paths; each path copy has the same forward values (its context is the
    same ancestors-plus-earlier-rows list) and carries ``dO_t / mult(t)``, so
    its dS row is ``1 / mult(t)`` of the dS row formed with the whole
    ``dO_t``, and the ``mult(t)`` copies together contribute exactly that
    row once.  So each row that can see a selected key is visited once, with
    its whole dO: S = scale q_t K_ctx^T over its context (its node's
    ancestors root first, then its own segment up to t), P its softmax, dP =
    dO_t V_ctx^T, dS = P (dP - P.dP), and for every selected key u of the
    context dK_u += scale dS_u q_t, dV_u += P_u dO_t, summed over the group's
    query heads.  The rows that can see a key are the later rows of its node
    and every row of every node below it.  A node's rows are taken
    ``row_block`` at a time to bound memory.  Returns ``dk, dv`` [K, D].
    """
    n, hq, hkv, d = _check_shapes(q, k, v, do)
    g_size = hq // hkv
    parent = np.asarray(parent, np.int64)
    seg_start = np.asarray(seg_start, np.int64)
    seg_len = np.asarray(seg_len, np.int64)
    keys = np.asarray(keys, np.int64)
    m = parent.shape[0]
    children = [[] for _ in range(m)]
    for i in range(m):
        if parent[i] >= 0:
            children[parent[i]].append(i)
    key_node = _node_of_rows(seg_start, seg_len, keys)
    # nodes whose rows may see a selected key: the keys' nodes and everything
    # below them
    todo = sorted(set(int(x) for x in key_node))
    visit = set()
    while todo:
        a = todo.pop()
        if a in visit:
            continue
        visit.add(a)
        todo.extend(children[a])
    dk = np.zeros((len(keys), d))
    dv = np.zeros((len(keys), d))
    g = kv_head
    for node in sorted(visit):
        chain = []
        a = int(parent[node])
        while a >= 0:
            chain.append(a)
            a = int(parent[a])
        chain.reverse()
        anc = (np.concatenate([np.arange(seg_start[c], seg_start[c] + seg_len[c]) for c in chain])
               if chain else np.zeros(0, np.int64))
        own = np.arange(seg_start[node], seg_start[node] + seg_len[node])
        ctx_all = np.concatenate([anc, own])
        col = {int(t): i for i, t in enumerate(ctx_all)}
        sel = [(ki, col[int(t)]) for ki, t in enumerate(keys) if int(t) in col]
        if not sel:
            continue
        kidx = np.array([s[0] for s in sel])
        kcol = np.array([s[1] for s in sel])
        A = anc.shape[0]
        # rows of this node before its first selected own key see none of them
        # unless a selected key is an ancestor row
        first = 0 if kcol.min() < A else int(kcol.min()) - A
        kc = np.asarray(k[ctx_all, g], np.float64)
        vc = np.asarray(v[ctx_all, g], np.float64)
        for r0 in range(first, own.shape[0], row_block):
            r1 = min(own.shape[0], r0 + row_block)
            rows = own[r0:r1]
            width = A + r1  # context columns any of these rows can see
            future = np.arange(width)[None, :] > (A + np.arange(r0, r1))[:, None]
            live = kcol < width
            kl, cl = kidx[live], kcol[live]
            for h in range(g * g_size, (g + 1) * g_size):
                qr = np.asarray(q[rows, h], np.float64)
                dor = np.asarray(do[rows, h], np.float64)
                s = scale * (qr @ kc[:width].T)
                s[future] = -np.inf
                mx = s.max(axis=1, keepdims=True)
                e = np.exp(s - mx)
                pr = e / e.sum(axis=1, keepdims=True)
                dp = dor @ vc[:width].T
                ds = pr * (dp - (pr * dp).sum(axis=1, keepdims=True))
                dk[kl] += scale * (ds[:, cl].T @ qr)
                dv[kl] += pr[:, cl].T @ dor
    return dk, dv
