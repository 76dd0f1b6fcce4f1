"""Pins for the fp64 oracle, independent of the oracle's own code.

Each pin checks the oracle against something other than itself:
* a brute-force dense softmax over all unique tokens with an ancestor mask
  built by transitive closure of the parent relation, differentiated by torch
  fp64 autograd (the packed tree-mask formulation that AReaL-DTA's abstract
  names as the alternative to per-trajectory training);
* torch's scaled_dot_product_attention(is_causal=True) on single paths, where
  tree attention is ordinary causal attention;
* central finite differences of the unique-token loss;
* closed forms and invariances that any correct implementation satisfies;
* a hand-derived golden tree (tests/golden/tiny_tree_uniform.json).
"""

import json
import os

import numpy as np
import pytest
import torch

import oracle
import oracle.path_expansion as ota
from tree_inputs import (NodeTable, binary_tree, chain_tree, config_spec, config_tree,
                         make_inputs, random_tree, star_tree, tree_stats, bf16_round_bits,
                         bf16_bits_to_f32)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_qkvdo(rng, n, hq, hkv, d):
    q = rng.standard_normal((n, hq, d))
    k = rng.standard_normal((n, hkv, d))
    v = rng.standard_normal((n, hkv, d))
    do = rng.standard_normal((n, hq, d))
    return q, k, v, do


def _run(t: NodeTable, q, k, v, do, scale, **kw):
    return oracle.tree_attention(q, k, v, do, t.parent, t.seg_start, t.seg_len, scale, **kw)


def visibility_mask(t: NodeTable) -> np.ndarray:
    """[N, N] bool: token t may see token u.  Built independently of the
    oracle: node-level ancestry by Warshall's transitive closure of the parent
    relation, then t sees u iff u's node is a proper ancestor of t's node, or
    both share a node and u is not later in the segment."""
    m = t.num_nodes
    n = t.num_tokens
    anc = np.eye(m, dtype=bool)
    for i in range(m):
        if t.parent[i] >= 0:
            anc[i, t.parent[i]] = True
    for mid in range(m):
        anc |= anc[:, mid:mid + 1] & anc[mid:mid + 1, :]
    node_of = np.empty(n, np.int64)
    offset = np.empty(n, np.int64)
    for i in range(m):
        s, l = int(t.seg_start[i]), int(t.seg_len[i])
        node_of[s:s + l] = i
        offset[s:s + l] = np.arange(l)
    a, b = node_of[:, None], node_of[None, :]
    return (anc[a, b] & (a != b)) | ((a == b) & (offset[None, :] <= offset[:, None]))


def brute_force(t: NodeTable, q, k, v, do, scale):
    """Dense masked attention over all N unique tokens, torch fp64 autograd,
    with the independent mask of ``visibility_mask``."""
    m = t.num_nodes
    n = t.num_tokens
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
        s = scale * (Q[:, h] @ K[:, g].T)
        s = s.masked_fill(~mask_t, float("-inf"))
        lses.append(torch.logsumexp(s, dim=1))
        outs.append(torch.softmax(s, dim=1) @ V[:, g])
    O = torch.stack(outs, dim=1)
    (O * dO).sum().backward()
    return {"o": O.detach().numpy(), "lse": torch.stack(lses).detach().numpy(),
            "dq": Q.grad.numpy(), "dk": K.grad.numpy(), "dv": V.grad.numpy()}


def _rel(a, b):
    return float(np.linalg.norm((a - b).ravel()) / max(np.linalg.norm(b.ravel()), 1e-300))


# ---------------------------------------------------------------- golden

def test_golden_tiny_tree():
    with open(os.path.join(GOLDEN, "tiny_tree_uniform.json")) as f:
        gd = json.load(f)
    t = NodeTable(np.array(gd["parent"], np.int32), np.array(gd["seg_start"], np.int32),
                  np.array(gd["seg_len"], np.int32), 4)
    q = np.array(gd["q"], float)[:, None, :]
    k = np.array(gd["k"], float)[:, None, :]
    v = np.array(gd["v"], float)[:, None, :]
    do = np.array(gd["do"], float)[:, None, :]
    r = _run(t, q, k, v, do, gd["scale"])
    ex = gd["expected"]
    np.testing.assert_allclose(r["o"][:, 0], ex["o"], atol=1e-14)
    np.testing.assert_allclose(r["lse"][0], ex["lse"], atol=1e-14)
    np.testing.assert_allclose(r["dq"][:, 0], ex["dq"], atol=1e-14)
    np.testing.assert_allclose(r["dk"][:, 0], ex["dk"], atol=1e-14)
    np.testing.assert_allclose(r["dv"][:, 0], ex["dv"], atol=1e-14)
    # the sampled-row and sampled-key functions agree with the hand values too
    o, lse, dq = oracle.query_rows(q, k, v, do, t.parent, t.seg_start, t.seg_len,
                                   gd["scale"], [0, 1, 2, 3], [0])
    np.testing.assert_allclose(o[:, 0], ex["o"], atol=1e-14)
    np.testing.assert_allclose(lse[0], ex["lse"], atol=1e-14)
    np.testing.assert_allclose(dq[:, 0], ex["dq"], atol=1e-14)
    dk, dv = oracle.key_rows(q, k, v, do, t.parent, t.seg_start, t.seg_len, gd["scale"],
                             [0, 1, 2, 3], 0)
    np.testing.assert_allclose(dk, ex["dk"], atol=1e-14)
    np.testing.assert_allclose(dv, ex["dv"], atol=1e-14)


# ------------------------------------------------------------- positions

def test_positions_golden():
    with open(os.path.join(GOLDEN, "tiny_tree_uniform.json")) as f:
        gd = json.load(f)
    node_id, pos_id = oracle.token_positions(gd["parent"], gd["seg_start"], gd["seg_len"], 4)
    assert node_id.tolist() == gd["expected"]["node_id"]
    assert pos_id.tolist() == gd["expected"]["pos_id"]


@pytest.mark.parametrize("seed", range(6))
def test_positions_equal_visible_count(seed):
    """The position of a token is the number of tokens it sees besides
    itself: checked against the independent transitive-closure mask."""
    rng = np.random.default_rng(100 + seed)
    t = random_tree(rng, int(rng.integers(1, 12)), max_len=40, n_roots=int(rng.integers(1, 3)),
                    shuffle=bool(seed % 2))
    node_id, pos_id = oracle.token_positions(t.parent, t.seg_start, t.seg_len, t.num_tokens)
    mask = visibility_mask(t)
    np.testing.assert_array_equal(pos_id, mask.sum(axis=1) - 1)
    for i in range(t.num_nodes):
        s, l = int(t.seg_start[i]), int(t.seg_len[i])
        assert np.all(node_id[s:s + l] == i)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_positions_sum_to_pairs(cfg):
    """sum_t (pos(t) + 1) is the number of (query, key) pairs, counted by the
    tree generator independently of the oracle."""
    t = config_tree(cfg)
    _, pos_id = oracle.token_positions(t.parent, t.seg_start, t.seg_len, t.num_tokens)
    assert int((pos_id + 1).sum()) == tree_stats(t)["pairs"]


# ------------------------------------------------------------ brute force

@pytest.mark.parametrize("seed,nodes,roots,hq,hkv,d", [
    (0, 1, 1, 1, 1, 4), (1, 5, 1, 2, 1, 8), (2, 9, 2, 4, 2, 8), (3, 14, 1, 3, 3, 16),
    (4, 20, 3, 4, 1, 8), (5, 12, 1, 6, 2, 4),
])
def test_bruteforce_random_forest(seed, nodes, roots, hq, hkv, d):
    rng = np.random.default_rng(seed)
    t = random_tree(rng, nodes, max_len=12, n_roots=roots)
    q, k, v, do = _rand_qkvdo(rng, t.num_tokens, hq, hkv, d)
    scale = 1.0 / np.sqrt(d)
    r = _run(t, q, k, v, do, scale)
    b = brute_force(t, q, k, v, do, scale)
    for key in ("o", "lse", "dq", "dk", "dv"):
        assert _rel(r[key], b[key]) < 1e-12, key
    assert r["path_spread"] < 1e-12


def test_bruteforce_config1():
    t = config_tree(1)
    spec = config_spec(1)
    x = make_inputs(t.num_tokens, 1, 1, 64, dtype="fp32", do_std=1.0)
    r = _run(t, x.q, x.k, x.v, x.do, spec["scale"])
    b = brute_force(t, x.q.astype(float), x.k.astype(float), x.v.astype(float),
                    x.do.astype(float), spec["scale"])
    for key in ("o", "lse", "dq", "dk", "dv"):
        assert _rel(r[key], b[key]) < 1e-12, key


def test_bruteforce_catches_planted_mistakes(monkeypatch):
    """Plausible oracle mistakes (a dropped dO split, a wrong scale) must be
    caught by the brute-force pin."""
    rng = np.random.default_rng(11)
    t = random_tree(rng, 8, max_len=6)
    q, k, v, do = _rand_qkvdo(rng, t.num_tokens, 2, 1, 4)
    b = brute_force(t, q, k, v, do, 0.5)
    monkeypatch.setattr(ota, "path_multiplicity", lambda paths, n: np.ones(n, np.int64))
    r = _run(t, q, k, v, do, 0.5)
    assert _rel(r["dk"], b["dk"]) > 1e-3
    monkeypatch.undo()
    r = _run(t, q, k, v, do, 0.5 * 1.01)
    assert _rel(r["o"], b["o"]) > 1e-6


# ------------------------------------------------------- library routine

def _sdpa_ref(q, k, v, do, scale):
    """torch SDPA with a causal mask, fp64, per head (q [L,H,D])."""
    hq, hkv = q.shape[1], k.shape[1]
    gs = hq // hkv
    Q = torch.tensor(q.transpose(1, 0, 2), requires_grad=True)
    K = torch.tensor(np.repeat(k, gs, axis=1).transpose(1, 0, 2), requires_grad=True)
    V = torch.tensor(np.repeat(v, gs, axis=1).transpose(1, 0, 2), requires_grad=True)
    O = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=scale)
    (O * torch.tensor(do.transpose(1, 0, 2))).sum().backward()
    dk = K.grad.numpy().transpose(1, 0, 2).reshape(q.shape[0], hkv, gs, -1).sum(2)
    dv = V.grad.numpy().transpose(1, 0, 2).reshape(q.shape[0], hkv, gs, -1).sum(2)
    return O.detach().numpy().transpose(1, 0, 2), Q.grad.numpy().transpose(1, 0, 2), dk, dv


@pytest.mark.parametrize("lens", [[1], [7], [5, 3, 9], [16, 16, 16, 1]])
def test_chain_equals_sdpa(lens):
    rng = np.random.default_rng(len(lens))
    t = chain_tree(lens)
    q, k, v, do = _rand_qkvdo(rng, t.num_tokens, 4, 2, 8)
    r = _run(t, q, k, v, do, 0.3)
    o, dq, dk, dv = _sdpa_ref(q, k, v, do, 0.3)
    assert _rel(r["o"], o) < 1e-12
    assert _rel(r["dq"], dq) < 1e-12
    assert _rel(r["dk"], dk) < 1e-12
    assert _rel(r["dv"], dv) < 1e-12


def test_forest_of_chains_equals_sdpa_per_sequence():
    rng = np.random.default_rng(3)
    # two independent chains packed back to back (a forest of two paths)
    t = NodeTable(np.array([-1, 0, -1], np.int32), np.array([0, 6, 10], np.int32),
                  np.array([6, 4, 9], np.int32), 19)
    q, k, v, do = _rand_qkvdo(rng, 19, 2, 2, 8)
    r = _run(t, q, k, v, do, 0.25)
    for sl in (slice(0, 10), slice(10, 19)):
        o, dq, dk, dv = _sdpa_ref(q[sl], k[sl], v[sl], do[sl], 0.25)
        assert _rel(r["o"][sl], o) < 1e-12
        assert _rel(r["dq"][sl], dq) < 1e-12
        assert _rel(r["dk"][sl], dk) < 1e-12
        assert _rel(r["dv"][sl], dv) < 1e-12


# ---------------------------------------------------- finite differences

def test_finite_differences():
    rng = np.random.default_rng(5)
    t = random_tree(rng, 5, max_len=4)
    n = t.num_tokens
    assert n <= 64
    q, k, v, do = _rand_qkvdo(rng, n, 2, 1, 3)
    scale = 0.7
    r = _run(t, q, k, v, do, scale)

    def loss(args):
        o = _run(t, args["q"], args["k"], args["v"], do, scale)["o"]
        return float(np.sum(o * do))

    base = {"q": q, "k": k, "v": v}
    eps = 1e-6
    for name, grad in (("q", r["dq"]), ("k", r["dk"]), ("v", r["dv"])):
        arr = base[name]
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            a_p = arr.copy()
            a_p[idx] += eps
            a_m = arr.copy()
            a_m[idx] -= eps
            num[idx] = (loss({**base, name: a_p}) - loss({**base, name: a_m})) / (2 * eps)
        np.testing.assert_allclose(grad, num, atol=1e-7, rtol=1e-6, err_msg=name)


# -------------------------------------------- closed forms / invariances

def _tree_and_inputs(seed=7, nodes=15, hq=4, hkv=2, d=8, roots=1):
    rng = np.random.default_rng(seed)
    t = random_tree(rng, nodes, max_len=20, n_roots=roots)
    return t, _rand_qkvdo(rng, t.num_tokens, hq, hkv, d)


def test_closed_forms():
    t, (q, k, v, do) = _tree_and_inputs()
    r = _run(t, q, k, v, do, 0.35)
    gs = q.shape[1] // k.shape[1]
    for g in range(k.shape[1]):
        hs = slice(g * gs, (g + 1) * gs)
        # each softmax row sums to one, so sum_u dV_u = sum of dO over the group
        np.testing.assert_allclose(r["dv"][:, g].sum(0), do[:, hs].sum((0, 1)), atol=1e-11)
        # softmax is shift invariant per row, so sum_u dK_u = 0
        np.testing.assert_allclose(r["dk"][:, g].sum(0), 0.0, atol=1e-11)
    # scores depend on q.k only: q*(1+e), k/(1+e) leaves them fixed
    np.testing.assert_allclose(np.sum(r["dq"] * q), np.sum(r["dk"] * k), rtol=1e-10)
    # each output row lies in the convex hull of the V rows it sees
    assert np.all(r["o"] <= v.max(0).max(0) + 1e-12)
    assert np.all(r["o"] >= v.min(0).min(0) - 1e-12)


def test_first_token_of_each_root():
    t, (q, k, v, do) = _tree_and_inputs(roots=3)
    scale = 0.35
    r = _run(t, q, k, v, do, scale)
    gs = q.shape[1] // k.shape[1]
    for i in np.nonzero(t.parent < 0)[0]:
        s0 = int(t.seg_start[i])
        for h in range(q.shape[1]):
            g = h // gs
            np.testing.assert_allclose(r["o"][s0, h], v[s0, g], atol=1e-14)
            np.testing.assert_allclose(r["lse"][h, s0], scale * q[s0, h] @ k[s0, g], atol=1e-13)


def test_segmentation_invariance():
    """Splitting a node's segment into a parent->child chain changes nothing."""
    t, (q, k, v, do) = _tree_and_inputs(seed=8)
    r = _run(t, q, k, v, do, 0.4)
    i = int(np.argmax(t.seg_len))
    L = int(t.seg_len[i])
    assert L >= 2
    cut = L // 2
    m = t.num_nodes
    par = np.append(t.parent, i).astype(np.int32)
    # children of i now hang below the new tail node m
    for c in range(m):
        if t.parent[c] == i:
            par[c] = m
    st = np.append(t.seg_start, t.seg_start[i] + cut).astype(np.int32)
    ln = np.append(t.seg_len, L - cut).astype(np.int32)
    ln[i] = cut
    t2 = NodeTable(par, st, ln, t.num_tokens)
    r2 = _run(t2, q, k, v, do, 0.4)
    for key in ("o", "lse", "dq", "dk", "dv"):
        assert _rel(r2[key], r[key]) < 1e-12, key


def test_permutation_invariance():
    """Relabelling nodes and repacking segments only permutes rows."""
    t, (q, k, v, do) = _tree_and_inputs(seed=9)
    r = _run(t, q, k, v, do, 0.4)
    rng = np.random.default_rng(99)
    m = t.num_nodes
    perm = rng.permutation(m)  # old id -> new id
    order = rng.permutation(m)  # packing order of new ids
    par = np.empty(m, np.int32)
    ln = np.empty(m, np.int32)
    for old in range(m):
        par[perm[old]] = -1 if t.parent[old] < 0 else perm[t.parent[old]]
        ln[perm[old]] = t.seg_len[old]
    st = np.empty(m, np.int32)
    pos = 0
    for new in order:
        st[new] = pos
        pos += ln[new]
    t2 = NodeTable(par, st, ln, t.num_tokens)
    rowmap = np.empty(t.num_tokens, np.int64)  # new row -> old row
    for old in range(m):
        new = perm[old]
        rowmap[st[new]:st[new] + ln[new]] = np.arange(t.seg_start[old], t.seg_start[old] + t.seg_len[old])
    r2 = _run(t2, q[rowmap], k[rowmap], v[rowmap], do[rowmap], 0.4)
    for key in ("o", "dq", "dk", "dv"):
        assert _rel(r2[key], r[key][rowmap]) < 1e-12, key
    assert _rel(r2["lse"], r["lse"][:, rowmap]) < 1e-12


def test_forest_is_independent_trees():
    rng = np.random.default_rng(12)
    a = random_tree(rng, 6, max_len=10, shuffle=False)
    b = random_tree(rng, 7, max_len=10, shuffle=False)
    par = np.concatenate([a.parent, np.where(b.parent < 0, -1, b.parent + a.num_nodes)]).astype(np.int32)
    st = np.concatenate([a.seg_start, b.seg_start + a.num_tokens]).astype(np.int32)
    ln = np.concatenate([a.seg_len, b.seg_len]).astype(np.int32)
    f = NodeTable(par, st, ln, a.num_tokens + b.num_tokens)
    q, k, v, do = _rand_qkvdo(rng, f.num_tokens, 2, 1, 8)
    rf = _run(f, q, k, v, do, 0.3)
    sa = slice(0, a.num_tokens)
    sb = slice(a.num_tokens, f.num_tokens)
    ra = _run(a, q[sa], k[sa], v[sa], do[sa], 0.3)
    rb = _run(b, q[sb], k[sb], v[sb], do[sb], 0.3)
    for key in ("o", "dq", "dk", "dv"):
        assert _rel(rf[key][sa], ra[key]) < 1e-12
        assert _rel(rf[key][sb], rb[key]) < 1e-12


def test_gqa_equals_mha_with_repeated_kv():
    t, (q, k, v, do) = _tree_and_inputs(seed=10, hq=6, hkv=2)
    r = _run(t, q, k, v, do, 0.3)
    rm = _run(t, q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), do, 0.3)
    assert _rel(r["o"], rm["o"]) < 1e-12
    assert _rel(r["dq"], rm["dq"]) < 1e-12
    n, _, d = k.shape
    assert _rel(r["dk"], rm["dk"].reshape(n, 2, 3, d).sum(2)) < 1e-12
    assert _rel(r["dv"], rm["dv"].reshape(n, 2, 3, d).sum(2)) < 1e-12


def test_multiplicity_identity():
    """Giving every path copy the full dO_t equals the tree gradient for
    dO_t * mult(t): checks that the oracle splits dO across path copies."""
    t, (q, k, v, do) = _tree_and_inputs(seed=13, hq=2, hkv=1)
    paths = oracle.root_to_leaf_paths(t.parent, t.seg_start, t.seg_len)
    mult = oracle.path_multiplicity(paths, t.num_tokens)
    assert mult.max() > 1
    dq = np.zeros_like(q); dk = np.zeros_like(k); dv = np.zeros_like(v)
    for p in paths:
        for h in range(2):
            _, _, a, b, c = oracle.causal_attention(q[p, h], k[p, 0], v[p, 0], do[p, h], 0.3)
            dq[p, h] += a; dk[p, 0] += b; dv[p, 0] += c
    r = _run(t, q, k, v, do * mult[:, None, None], 0.3)
    assert _rel(r["dq"], dq) < 1e-12
    assert _rel(r["dk"], dk) < 1e-12
    assert _rel(r["dv"], dv) < 1e-12


def test_sampled_rows_match_full():
    t, (q, k, v, do) = _tree_and_inputs(seed=14, hq=4, hkv=2)
    r = _run(t, q, k, v, do, 0.3)
    rows = [0, 3, t.num_tokens // 2, t.num_tokens - 1]
    o, lse, dq = oracle.query_rows(q, k, v, do, t.parent, t.seg_start, t.seg_len, 0.3,
                                   rows, [0, 3])
    np.testing.assert_allclose(o, r["o"][rows][:, [0, 3]], atol=1e-12)
    np.testing.assert_allclose(lse, r["lse"][[0, 3]][:, rows], atol=1e-12)
    np.testing.assert_allclose(dq, r["dq"][rows][:, [0, 3]], atol=1e-12)
    # every token as a key, with row blocks much shorter than the paths
    keys = list(range(t.num_tokens))
    dk, dv = oracle.key_rows(q, k, v, do, t.parent, t.seg_start, t.seg_len, 0.3, keys, 1,
                             row_block=7)
    np.testing.assert_allclose(dk, r["dk"][keys, 1], atol=1e-12)
    np.testing.assert_allclose(dv, r["dv"][keys, 1], atol=1e-12)
    for kk in ([0], [t.num_tokens - 1], [3, t.num_tokens // 2]):
        dk, dv = oracle.key_rows(q, k, v, do, t.parent, t.seg_start, t.seg_len, 0.3, kk, 0,
                                 row_block=5)
        np.testing.assert_allclose(dk, r["dk"][kk, 0], atol=1e-12)
        np.testing.assert_allclose(dv, r["dv"][kk, 0], atol=1e-12)


def test_head_subset_and_row_blocking():
    t, (q, k, v, do) = _tree_and_inputs(seed=15, hq=4, hkv=2)
    full = _run(t, q, k, v, do, 0.3)
    part = _run(t, q, k, v, do, 0.3, kv_heads=[1], row_block=5)
    assert np.isnan(part["o"][:, 0]).all()
    for key in ("o", "dq"):
        assert _rel(part[key][:, 2:], full[key][:, 2:]) < 1e-12
    assert _rel(part["dk"][:, 1], full["dk"][:, 1]) < 1e-12


# ------------------------------------------------------- input generator

def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32)
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0]  # ties
    ours = bf16_round_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_workload_trees():
    s = {i: tree_stats(config_tree(i)) for i in (1, 2, 4, 5)}
    assert (s[1]["nodes"], s[1]["leaves"], s[1]["tokens"], s[1]["max_path"]) == (15, 8, 256, 80)
    assert (s[2]["nodes"], s[2]["leaves"], s[2]["tokens"], s[2]["max_path"]) == (17, 16, 33792, 3072)
    assert (s[4]["nodes"], s[4]["leaves"], s[4]["tokens"], s[4]["max_path"]) == (127, 64, 65024, 3584)
    assert s[5]["tokens"] == 163840 and 32768 < s[5]["max_path"] <= 32768 + 2048
    s3 = tree_stats(config_tree(3))
    assert 30720 <= s3["tokens"] <= 34816 and s3["max_path"] <= 16384
    # the oracle's own path list agrees with the generator's leaf count
    for i in (1, 2, 4):
        t = config_tree(i)
        assert len(oracle.root_to_leaf_paths(t.parent, t.seg_start, t.seg_len)) == s[i]["leaves"]


# ------------------------------------------------- key gradients by unique row

@pytest.mark.parametrize("seed,nodes,roots,hq,hkv,d,shuffle,block", [
    (21, 1, 1, 2, 1, 8, False, 1024), (22, 9, 1, 4, 2, 8, False, 3),
    (23, 15, 2, 6, 2, 4, True, 5), (24, 20, 3, 3, 3, 16, True, 1024),
    (25, 12, 1, 8, 1, 8, False, 2),
])
def test_key_rows_by_row_against_bruteforce(seed, nodes, roots, hq, hkv, d, shuffle, block):
    """The per-row arrangement of the key gradients against the dense
    closure-mask softmax differentiated by torch autograd, on every key of
    every kv head, with row blocks shorter than the segments and nodes
    packed in random order."""
    rng = np.random.default_rng(seed)
    t = random_tree(rng, nodes, max_len=14, n_roots=roots, shuffle=shuffle)
    q, k, v, do = _rand_qkvdo(rng, t.num_tokens, hq, hkv, d)
    scale = 1.0 / np.sqrt(d)
    b = brute_force(t, q, k, v, do, scale)
    keys = list(range(t.num_tokens))
    for g in range(hkv):
        dk, dv = oracle.key_rows_by_row(q, k, v, do, t.parent, t.seg_start, t.seg_len, scale,
                                        keys, g, row_block=block)
        assert _rel(dk, b["dk"][:, g]) < 1e-12
        assert _rel(dv, b["dv"][:, g]) < 1e-12
    # a subset of keys, repeated and out of order
    sub = [t.num_tokens - 1, 0, t.num_tokens // 2, 0]
    dk, dv = oracle.key_rows_by_row(q, k, v, do, t.parent, t.seg_start, t.seg_len, scale, sub,
                                    hkv - 1, row_block=block)
    np.testing.assert_allclose(dk, b["dk"][sub, hkv - 1], atol=1e-12)
    np.testing.assert_allclose(dv, b["dv"][sub, hkv - 1], atol=1e-12)


def test_key_rows_by_row_catches_planted_mistakes():
    """Plausible mistakes must fail the brute-force pin: a wrong scale, the
    per-copy dO / mult(t) carried into the per-row sums (each row is visited
    once, so it must carry its whole dO), and a dropped parent edge."""
    rng = np.random.default_rng(31)
    t = random_tree(rng, 7, max_len=9)
    q, k, v, do = _rand_qkvdo(rng, t.num_tokens, 2, 1, 8)
    b = brute_force(t, q, k, v, do, 0.4)
    keys = list(range(t.num_tokens))

    def run(tt, dd, scale):
        return oracle.key_rows_by_row(q, k, v, dd, tt.parent, tt.seg_start, tt.seg_len, scale,
                                      keys, 0)[0]
    assert _rel(run(t, do, 0.4), b["dk"][:, 0]) < 1e-12
    assert _rel(run(t, do, 0.4 * 1.01), b["dk"][:, 0]) > 1e-4
    mult = oracle.path_multiplicity(oracle.root_to_leaf_paths(t.parent, t.seg_start, t.seg_len),
                                    t.num_tokens)
    assert mult.max() > 1
    assert _rel(run(t, do / mult[:, None, None], 0.4), b["dk"][:, 0]) > 1e-4
    child = int(np.nonzero(t.parent >= 0)[0][0])
    t2 = t.copy()
    t2.parent[child] = -1
    assert _rel(run(t2, do, 0.4), b["dk"][:, 0]) > 1e-4
