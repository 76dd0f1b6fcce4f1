"""Pins for the fp64 linear-attention oracle, independent of its own code.

* brute force over all unique tokens: scale * (mask o Q K^T) V with the
  transitive-closure visibility mask of test_oracle, differentiated by torch
  fp64 autograd;
* the running-state recurrence S_t = S_{t-1} + k_t v_t^T, o_t = scale S_t^T q_t
  on chains (a different algorithm from the oracle's quadratic form),
  differentiated by torch autograd;
* central finite differences of the unique-token loss;
* a three-node tree with scalar heads solved by hand;
* homogeneity: O is linear in each of Q, K and V, so
  <dQ, Q> = <dK, K> = <dV, V> = sum_t <dO_t, O_t>;
* path consistency and the effect of the scale.
"""

import numpy as np
import pytest
import torch

import oracle
from tree_inputs import NodeTable, binary_tree, chain_tree, random_tree, star_tree
from test_oracle import visibility_mask


def _rand(rng, n, hq, hkv, d):
    return (rng.standard_normal((n, hq, d)), rng.standard_normal((n, hkv, d)),
            rng.standard_normal((n, hkv, d)), rng.standard_normal((n, hq, d)))


def _lin(t: NodeTable, q, k, v, do, scale):
    return oracle.tree_linear_attention(q, k, v, do, t.parent, t.seg_start, t.seg_len, scale)


def _brute(t: NodeTable, q, k, v, do, scale):
    mask = torch.from_numpy(visibility_mask(t)).to(torch.float64)
    hq, hkv = q.shape[1], k.shape[1]
    gs = hq // hkv
    Q = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    K = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    V = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    outs = []
    for h in range(hq):
        a = scale * (Q[:, h] @ K[:, h // gs].T) * mask
        outs.append(a @ V[:, h // gs])
    O = torch.stack(outs, 1)
    (O * torch.tensor(do)).sum().backward()
    return O.detach().numpy(), Q.grad.numpy(), K.grad.numpy(), V.grad.numpy()


def _recurrent(q, k, v, do, scale):
    """One sequence, [L, D] each: the state recurrence, torch autograd."""
    Q = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    K = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    V = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    S = torch.zeros(q.shape[1], v.shape[1], dtype=torch.float64)
    outs = []
    for i in range(q.shape[0]):
        S = S + torch.outer(K[i], V[i])
        outs.append(scale * (S.T @ Q[i]))
    O = torch.stack(outs)
    (O * torch.tensor(do)).sum().backward()
    return O.detach().numpy(), Q.grad.numpy(), K.grad.numpy(), V.grad.numpy()


def _close(a, b, tol=1e-10):
    scale = max(1.0, float(np.abs(b).max()))
    assert np.abs(a - b).max() <= tol * scale, float(np.abs(a - b).max())


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("hq,hkv", [(1, 1), (4, 2)])
def test_brute_force_random_forests(seed, hq, hkv):
    rng = np.random.default_rng(100 + seed)
    t = random_tree(rng, n_nodes=9, max_len=7, n_roots=1 + seed % 2)
    q, k, v, do = _rand(rng, t.num_tokens, hq, hkv, 8)
    r = _lin(t, q, k, v, do, 0.3)
    o, dq, dk, dv = _brute(t, q, k, v, do, 0.3)
    for name, ref in (("o", o), ("dq", dq), ("dk", dk), ("dv", dv)):
        _close(r[name], ref)
    assert r["path_spread"] < 1e-12


@pytest.mark.parametrize("lengths", [[13], [5, 1, 7], [1, 1, 1, 1]])
def test_chain_matches_state_recurrence(lengths):
    rng = np.random.default_rng(sum(lengths))
    t = chain_tree(lengths)
    q, k, v, do = _rand(rng, t.num_tokens, 1, 1, 6)
    r = _lin(t, q, k, v, do, 0.7)
    o, dq, dk, dv = _recurrent(q[:, 0], k[:, 0], v[:, 0], do[:, 0], 0.7)
    _close(r["o"][:, 0], o)
    _close(r["dq"][:, 0], dq)
    _close(r["dk"][:, 0], dk)
    _close(r["dv"][:, 0], dv)


def test_finite_differences():
    rng = np.random.default_rng(7)
    t = binary_tree(3, 2, 2)
    q, k, v, do = _rand(rng, t.num_tokens, 2, 1, 3)
    r = _lin(t, q, k, v, do, 0.5)

    def loss(q_, k_, v_):
        return float((_lin(t, q_, k_, v_, do, 0.5)["o"] * do).sum())

    eps = 1e-6
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        idx = [tuple(rng.integers(0, s) for s in x.shape) for _ in range(6)]
        for ix in idx:
            xp, xm = x.copy(), x.copy()
            xp[ix] += eps
            xm[ix] -= eps
            args_p = [xp if a is x else a for a in (q, k, v)]
            args_m = [xm if a is x else a for a in (q, k, v)]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(fd - r[name][ix]) < 1e-6 * max(1.0, abs(fd)), (name, ix)


def test_hand_solved_three_node_tree():
    # root token 0; children: node 1 = token 1, node 2 = token 2; D = 1
    t = NodeTable(parent=np.array([-1, 0, 0]), seg_start=np.array([0, 1, 2]),
                  seg_len=np.array([1, 1, 1]), num_tokens=3, name="y")
    qs, ks, vs, dos = [2.0, -1.0, 0.5], [1.5, 3.0, -2.0], [4.0, 0.25, 1.0], [1.0, 2.0, -3.0]
    c = 0.5
    q = np.array(qs).reshape(3, 1, 1)
    k = np.array(ks).reshape(3, 1, 1)
    v = np.array(vs).reshape(3, 1, 1)
    do = np.array(dos).reshape(3, 1, 1)
    r = _lin(t, q, k, v, do, c)
    # o_0 = c q0 k0 v0; o_i = c q_i (k0 v0 + k_i v_i) for the two leaves
    o = [c * 2.0 * 1.5 * 4.0,
         c * -1.0 * (1.5 * 4.0 + 3.0 * 0.25),
         c * 0.5 * (1.5 * 4.0 + -2.0 * 1.0)]
    assert np.allclose(r["o"].ravel(), o, rtol=0, atol=1e-14)
    # dq_i = c * do_i * (state of token i)
    dq = [c * 1.0 * 6.0, c * 2.0 * 6.75, c * -3.0 * 4.0]
    assert np.allclose(r["dq"].ravel(), dq, rtol=0, atol=1e-14)
    # token 0 is seen by all three tokens; a leaf only by itself
    dk0 = c * 4.0 * (2.0 * 1.0 + -1.0 * 2.0 + 0.5 * -3.0)
    dv0 = c * 1.5 * (2.0 * 1.0 + -1.0 * 2.0 + 0.5 * -3.0)
    dk = [dk0, c * 0.25 * -1.0 * 2.0, c * 1.0 * 0.5 * -3.0]
    dv = [dv0, c * 3.0 * -1.0 * 2.0, c * -2.0 * 0.5 * -3.0]
    assert np.allclose(r["dk"].ravel(), dk, rtol=0, atol=1e-14)
    assert np.allclose(r["dv"].ravel(), dv, rtol=0, atol=1e-14)
    assert list(r["mult"]) == [2, 1, 1]


@pytest.mark.parametrize("tree", ["star", "binary", "random"])
def test_homogeneity_identities(tree):
    rng = np.random.default_rng(11)
    t = {"star": star_tree(6, 3, 5), "binary": binary_tree(4, 3, 3),
         "random": random_tree(rng, n_nodes=12, max_len=6)}[tree]
    q, k, v, do = _rand(rng, t.num_tokens, 4, 2, 5)
    r = _lin(t, q, k, v, do, 0.4)
    total = float((r["o"] * do).sum())
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        assert abs(float((r[name] * x).sum()) - total) < 1e-9 * max(1.0, abs(total)), name


def test_scale_and_path_consistency():
    rng = np.random.default_rng(5)
    t = star_tree(7, 4, 6)
    q, k, v, do = _rand(rng, t.num_tokens, 2, 2, 4)
    r1 = _lin(t, q, k, v, do, 1.0)
    r2 = _lin(t, q, k, v, do, 0.25)
    _close(r2["o"], 0.25 * r1["o"])
    _close(r2["dv"], 0.25 * r1["dv"])
    assert r1["path_spread"] < 1e-12
    # the prompt's outputs equal those of the prompt alone
    p = _lin(chain_tree([7]), q[:7], k[:7], v[:7], do[:7], 1.0)
    _close(r1["o"][:7], p["o"])


@pytest.mark.parametrize("seed", [0, 1])
def test_sampled_rows_match_full_expansion(seed):
    rng = np.random.default_rng(40 + seed)
    t = random_tree(rng, n_nodes=10, max_len=9, n_roots=1 + seed)
    q, k, v, do = _rand(rng, t.num_tokens, 4, 2, 6)
    r = _lin(t, q, k, v, do, 0.3)
    rows = rng.choice(t.num_tokens, size=7, replace=False)
    o, dq = oracle.linear_query_rows(q, k, v, do, t.parent, t.seg_start, t.seg_len, 0.3,
                                     rows, [0, 3])
    _close(o, r["o"][rows][:, [0, 3]])
    _close(dq, r["dq"][rows][:, [0, 3]])
    for g in range(2):
        dk, dv = oracle.linear_key_rows(q, k, v, do, t.parent, t.seg_start, t.seg_len, 0.3,
                                        rows, g)
        _close(dk, r["dk"][rows, g])
        _close(dv, r["dv"][rows, g])


def test_kv_head_restriction():
    rng = np.random.default_rng(21)
    t = star_tree(5, 3, 4)
    q, k, v, do = _rand(rng, t.num_tokens, 4, 2, 3)
    full = _lin(t, q, k, v, do, 0.5)
    part = oracle.tree_linear_attention(q, k, v, do, t.parent, t.seg_start, t.seg_len, 0.5,
                                        kv_heads=[1])
    _close(part["o"][:, 2:], full["o"][:, 2:])
    _close(part["dk"][:, 1], full["dk"][:, 1])
    assert np.isnan(part["o"][:, :2]).all() and np.isnan(part["dv"][:, 0]).all()
