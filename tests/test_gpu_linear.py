"""GPU parity of chunkwise linear attention over the tree (C ABI against the
fp64 oracle of oracle/linear_attention.py).

Bar: relative L2 error <= 1e-2 on O, dQ, dK, dV (bf16 inputs; the kernels
round the attention block and the fp32 states to bf16 as matrix-core
operands, a relative error near 2^-9).  Small trees are compared over whole
tensors; they span several 64-token chunks, chunk boundaries inside nodes,
branch points inside a chunk, ragged tails, forests and GQA groups.  The
workload trees run at full size in the benchmark's launch configuration and
are compared on rows and keys the oracle computes one by one.
"""

import numpy as np
import pytest

import oracle
from tree_inputs import (NodeTable, binary_tree, caterpillar_tree, chain_tree, config_spec,
                         config_tree, random_tree, star_tree)
from gpu_util import REL_L2, device_inputs, make, rel_l2

pytestmark = pytest.mark.gpu


def _run(t: NodeTable, x, hq, hkv, d, scale):
    import torch
    import prefix_shared_tree_attn_amd as ta
    dev = device_inputs(x, "bf16")
    p = ta.plan(t.parent, t.seg_start, t.seg_len, t.num_tokens, hq, hkv, d, "bf16")
    o = ta.lin_fwd(p, dev["q"], dev["k"], dev["v"], scale)
    dq, dk, dv = ta.lin_bwd(p, dev["q"], dev["k"], dev["v"], dev["do"], scale)
    torch.cuda.synchronize()
    p.close()
    return {k: val.float().cpu().numpy().astype(np.float64)
            for k, val in (("o", o), ("dq", dq), ("dk", dk), ("dv", dv))}


def _random(seed, nodes, max_len, roots=1):
    return random_tree(np.random.default_rng(seed), nodes, max_len=max_len, n_roots=roots)


CASES = {
    "single-token": (chain_tree([1]), 1, 1, 128),
    "chain-1000": (chain_tree([1000]), 2, 1, 128),
    "chain-ragged": (chain_tree([70, 1, 129, 64, 200]), 4, 2, 128),
    "star": (star_tree(100, 5, 70), 4, 2, 128),
    "binary-small-segments": (binary_tree(32, 16, 3), 2, 1, 64),
    "random": (_random(1, 12, 200), 4, 2, 128),
    "forest": (_random(3, 10, 160, roots=3), 6, 2, 128),
    "gqa8-d64": (_random(4, 9, 150), 8, 1, 64),
    "mha": (_random(5, 6, 150), 3, 3, 128),
    "star-1024": (star_tree(1024, 6, 300), 4, 1, 128),
}



@pytest.mark.parametrize("seed", range(12))
def test_linear_random_sweep(seed):
    """Seeded random forests and caterpillars (many nodes shorter than a
    64-token chunk, so most pieces start at branch points), depth-first or
    random packing, GQA groups of 1-8, D 64/128."""
    rng = np.random.default_rng(7000 + seed)
    if seed % 4 == 3:
        t = caterpillar_tree([int(x) for x in rng.integers(1, 30, int(rng.integers(5, 50)))],
                             int(rng.integers(1, 90)))
    else:
        t = random_tree(rng, int(rng.integers(1, 30)), max_len=int(rng.choice([10, 70, 250])),
                        n_roots=int(rng.integers(1, 3)), shuffle=bool(seed % 3 == 0))
    hkv = int(rng.choice([1, 2]))
    hq = hkv * int(rng.choice([1, 2, 8]))
    d = int(rng.choice([64, 128]))
    scale = 1.0 / np.sqrt(d)
    x = make(t, hq, hkv, d, "bf16")
    print(f"linear sweep seed {seed}: N={t.num_tokens} nodes={t.num_nodes} hq={hq} hkv={hkv} "
          f"d={d}", flush=True)
    got = _run(t, x, hq, hkv, d, scale)
    ref = oracle.tree_linear_attention(x.q, x.k, x.v, x.do, t.parent, t.seg_start, t.seg_len,
                                       scale)
    errs = {k: rel_l2(got[k], ref[k]) for k in ("o", "dq", "dk", "dv")}
    print("errors:", errs, flush=True)
    for k, v in errs.items():
        assert v <= REL_L2, (k, errs)

@pytest.mark.parametrize("name", list(CASES))
def test_linear_parity(name):
    t, hq, hkv, d = CASES[name]
    scale = 1.0 / np.sqrt(d)
    x = make(t, hq, hkv, d, "bf16")
    print(f"case {name}: N={t.num_tokens} nodes={t.num_nodes} hq={hq} hkv={hkv} d={d}",
          flush=True)
    got = _run(t, x, hq, hkv, d, scale)
    ref = oracle.tree_linear_attention(x.q, x.k, x.v, x.do, t.parent, t.seg_start,
                                       t.seg_len, scale)
    errs = {k: rel_l2(got[k], ref[k]) for k in ("o", "dq", "dk", "dv")}
    print("errors:", errs, flush=True)
    for k, e in errs.items():
        assert e <= REL_L2, (k, errs)


def test_linear_repeatable_and_workspace_reuse():
    """Two calls with one workspace give bit-identical results (no state
    survives between calls)."""
    import torch
    import prefix_shared_tree_attn_amd as ta
    t = _random(9, 10, 200)
    x = make(t, 4, 2, 128, "bf16")
    dev = device_inputs(x, "bf16")
    p = ta.plan(t.parent, t.seg_start, t.seg_len, t.num_tokens, 4, 2, 128, "bf16")
    ws = ta.lin_workspace(p, "bwd")
    o1 = ta.lin_fwd(p, dev["q"], dev["k"], dev["v"], 0.1, ws=ws).clone()
    g1 = [g.clone() for g in ta.lin_bwd(p, dev["q"], dev["k"], dev["v"], dev["do"], 0.1, ws=ws)]
    o2 = ta.lin_fwd(p, dev["q"], dev["k"], dev["v"], 0.1, ws=ws)
    g2 = ta.lin_bwd(p, dev["q"], dev["k"], dev["v"], dev["do"], 0.1, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
    p.close()


def test_linear_rejects_fp32_and_short_workspace():
    import torch
    import prefix_shared_tree_attn_amd as ta
    t = star_tree(10, 2, 5)
    p = ta.plan(t.parent, t.seg_start, t.seg_len, t.num_tokens, 2, 1, 64, "fp32")
    z = torch.zeros((t.num_tokens, 2, 64), device="cuda")
    zk = torch.zeros((t.num_tokens, 1, 64), device="cuda")
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    with pytest.raises(ta.TreeAttnError, match="UNSUPPORTED"):
        ta.lin_fwd(p, z, zk, zk, 1.0, ws=ws)
    p.close()
    p = ta.plan(t.parent, t.seg_start, t.seg_len, t.num_tokens, 2, 1, 64, "bf16")
    zb, zkb = z.bfloat16(), zk.bfloat16()
    with pytest.raises(ta.TreeAttnError, match="WORKSPACE"):
        ta.lin_fwd(p, zb, zkb, zkb, 1.0, ws=ws[:256])
    p.close()


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_linear_full_size_sampled(cfg):
    t = config_tree(cfg)
    sp = config_spec(cfg)
    hq, hkv, d = sp["heads_q"], sp["heads_kv"], sp["head_dim"]
    scale = sp["scale"]
    x = make(t, hq, hkv, d, "bf16")
    print(f"config {cfg}: N={t.num_tokens} nodes={t.num_nodes} hq={hq} hkv={hkv}", flush=True)
    got = _run(t, x, hq, hkv, d, scale)
    rng = np.random.default_rng(cfg)
    rows = np.sort(rng.choice(t.num_tokens, size=16, replace=False))
    # the first and last tokens of the tree, and one at a chunk boundary
    rows = np.unique(np.concatenate([rows, [0, 63, 64, t.num_tokens - 1]]))
    heads = [0, hq - 1]
    o, dq = oracle.linear_query_rows(x.q, x.k, x.v, x.do, t.parent, t.seg_start, t.seg_len,
                                     scale, rows, heads)
    errs = {"o": rel_l2(got["o"][rows][:, heads], o),
            "dq": rel_l2(got["dq"][rows][:, heads], dq)}
    # the long trunk's keys are seen by 64 paths of ~35K tokens: fewer there
    keys = rows if cfg != 5 else rows[::3]
    for g in ((0, hkv - 1) if cfg != 5 else (hkv - 1,)):
        dk, dv = oracle.linear_key_rows(x.q, x.k, x.v, x.do, t.parent, t.seg_start, t.seg_len,
                                        scale, keys, g)
        errs[f"dk{g}"] = rel_l2(got["dk"][keys, g], dk)
        errs[f"dv{g}"] = rel_l2(got["dv"][keys, g], dv)
    print("errors:", errs, flush=True)
    for k, e in errs.items():
        assert e <= REL_L2, (k, errs)
