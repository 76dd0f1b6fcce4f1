"""GPU parity: the HIP library (through the C ABI) against the fp64 oracle.

Bar: relative L2 error <= 1e-2 on O, dQ, dK, dV and max |LSE error| <= 1e-3.
Small trees are compared element by element over whole tensors; they span
several tiles and ragged tails (segments that are not multiples of the 128
-row query tiles, 64-key forward steps or 128-key backward tiles).  The five
workload trees are run at full size in the launch configuration of the
benchmark and compared on sampled rows and keys that the oracle computes one
by one, plus closed-form properties over the whole tensors.
"""

import numpy as np
import pytest

import oracle
from tree_inputs import (NodeTable, binary_tree, caterpillar_tree, chain_tree, config_spec,
                         config_tree, random_tree, star_tree, trunk_tree)
from gpu_util import (FP32_LSE_ABS, FP32_REL_L2, LSE_ABS, REL_L2, cancel_scale, make, rel_l2,
                      run_library)

pytestmark = pytest.mark.gpu


def _compare_full(t: NodeTable, hq, hkv, d, dtype, scale=None, do_std=1e-2, seed_offset=0):
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    x = make(t, hq, hkv, d, dtype, do_std=do_std, seed_offset=seed_offset)
    print(f"case: N={t.num_tokens} nodes={t.num_nodes} hq={hq} hkv={hkv} d={d} {dtype}",
          flush=True)
    got = run_library(t, x, hq, hkv, d, dtype, scale)
    ref = oracle.tree_attention(x.q, x.k, x.v, x.do, t.parent, t.seg_start, t.seg_len, scale)
    zero = {"dk": cancel_scale(x.q, ref["o"], x.do, scale),
            "dq": cancel_scale(x.k, ref["o"], x.do, scale)}
    errs = {k: rel_l2(got[k], ref[k], zero.get(k, 0.0)) for k in ("o", "dq", "dk", "dv")}
    errs["lse"] = float(np.abs(got["lse"] - ref["lse"]).max())
    print("errors:", errs, flush=True)
    _per_node(t, got, ref)
    rel_bar, lse_bar = (FP32_REL_L2, FP32_LSE_ABS) if dtype == "fp32" else (REL_L2, LSE_ABS)
    for k in ("o", "dq", "dk", "dv"):
        assert errs[k] <= rel_bar, (k, errs)
    assert errs["lse"] <= lse_bar, errs
    return errs


def _per_node(t: NodeTable, got, ref):
    """Diagnostic only: the node with the largest relative L2 error of each
    output over that node's rows (a wrong ancestor list or branch sum shows
    up on one node long before it moves the whole-tensor error)."""
    worst = {}
    for k in ("o", "dq", "dk", "dv"):
        e_max, n_max = 0.0, -1
        for i in range(t.num_nodes):
            r0, r1 = int(t.seg_start[i]), int(t.seg_start[i] + t.seg_len[i])
            den = float(np.linalg.norm(ref[k][r0:r1]))
            if den == 0.0:
                continue
            e = float(np.linalg.norm(np.asarray(got[k][r0:r1], np.float64) - ref[k][r0:r1])) / den
            if e > e_max:
                e_max, n_max = e, i
        worst[k] = (n_max, round(e_max, 6))
    print("worst node per output (node, rel-L2):", worst, flush=True)


def _random(seed, nodes, max_len, roots=1):
    return random_tree(np.random.default_rng(seed), nodes, max_len=max_len, n_roots=roots)


CASES = {
    "single-token": (chain_tree([1]), 1, 1, 128, "bf16"),
    "chain-1000": (chain_tree([1000]), 2, 1, 128, "bf16"),
    "chain-ragged": (chain_tree([70, 1, 129, 64, 200]), 4, 2, 128, "bf16"),
    "star": (star_tree(300, 5, 257), 4, 2, 128, "bf16"),
    "binary-ragged": (binary_tree(129, 97, 3), 4, 2, 128, "bf16"),
    "random-a": (_random(1, 9, 300), 4, 2, 128, "bf16"),
    "random-b": (_random(2, 12, 200), 8, 1, 128, "bf16"),
    "forest": (_random(3, 10, 260, roots=3), 6, 2, 128, "bf16"),
    "gqa7": (_random(4, 7, 300), 7, 1, 128, "bf16"),
    "mha": (_random(5, 6, 250), 3, 3, 128, "bf16"),
    # groups wider than the workloads' (16 query heads on one kv head)
    "mqa16": (_random(9, 7, 260), 16, 1, 128, "bf16"),
    "gqa12-d64": (_random(10, 6, 200), 24, 2, 64, "bf16"),
    "d64-bf16": (_random(6, 9, 300), 4, 2, 64, "bf16"),
    "d64-fp32": (_random(7, 8, 200), 2, 1, 64, "fp32"),
    "d128-fp32": (_random(8, 6, 200), 2, 2, 128, "fp32"),
    # key tiles that cross node boundaries (key-limit entries) in the fp32 kernel
    "binary-fp32": (binary_tree(100, 70, 3), 2, 1, 128, "fp32"),
    "star-d64-fp32": (star_tree(200, 3, 150), 2, 1, 64, "fp32"),
    "heavy-prompt-split": (star_tree(1024, 16, 64), 4, 2, 128, "bf16"),
    # dozens of short trunk nodes per key tile, a key limit per leaf
    "caterpillar": (caterpillar_tree([1 + (7 * i) % 3 for i in range(150)], 5), 4, 2, 128,
                    "bf16"),
    "caterpillar-fp32": (caterpillar_tree([1 + (5 * i) % 4 for i in range(90)], 9), 2, 1, 64,
                         "fp32"),
    # few query tiles over long key paths: the planner cuts their keys into
    # parts (forward and dQ partial results merged after the launch); some
    # parts hold no key of some rows (causal ranges cut mid-way)
    "long-chain-key-parts": (chain_tree([3500, 300]), 4, 2, 128, "bf16"),
    "star-key-parts-fp32": (star_tree(3200, 3, 200), 2, 1, 64, "fp32"),
    "caterpillar-key-parts": (caterpillar_tree([1200, 1100, 1000, 900], 150), 4, 2, 128,
                              "bf16"),
}
KEY_PART_CASES = ("long-chain-key-parts", "star-key-parts-fp32", "caterpillar-key-parts")


@pytest.mark.parametrize("name", list(CASES))
def test_small_tree_elementwise(name):
    t, hq, hkv, d, dtype = CASES[name]
    _compare_full(t, hq, hkv, d, dtype, do_std=1.0 if dtype == "fp32" else 1e-2)


@pytest.mark.parametrize("seed", range(10))
def test_random_tree_sweep(seed):
    """Seeded random forests, packed depth first (parent-child runs, key
    tiles that cross node boundaries, key-limit entries) or in a random
    order, with random head counts, head dims and both dtypes."""
    import prefix_shared_tree_attn_amd as ta
    rng = np.random.default_rng(1000 + seed)
    t = random_tree(rng, int(rng.integers(2, 25)), max_len=int(rng.choice([40, 150, 300])),
                    n_roots=int(rng.integers(1, 3)), shuffle=seed % 2 == 1)
    hkv = int(rng.choice([1, 2]))
    hq = hkv * int(rng.choice([1, 2, 4]))
    d = int(rng.choice([64, 128]))
    dtype = "fp32" if seed % 5 == 4 else "bf16"
    ex = ta.plan_host(t.parent, t.seg_start, t.seg_len, t.num_tokens, hq, hkv, d, dtype).export()
    print(f"sweep seed {seed}: key-limit entries {int((ex['bwd_entries'][:, 3] < 0).sum())}",
          flush=True)
    _compare_full(t, hq, hkv, d, dtype, do_std=1.0 if dtype == "fp32" else 1e-2)


@pytest.mark.parametrize("seed", range(40))
def test_random_tree_sweep_wide(seed):
    """Forty more seeded trees: random forests of 1-39 nodes with segments up
    to 400 tokens (a third packed in random order) and, every eighth seed, a
    caterpillar; 1, 2 or 4 kv heads with groups of 1-8; both dtypes."""
    rng = np.random.default_rng(5000 + seed)
    if seed % 8 == 7:
        t = caterpillar_tree([int(x) for x in rng.integers(1, 40, int(rng.integers(5, 60)))],
                             int(rng.integers(1, 200)))
    else:
        t = random_tree(rng, int(rng.integers(1, 40)), max_len=int(rng.choice([20, 130, 400])),
                        min_len=1, n_roots=int(rng.integers(1, 4)), shuffle=bool(seed % 3 == 0))
    hkv = int(rng.choice([1, 2, 4]))
    hq = hkv * int(rng.choice([1, 2, 3, 8]))
    d = int(rng.choice([64, 128]))
    dtype = "fp32" if seed % 6 == 5 else "bf16"
    _compare_full(t, hq, hkv, d, dtype, do_std=1.0 if dtype == "fp32" else 1e-2)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_scores_growing_past_the_rescale_bound(dtype):
    """Keys scaled by 1, 12 and 25 in the first three 64-key blocks: the best
    base-2 score of a row grows by more than 64 from block 0 to block 1 and
    passes 128 in block 2 (2^128 overflows fp32), so those forward key
    blocks take the path that finds the row max and rescales O and l."""
    t = chain_tree([640])
    hq, hkv, d = 2, 1, 128
    scale = 1.0 / np.sqrt(d)
    x = make(t, hq, hkv, d, dtype)
    f = np.minimum(1.0 + 12.0 * (np.arange(t.num_tokens) // 64), 25.0).astype(np.float32)
    k = x.k * f[:, None, None]
    if dtype == "bf16":
        from tree_inputs.tensors import bf16_bits_to_f32, bf16_round_bits
        bits = bf16_round_bits(k)
        k = bf16_bits_to_f32(bits)
        x.bits["k"] = bits
    x.k[...] = k
    # the largest base-2 score per 64-key block, to show the jumps are there
    s = np.einsum("thd,jd->thj", x.q[:, :, :].astype(np.float64), x.k[:, 0, :].astype(np.float64))
    blocks = [float(np.abs(s[:, :, b:b + 64]).max()) * scale / np.log(2.0) for b in (0, 64, 128)]
    assert blocks[1] - blocks[0] > 64 and blocks[2] > 128, blocks
    print("largest base-2 score of blocks 0, 1, 2:", blocks, flush=True)
    got = run_library(t, x, hq, hkv, d, dtype, scale)
    ref = oracle.tree_attention(x.q, x.k, x.v, x.do, t.parent, t.seg_start, t.seg_len, scale)
    # The backward recomputes P = 2^(c s - LSE log2 e), a difference of two
    # numbers as large as the largest base-2 score M; fp32 rounds it to about
    # M 2^-24, so fp32 results carry relative errors of that order here (the
    # bf16 bar is far above it).
    big = float(np.abs(s).max()) * scale / np.log(2.0)
    rel_bar, lse_bar = ((max(FP32_REL_L2, 4.0 * big * 2.0 ** -24), FP32_LSE_ABS)
                        if dtype == "fp32" else (REL_L2, LSE_ABS))
    errs = {k_: rel_l2(got[k_], ref[k_]) for k_ in ("o", "dq", "dk", "dv")}
    # LSE reaches about 125 here, where fp32 values lie 7.6e-6 apart: its
    # error is taken relative to max(1, |LSE|)
    errs["lse"] = float(np.abs(got["lse"] - ref["lse"]).max() / max(1.0, np.abs(ref["lse"]).max()))
    print("errors:", errs, flush=True)
    for k_ in ("o", "dq", "dk", "dv"):
        assert errs[k_] <= rel_bar, (k_, errs)
    assert errs["lse"] <= lse_bar, errs


def test_split_case_really_splits():
    import prefix_shared_tree_attn_amd as ta
    t, hq, hkv, d, dtype = CASES["heavy-prompt-split"]
    p = ta.plan(t.parent, t.seg_start, t.seg_len, t.num_tokens, hq, hkv, d, dtype)
    assert p.stats()["bwd_split_tiles"] > 0
    for name in KEY_PART_CASES:
        t, hq, hkv, d, dtype = CASES[name]
        p = ta.plan(t.parent, t.seg_start, t.seg_len, t.num_tokens, hq, hkv, d, dtype)
        assert p.stats()["fwd_split_tiles"] > 0, name


def test_config1_full():
    t = config_tree(1)
    sp = config_spec(1)
    errs = _compare_full(t, sp["heads_q"], sp["heads_kv"], sp["head_dim"], sp["dtype"],
                         scale=sp["scale"], do_std=sp["do_std"])
    # fp32 inputs are computed in fp32 (held to FP32_REL_L2 in _compare_full)
    assert errs["lse"] < FP32_LSE_ABS and errs["o"] < FP32_REL_L2


def test_scaled_down_workloads():
    """Smaller trees of the same shapes as the benchmark workloads."""
    _compare_full(star_tree(512, 8, 640), 8, 2, 128, "bf16")
    _compare_full(binary_tree(96, 96, 5), 7, 1, 128, "bf16")
    _compare_full(trunk_tree(seed=1, trunk=3000, n_branches=8, branch_len=200), 8, 1, 128,
                  "bf16")


def test_empty_tree_is_a_no_op():
    import torch
    import prefix_shared_tree_attn_amd as ta
    p = ta.plan([], [], [], 0, 2, 1, 128)
    z = torch.empty((0, 2, 128), dtype=torch.bfloat16, device="cuda")
    zk = torch.empty((0, 1, 128), dtype=torch.bfloat16, device="cuda")
    o, lse = ta.fwd(p, z, zk, zk, 0.1)
    dq, dk, dv = ta.bwd(p, z, zk, zk, o, lse, z, 0.1)
    node_id, pos_id = ta.positions(p)
    torch.cuda.synchronize()
    assert o.shape == (0, 2, 128) and dk.shape == (0, 1, 128)
    assert node_id.shape == (0,) and pos_id.shape == (0,)


def test_repeat_runs_are_deterministic_where_promised():
    import torch
    import prefix_shared_tree_attn_amd as ta
    from gpu_util import device_inputs
    t = star_tree(1024, 16, 64)
    x = make(t, 4, 2, 128, "bf16")
    dev = device_inputs(x, "bf16")
    p = ta.plan(t.parent, t.seg_start, t.seg_len, t.num_tokens, 4, 2, 128)
    runs = []
    for _ in range(2):
        o, lse = ta.fwd(p, dev["q"], dev["k"], dev["v"], 0.088)
        dq, dk, dv = ta.bwd(p, dev["q"], dev["k"], dev["v"], o, lse, dev["do"], 0.088)
        torch.cuda.synchronize()
        runs.append([a.clone() for a in (o, lse, dq, dk, dv)])
    for i in range(5):  # o, lse, dq, dk, dv: no atomics, bitwise reproducible
        assert torch.equal(runs[0][i], runs[1][i]), i


# ------------------------------------------------------------------ full size

def _sample_keys(t: NodeTable, rng, cfg: int):
    """Key rows whose descendant work the oracle can afford: tokens of leaf
    nodes, of the smallest inner subtree, and for the star tree the first
    token of the prompt."""
    m = t.num_nodes
    has_child = np.zeros(m, bool)
    for i in range(m):
        if t.parent[i] >= 0:
            has_child[t.parent[i]] = True
    leaves = np.nonzero(~has_child)[0]
    keys = []
    for leaf in rng.choice(leaves, size=min(3, len(leaves)), replace=False):
        s, l = int(t.seg_start[leaf]), int(t.seg_len[leaf])
        keys += [s, s + l // 2, s + l - 1]
    inner = np.nonzero(has_child)[0]
    if len(inner):
        # the inner node with the fewest descendant tokens
        sizes = []
        for i in inner:
            stack, tot = [int(i)], 0
            while stack:
                n = stack.pop()
                tot += int(t.seg_len[n])
                stack += [c for c in range(m) if t.parent[c] == n]
            sizes.append(tot)
        i = int(inner[int(np.argmin(sizes))])
        keys += [int(t.seg_start[i] + t.seg_len[i] - 1)]
    if cfg == 2:  # the prompt's first token: every row of every path sees it
        keys.append(int(t.seg_start[np.nonzero(t.parent < 0)[0][0]]))
    return sorted(set(keys))


def _closed_forms(got, dev, hq, hkv):
    """Closed forms over whole tensors, in fp64 on the device: every softmax
    row sums to one and is shift invariant, so per kv group sum dV = sum dO
    over the group's heads and sum dK = 0; scores depend on q.k only, so
    <dQ, Q> = <dK, K>."""
    import torch
    gs = hq // hkv
    for gg in range(hkv):
        want = dev["do"][:, gg * gs:(gg + 1) * gs].double().sum((0, 1))
        have = got["dv"][:, gg].double().sum(0)
        assert float((have - want).norm() / want.norm()) <= REL_L2
        dkg = got["dk"][:, gg].double()
        assert float(dkg.sum(0).norm()) <= 1e-2 * float(dkg.norm())
    # <dQ, Q> = <dK, K> cancels heavily; each bf16 output element carries a
    # rounding error of up to 2^-9 relative, so the two sums may differ by a
    # few standard deviations u / sqrt(3) * ||x * y||_2 of that noise
    lhs = rhs = n_l = n_r = 0.0
    for h in range(hq):
        pr = got["dq"][:, h].double() * dev["q"][:, h].double()
        lhs += float(pr.sum())
        n_l += float((pr * pr).sum())
    for g_ in range(hkv):
        pr = got["dk"][:, g_].double() * dev["k"][:, g_].double()
        rhs += float(pr.sum())
        n_r += float((pr * pr).sum())
    noise = (2.0 ** -9 / np.sqrt(3.0)) * np.sqrt(n_l + n_r)
    print(f"<dQ,Q>={lhs:.6e} <dK,K>={rhs:.6e} rounding-noise std={noise:.3e}", flush=True)
    assert abs(lhs - rhs) <= 6.0 * noise + 1e-2 * max(abs(lhs), abs(rhs))
    for name in ("o", "dq", "dk", "dv", "lse"):
        assert bool(torch.isfinite(got[name]).all()), name


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_full_size_sampled(cfg):
    import torch
    from gpu_util import run_library_device
    t = config_tree(cfg)
    sp = config_spec(cfg)
    hq, hkv, d, dtype, scale = sp["heads_q"], sp["heads_kv"], sp["head_dim"], sp["dtype"], sp["scale"]
    print(f"config {cfg}: N={t.num_tokens} nodes={t.num_nodes}", flush=True)
    x = make(t, hq, hkv, d, dtype, do_std=sp["do_std"])
    print("inputs ready", flush=True)
    got, dev = run_library_device(t, x, hq, hkv, d, dtype, scale)
    print("library done", flush=True)
    rng = np.random.default_rng(100 + cfg)
    rows = sorted(set([0, t.num_tokens - 1] + [int(r) for r in rng.integers(0, t.num_tokens, 14)]))
    heads = sorted(set(int(h) for h in rng.integers(0, hq, 3)))
    g = int(heads[0]) // (hq // hkv)
    keys = _sample_keys(t, rng, cfg)
    ri = torch.tensor(rows, device="cuda")
    hi = torch.tensor(heads, device="cuda")
    ki = torch.tensor(keys, device="cuda")
    g_o = got["o"][ri][:, hi].double().cpu().numpy()
    g_dq = got["dq"][ri][:, hi].double().cpu().numpy()
    g_lse = got["lse"][hi][:, ri].double().cpu().numpy()
    g_dk = got["dk"][ki, g].double().cpu().numpy()
    g_dv = got["dv"][ki, g].double().cpu().numpy()
    o, lse, dq = oracle.query_rows(x.q, x.k, x.v, x.do, t.parent, t.seg_start, t.seg_len,
                                   scale, rows, heads)
    print("oracle rows done", flush=True)
    dk, dv = oracle.key_rows(x.q, x.k, x.v, x.do, t.parent, t.seg_start, t.seg_len, scale,
                             keys, g)
    print("oracle keys done", flush=True)
    e_o, e_dq, e_dk, e_dv = rel_l2(g_o, o), rel_l2(g_dq, dq), rel_l2(g_dk, dk), rel_l2(g_dv, dv)
    e_lse = float(np.abs(g_lse - lse).max())
    print(f"sampled errors: o={e_o:.2e} lse={e_lse:.2e} dq={e_dq:.2e} dk={e_dk:.2e} "
          f"dv={e_dv:.2e}", flush=True)
    assert max(e_o, e_dq, e_dk, e_dv) <= REL_L2
    assert e_lse <= LSE_ABS
    _closed_forms(got, dev, hq, hkv)
    _check_split_tiles(cfg, t, x, got)


def test_deep_chain_sampled():
    """One 98,304-token chain (2 query heads on one kv head, D 128, bf16):
    its last rows attend to 2.8 times as many keys as the deepest row of the
    workload trees (1,536 key steps for a query tile, the online softmax
    carried across all of them), and most of its key tiles split into
    partial slots.  Sampled rows, the last included, and keys of the last
    1,024 positions against the oracle; whole-tensor closed forms for the
    rest."""
    import torch
    from gpu_util import run_library_device
    n, hq, hkv, d = 98304, 2, 1, 128
    scale = 1.0 / np.sqrt(d)
    t = chain_tree([n])
    x = make(t, hq, hkv, d, "bf16")
    print(f"deep chain: N={n} hq={hq} hkv={hkv} d={d}", flush=True)
    got, dev = run_library_device(t, x, hq, hkv, d, "bf16", scale)
    print("library done", flush=True)
    rng = np.random.default_rng(11)
    rows = sorted(set([0, 1, 4095, n - 1] + [int(r) for r in rng.integers(0, n, 8)]))
    heads = [0, 1]
    keys = [n - 1024, n - 700, n - 129, n - 128, n - 2, n - 1]
    ri, hi, ki = (torch.tensor(a, device="cuda") for a in (rows, heads, keys))
    o, lse, dq = oracle.query_rows(x.q, x.k, x.v, x.do, t.parent, t.seg_start, t.seg_len,
                                   scale, rows, heads)
    print("oracle rows done", flush=True)
    dk, dv = oracle.key_rows(x.q, x.k, x.v, x.do, t.parent, t.seg_start, t.seg_len, scale,
                             keys, 0, row_block=256)
    print("oracle keys done", flush=True)
    errs = {"o": rel_l2(got["o"][ri][:, hi].double().cpu().numpy(), o),
            "dq": rel_l2(got["dq"][ri][:, hi].double().cpu().numpy(), dq),
            "dk": rel_l2(got["dk"][ki, 0].double().cpu().numpy(), dk),
            "dv": rel_l2(got["dv"][ki, 0].double().cpu().numpy(), dv),
            "lse": float(np.abs(got["lse"][hi][:, ri].double().cpu().numpy() - lse).max())}
    print("sampled errors:", errs, flush=True)
    for k in ("o", "dq", "dk", "dv"):
        assert errs[k] <= REL_L2, (k, errs)
    assert errs["lse"] <= LSE_ABS
    _closed_forms(got, dev, hq, hkv)


def _split_slots(t: NodeTable, sp, key: int, g: int):
    """Number of partial slots of the backward items that hold `key` for kv
    head g (0 when its key tile is not split)."""
    import prefix_shared_tree_attn_amd as ta
    ex = ta.plan_host(t.parent, t.seg_start, t.seg_len, t.num_tokens, sp["heads_q"],
                      sp["heads_kv"], sp["head_dim"], sp["dtype"]).export()
    it = ex["bwd_items"]
    hit = it[(it[:, 0] <= key) & (key < it[:, 1]) & (it[:, 2] == g) & (it[:, 4] > it[:, 3])]
    return int((hit[:, 5] >= 0).sum())


def _check_split_tiles(cfg: int, t: NodeTable, x, got):
    """dK / dV of keys in heavily shared key tiles whose gradient the library
    sums from several partial slots (the tile's query rows are split for load
    balance), in the first and the last kv head, element-wise against the
    fp64 oracle: live on the GRPO star (its 1024-token prompt), and on the
    agent, segment-search and long-trunk trees against values the oracle
    wrote beforehand (tests/golden/make_split_tile_golden.py), checked to
    come from these very inputs."""
    import json
    import os
    sp = config_spec(cfg)
    hkv = sp["heads_kv"]
    if cfg == 2:
        keys, heads = [0, 511, 1023], [0, hkv - 1]
        want = {}
        for g in heads:
            want[g] = oracle.key_rows_by_row(x.q, x.k, x.v, x.do, t.parent, t.seg_start,
                                             t.seg_len, sp["scale"], keys, g)
    else:
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "make_split_tile_golden",
            os.path.join(os.path.dirname(__file__), "golden", "make_split_tile_golden.py"))
        msg = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(msg)
        with open(msg.golden_path(cfg)) as f:
            rec = json.load(f)
        assert rec["input_fingerprint"] == msg.input_fingerprint(x), "golden from other inputs"
        keys, heads = rec["keys"], rec["kv_heads"]
        want = {g: (np.asarray(rec["dk"][str(g)]), np.asarray(rec["dv"][str(g)]))
                for g in heads}
    for g in heads:
        for kk in keys:
            n_slots = _split_slots(t, sp, kk, g)
            print(f"config {cfg} key {kk} kv head {g}: {n_slots} partial slots", flush=True)
            assert n_slots >= 2, "the sampled key's tile is not split in this plan"
        import torch
        ki = torch.tensor(keys, device="cuda")
        g_dk = got["dk"][ki, g].double().cpu().numpy()
        g_dv = got["dv"][ki, g].double().cpu().numpy()
        dk, dv = want[g]
        for i, kk in enumerate(keys):
            e_k, e_v = rel_l2(g_dk[i], dk[i]), rel_l2(g_dv[i], dv[i])
            print(f"  key {kk}: dk rel-L2 {e_k:.2e}, dv rel-L2 {e_v:.2e}", flush=True)
            assert e_k <= REL_L2 and e_v <= REL_L2


def _position_trees():
    out = [(name, case[0]) for name, case in CASES.items()]
    out += [(f"config{i}", config_tree(i)) for i in (1, 2, 3, 4, 5)]
    out.append(("shuffled", random_tree(np.random.default_rng(11), 13, max_len=90, n_roots=2,
                                        shuffle=True)))
    return out


def test_positions_bit_exact():
    """tree_attn_positions against the oracle's path walk, integer-exact."""
    import torch
    import prefix_shared_tree_attn_amd as ta
    for name, t in _position_trees():
        print(f"positions case {name}: N={t.num_tokens} nodes={t.num_nodes}", flush=True)
        p = ta.plan(t.parent, t.seg_start, t.seg_len, t.num_tokens, 2, 1, 128)
        node_id, pos_id = ta.positions(p)
        torch.cuda.synchronize()
        ref_node, ref_pos = oracle.token_positions(t.parent, t.seg_start, t.seg_len, t.num_tokens)
        np.testing.assert_array_equal(node_id.cpu().numpy(), ref_node)
        np.testing.assert_array_equal(pos_id.cpu().numpy(), ref_pos)
        p.close()


@pytest.mark.parametrize("name,dtype", [("heavy-prompt-split", "bf16"), ("caterpillar", "bf16"),
                                        ("binary-fp32", "fp32"),
                                        ("long-chain-key-parts", "bf16")])
def test_outputs_and_workspace_stay_inside_their_buffers(name, dtype):
    """Canary margins: O, LSE, dQ, dK, dV and the backward workspace are
    views into larger buffers whose margins (64 KiB before and after) hold
    a fixed byte pattern; after the forward and backward passes the margins
    are unchanged and the results still match the oracle."""
    import torch
    import prefix_shared_tree_attn_amd as ta
    from gpu_util import device_inputs
    t, hq, hkv, d, _ = CASES[name]
    x = make(t, hq, hkv, d, dtype, do_std=1.0 if dtype == "fp32" else 1e-2)
    dev = device_inputs(x, dtype)
    n = t.num_tokens
    tdt = dev["q"].dtype
    esz = dev["q"].element_size()
    MARGIN = 64 * 1024  # bytes, a multiple of 256 so the views keep their alignment
    PATTERN = 0xA5

    def fenced(nbytes):
        buf = torch.full((MARGIN + nbytes + MARGIN,), PATTERN, dtype=torch.uint8, device="cuda")
        return buf, buf[MARGIN:MARGIN + nbytes]

    def view(inner, shape, dt):
        return inner.view(dt).view(shape)

    bufs = {}
    shapes = {"o": ((n, hq, d), tdt, esz), "lse": ((hq, n), torch.float32, 4),
              "dq": ((n, hq, d), tdt, esz), "dk": ((n, hkv, d), tdt, esz),
              "dv": ((n, hkv, d), tdt, esz)}
    outs = {}
    for key, (shape, dt, es) in shapes.items():
        buf, inner = fenced(int(np.prod(shape)) * es)
        bufs[key] = buf
        outs[key] = view(inner, shape, dt)
    p = ta.plan(t.parent, t.seg_start, t.seg_len, n, hq, hkv, d, dtype)
    wsf, wsz = p.workspace_size()
    bufs["ws"], ws = fenced(wsz)
    bufs["ws_fwd"], ws_f = fenced(max(wsf, 256))
    scale = 1.0 / np.sqrt(d)
    ta.fwd(p, dev["q"], dev["k"], dev["v"], scale, o=outs["o"], lse=outs["lse"], ws=ws_f)
    ta.bwd(p, dev["q"], dev["k"], dev["v"], outs["o"], outs["lse"], dev["do"], scale,
           dq=outs["dq"], dk=outs["dk"], dv=outs["dv"], ws=ws)
    torch.cuda.synchronize()
    for key, buf in bufs.items():
        head, tail = buf[:MARGIN], buf[-MARGIN:]
        assert bool((head == PATTERN).all()) and bool((tail == PATTERN).all()), key
    ref = oracle.tree_attention(x.q, x.k, x.v, x.do, t.parent, t.seg_start, t.seg_len, scale)
    for key in ("o", "dq", "dk", "dv"):
        got = outs[key].float().cpu().numpy().astype(np.float64)
        assert rel_l2(got, ref[key]) <= REL_L2, key
    p.close()
