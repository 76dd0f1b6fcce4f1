"""GPU parity of the depth-first schedule: query-subset plans, the
accumulating backward and the final cast, through the C ABI.

A depth-first walk (AReaL-DTA, abstract: one root-to-leaf path resident at a
time, each shared prefix computed once) runs forward calls in preorder and
accumulating backward calls in reverse order, one node per call or one run
of preorder nodes per call (tree_attn_walk_runs).  Summed over the walk,
the results must be the whole tree's: checked against the fp64 oracle
(whole tensors on small trees, sampled rows and keys on the GRPO-star,
agent and segment-search workloads at full size) and against the one-call
library path, to rounding: a walk's call has few query tiles, so the
planner cuts their keys into parts that run side by side and merges the
parts' partial results, where the whole-tree pass may not (another
summation order, then one rounding).  One call on a
random set of nodes is checked against ``oracle.tree_attention_subset``.
Bar: relative L2 <= 1e-2 on O, dQ, dK, dV and max |LSE error| <= 1e-3.
"""

import numpy as np
import pytest

import oracle
from tree_inputs import binary_tree, config_spec, config_tree, dfs_preorder, random_tree, star_tree
from gpu_util import FP32_LSE_ABS, FP32_REL_L2, LSE_ABS, REL_L2, device_inputs, make, rel_l2

pytestmark = pytest.mark.gpu


def _walk(t, dev, hq, hkv, d, dtype, scale, calls=None):
    """Depth-first walk, one node per call unless ``calls`` lists the query
    nodes of each call (in walk order); returns device outputs."""
    import torch
    import prefix_shared_tree_attn_amd as ta
    n = t.num_tokens
    if calls is None:
        calls = [[i] for i in dfs_preorder(t.parent)]
    plans = [ta.plan(t.parent, t.seg_start, t.seg_len, n, hq, hkv, d, dtype, query_nodes=c)
             for c in calls]
    tdt = dev["q"].dtype
    o = torch.empty((n, hq, d), dtype=tdt, device="cuda")
    lse = torch.empty((hq, n), dtype=torch.float32, device="cuda")
    dq = torch.empty((n, hq, d), dtype=tdt, device="cuda")
    dk_acc = torch.zeros((n, hkv, d), dtype=torch.float32, device="cuda")
    dv_acc = torch.zeros((n, hkv, d), dtype=torch.float32, device="cuda")
    ws_bytes = max(p.workspace_size()[1] for p in plans)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    for p in plans:
        ta.fwd(p, dev["q"], dev["k"], dev["v"], scale, o=o, lse=lse)
    for p in reversed(plans):
        ta.bwd_accum(p, dev["q"], dev["k"], dev["v"], o, lse, dev["do"], scale, dk_acc, dv_acc,
                     dq=dq, ws=ws)
    dk = ta.accum_cast(dk_acc, dtype)
    dv = ta.accum_cast(dv_acc, dtype)
    torch.cuda.synchronize()
    for p in plans:
        p.close()
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv, "dk_acc": dk_acc, "dv_acc": dv_acc}


def _whole(t, dev, hq, hkv, d, dtype, scale):
    import torch
    import prefix_shared_tree_attn_amd as ta
    p = ta.plan(t.parent, t.seg_start, t.seg_len, t.num_tokens, hq, hkv, d, dtype)
    o, lse = ta.fwd(p, dev["q"], dev["k"], dev["v"], scale)
    dq, dk, dv = ta.bwd(p, dev["q"], dev["k"], dev["v"], o, lse, dev["do"], scale)
    torch.cuda.synchronize()
    p.close()
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


def _host(x):
    return x.double().cpu().numpy()


WALK_CASES = {
    "binary-ragged": (binary_tree(129, 97, 3), 4, 2, 128, "bf16"),
    "star-heavy-prompt": (star_tree(1024, 16, 64), 4, 2, 128, "bf16"),
    "forest": (random_tree(np.random.default_rng(3), 10, max_len=260, n_roots=3), 6, 2, 128,
               "bf16"),
    "d64-bf16": (random_tree(np.random.default_rng(6), 9, max_len=300), 4, 2, 64, "bf16"),
    "d64-fp32": (random_tree(np.random.default_rng(7), 8, max_len=200), 2, 1, 64, "fp32"),
}


@pytest.mark.parametrize("name", list(WALK_CASES))
def test_depth_first_walk_equals_whole_tree(name):
    import torch
    t, hq, hkv, d, dtype = WALK_CASES[name]
    scale = 1.0 / np.sqrt(d)
    print(f"case {name}: N={t.num_tokens} nodes={t.num_nodes} hq={hq} hkv={hkv} d={d} {dtype}",
          flush=True)
    x = make(t, hq, hkv, d, dtype, do_std=1.0 if dtype == "fp32" else 1e-2)
    dev = device_inputs(x, dtype)
    got = _walk(t, dev, hq, hkv, d, dtype, scale)
    ref = oracle.tree_attention(x.q, x.k, x.v, x.do, t.parent, t.seg_start, t.seg_len, scale)
    errs = {k: rel_l2(_host(got[k]), ref[k]) for k in ("o", "dq", "dk", "dv")}
    errs["lse"] = float(np.abs(_host(got["lse"]) - ref["lse"]).max())
    print("errors:", errs, flush=True)
    rel_bar, lse_bar = (FP32_REL_L2, FP32_LSE_ABS) if dtype == "fp32" else (REL_L2, LSE_ABS)
    for k in ("o", "dq", "dk", "dv"):
        assert errs[k] <= rel_bar, (k, errs)
    assert errs["lse"] <= lse_bar
    whole = _whole(t, dev, hq, hkv, d, dtype, scale)
    # fp32 sums in another order, then one rounding to the output type
    close = 2 * FP32_REL_L2 if dtype == "fp32" else 4e-3
    for k in ("o", "dq", "dk", "dv"):
        assert rel_l2(_host(got[k]), _host(whole[k])) <= close, k
    assert float((got["lse"] - whole["lse"]).abs().max()) <= 1e-4


@pytest.mark.parametrize("name,budget", [(name, 0) for name in WALK_CASES] +
                         [("forest", 400), ("binary-ragged", 300)])
def test_walk_in_runs_equals_whole_tree(name, budget):
    """The walk with one call per run of preorder nodes (tree_attn_walk_runs;
    budget 0: the deepest root path's rows).  A run holding a parent and the
    child stored after it has query tiles and key tiles that cross the node
    boundary (key-limit entries on the backward side)."""
    import prefix_shared_tree_attn_amd as ta
    t, hq, hkv, d, dtype = WALK_CASES[name]
    scale = 1.0 / np.sqrt(d)
    calls = ta.walk_runs(t.parent, t.seg_len, budget)
    print(f"case {name}: N={t.num_tokens} nodes={t.num_nodes} budget={budget} "
          f"runs={[len(c) for c in calls]}", flush=True)
    assert len(calls) < t.num_nodes  # some run holds several nodes
    x = make(t, hq, hkv, d, dtype, do_std=1.0 if dtype == "fp32" else 1e-2)
    dev = device_inputs(x, dtype)
    got = _walk(t, dev, hq, hkv, d, dtype, scale, calls)
    ref = oracle.tree_attention(x.q, x.k, x.v, x.do, t.parent, t.seg_start, t.seg_len, scale)
    errs = {k: rel_l2(_host(got[k]), ref[k]) for k in ("o", "dq", "dk", "dv")}
    errs["lse"] = float(np.abs(_host(got["lse"]) - ref["lse"]).max())
    print("errors:", errs, flush=True)
    rel_bar, lse_bar = (FP32_REL_L2, FP32_LSE_ABS) if dtype == "fp32" else (REL_L2, LSE_ABS)
    for k in ("o", "dq", "dk", "dv"):
        assert errs[k] <= rel_bar, (k, errs)
    assert errs["lse"] <= lse_bar


def test_one_call_on_a_node_subset():
    import torch
    import prefix_shared_tree_attn_amd as ta
    t = random_tree(np.random.default_rng(21), 14, max_len=220, n_roots=2)
    hq, hkv, d, dtype = 4, 2, 128, "bf16"
    scale = 1.0 / np.sqrt(d)
    rng = np.random.default_rng(5)
    qn = sorted(int(i) for i in rng.choice(t.num_nodes, size=6, replace=False))
    print(f"subset case: N={t.num_tokens} nodes={t.num_nodes} query nodes={qn}", flush=True)
    x = make(t, hq, hkv, d, dtype)
    dev = device_inputs(x, dtype)
    n = t.num_tokens
    p = ta.plan(t.parent, t.seg_start, t.seg_len, n, hq, hkv, d, dtype, query_nodes=qn)
    sentinel = 7.0
    o = torch.full((n, hq, d), sentinel, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((hq, n), sentinel, dtype=torch.float32, device="cuda")
    dq = torch.full((n, hq, d), sentinel, dtype=torch.bfloat16, device="cuda")
    gen = torch.Generator(device="cpu").manual_seed(1)
    acc0 = torch.randn((2, n, hkv, d), generator=gen, dtype=torch.float32).cuda()
    dk_acc, dv_acc = acc0[0].clone(), acc0[1].clone()
    ta.fwd(p, dev["q"], dev["k"], dev["v"], scale, o=o, lse=lse)
    ta.bwd_accum(p, dev["q"], dev["k"], dev["v"], o, lse, dev["do"], scale, dk_acc, dv_acc, dq=dq)
    torch.cuda.synchronize()
    ref = oracle.tree_attention_subset(x.q, x.k, x.v, x.do, t.parent, t.seg_start, t.seg_len,
                                       scale, qn)
    rows = ref["rows"]
    rt = torch.from_numpy(rows).cuda()
    # rows outside the subset are untouched
    assert bool((o[~rt] == sentinel).all()) and bool((dq[~rt] == sentinel).all())
    assert bool((lse[:, ~rt] == sentinel).all())
    errs = {"o": rel_l2(_host(o)[rows], ref["o"][rows]),
            "dq": rel_l2(_host(dq)[rows], ref["dq"][rows]),
            "dk": rel_l2(_host(dk_acc - acc0[0]), ref["dk"]),
            "dv": rel_l2(_host(dv_acc - acc0[1]), ref["dv"]),
            "lse": float(np.abs(_host(lse)[:, rows] - ref["lse"][:, rows]).max())}
    print("errors:", errs, flush=True)
    for k in ("o", "dq", "dk", "dv"):
        assert errs[k] <= REL_L2, (k, errs)
    assert errs["lse"] <= LSE_ABS
    # keys that no query row sees keep their accumulator bit for bit
    unseen = torch.from_numpy(np.all(ref["dk"] == 0, axis=(1, 2))).cuda()
    print(f"keys no query row sees: {int(unseen.sum())}", flush=True)
    assert torch.equal(dk_acc[unseen], acc0[0][unseen])
    assert torch.equal(dv_acc[unseen], acc0[1][unseen])
    p.close()


def test_plan_kind_checks_and_empty_subset():
    import torch
    import prefix_shared_tree_attn_amd as ta
    t = binary_tree(100, 60, 2)
    x = make(t, 2, 1, 128, "bf16")
    dev = device_inputs(x, "bf16")
    n = t.num_tokens
    whole = ta.plan(t.parent, t.seg_start, t.seg_len, n, 2, 1, 128)
    sub = ta.plan(t.parent, t.seg_start, t.seg_len, n, 2, 1, 128, query_nodes=[1])
    empty = ta.plan(t.parent, t.seg_start, t.seg_len, n, 2, 1, 128, query_nodes=[])
    o, lse = ta.fwd(whole, dev["q"], dev["k"], dev["v"], 0.1)
    acc = torch.zeros((n, 1, 128), dtype=torch.float32, device="cuda")
    acc2 = torch.zeros_like(acc)
    with pytest.raises(ta.TreeAttnError) as ei:
        ta.bwd(sub, dev["q"], dev["k"], dev["v"], o, lse, dev["do"], 0.1)
    assert ei.value.status == "INVALID_ARG"
    with pytest.raises(ta.TreeAttnError) as ei:
        ta.bwd_accum(whole, dev["q"], dev["k"], dev["v"], o, lse, dev["do"], 0.1, acc, acc2)
    assert ei.value.status == "INVALID_ARG"
    with pytest.raises(ta.TreeAttnError) as ei:
        ta.lin_fwd(sub, dev["q"], dev["k"], dev["v"], 0.1)
    assert ei.value.status == "UNSUPPORTED"
    o2 = o.clone()
    ta.fwd(empty, dev["q"], dev["k"], dev["v"], 0.1, o=o2, lse=lse.clone())
    ta.bwd_accum(empty, dev["q"], dev["k"], dev["v"], o, lse, dev["do"], 0.1, acc, acc2)
    torch.cuda.synchronize()
    assert torch.equal(o2, o) and bool((acc == 0).all()) and bool((acc2 == 0).all())
    # the cast: nearest-even bf16 of fp32 values, ragged length
    src = torch.randn(1027, dtype=torch.float32, device="cuda")
    got = ta.accum_cast(src, "bf16")
    torch.cuda.synchronize()
    assert torch.equal(got, src.to(torch.bfloat16))
    for p in (whole, sub, empty):
        p.close()


@pytest.mark.parametrize("cfg,walk", [(2, "node"), (4, "node"), (3, "runs"), (4, "runs")])
def test_full_size_walk(cfg, walk):
    """The GRPO-star (17 nodes), agent (config 3) and segment-search (127
    nodes) workloads at full size, one node per call or one run of preorder
    nodes per call (tree_attn_walk_runs): sampled rows and keys against the
    oracle, whole tensors against the one-call path to rounding (a walk's
    call has fewer query tiles than the one call, so the planner may cut
    their keys into parts)."""
    import torch
    import prefix_shared_tree_attn_amd as ta
    t = config_tree(cfg)
    sp = config_spec(cfg)
    hq, hkv, d, dtype, scale = sp["heads_q"], sp["heads_kv"], sp["head_dim"], sp["dtype"], sp["scale"]
    calls = ta.walk_runs(t.parent, t.seg_len) if walk == "runs" else None
    print(f"config {cfg} walk ({walk}): N={t.num_tokens} nodes={t.num_nodes} "
          f"calls={len(calls) if calls else t.num_nodes}", flush=True)
    x = make(t, hq, hkv, d, dtype, do_std=sp["do_std"])
    dev = device_inputs(x, dtype)
    got = _walk(t, dev, hq, hkv, d, dtype, scale, calls)
    print("walk done", flush=True)
    whole = _whole(t, dev, hq, hkv, d, dtype, scale)
    for k in ("o", "dq", "dk", "dv"):
        e = rel_l2(_host(got[k]), _host(whole[k]))
        print(f"{k}: walk vs one call rel-L2 {e:.2e}", flush=True)
        assert e <= 4e-3, k
    assert float((got["lse"] - whole["lse"]).abs().max()) <= 1e-4
    rng = np.random.default_rng(7)
    rows = sorted(set([0, t.num_tokens - 1] + [int(r) for r in rng.integers(0, t.num_tokens, 10)]))
    heads = [int(rng.integers(0, hq))]
    g = heads[0] // (hq // hkv)
    prompt = int(t.seg_len[0])  # node 0 is the root, stored first, on these trees
    keys = [0, prompt - 1, prompt + 5, t.num_tokens - 1]
    o, lse, dq = oracle.query_rows(x.q, x.k, x.v, x.do, t.parent, t.seg_start, t.seg_len, scale,
                                   rows, heads)
    dk, dv = oracle.key_rows(x.q, x.k, x.v, x.do, t.parent, t.seg_start, t.seg_len, scale, keys, g)
    ri, hi, ki = (torch.tensor(a, device="cuda") for a in (rows, heads, keys))
    errs = {"o": rel_l2(_host(got["o"][ri][:, hi]), o),
            "dq": rel_l2(_host(got["dq"][ri][:, hi]), dq),
            "dk": rel_l2(_host(got["dk"][ki, g]), dk),
            "dv": rel_l2(_host(got["dv"][ki, g]), dv),
            "lse": float(np.abs(_host(got["lse"][hi][:, ri]) - lse).max())}
    print("sampled errors:", errs, flush=True)
    for k in ("o", "dq", "dk", "dv"):
        assert errs[k] <= REL_L2, (k, errs)
    assert errs["lse"] <= LSE_ABS


@pytest.mark.parametrize("seed", range(6))
def test_subset_sweep(seed):
    """Seeded random forests (depth-first or random packing, both dtypes,
    D 64/128, GQA) with a random set of query nodes, one call, against
    ``oracle.tree_attention_subset``; accumulators start from zero."""
    import torch
    import prefix_shared_tree_attn_amd as ta
    rng = np.random.default_rng(2000 + seed)
    t = random_tree(rng, int(rng.integers(3, 20)), max_len=int(rng.choice([60, 200])),
                    n_roots=int(rng.integers(1, 3)), shuffle=seed % 2 == 1)
    hkv = int(rng.choice([1, 2]))
    hq = hkv * int(rng.choice([1, 2, 4]))
    d = int(rng.choice([64, 128]))
    dtype = "fp32" if seed % 3 == 2 else "bf16"
    qn = sorted(int(i) for i in rng.choice(t.num_nodes, size=int(rng.integers(1, t.num_nodes + 1)),
                                           replace=False))
    print(f"subset sweep seed {seed}: N={t.num_tokens} nodes={t.num_nodes} hq={hq} hkv={hkv} "
          f"d={d} {dtype} query nodes={qn}", flush=True)
    scale = 1.0 / np.sqrt(d)
    x = make(t, hq, hkv, d, dtype, do_std=1.0 if dtype == "fp32" else 1e-2)
    dev = device_inputs(x, dtype)
    n = t.num_tokens
    p = ta.plan(t.parent, t.seg_start, t.seg_len, n, hq, hkv, d, dtype, query_nodes=qn)
    tdt = dev["q"].dtype
    o = torch.zeros((n, hq, d), dtype=tdt, device="cuda")
    lse = torch.zeros((hq, n), dtype=torch.float32, device="cuda")
    dq = torch.zeros((n, hq, d), dtype=tdt, device="cuda")
    dk_acc = torch.zeros((n, hkv, d), dtype=torch.float32, device="cuda")
    dv_acc = torch.zeros_like(dk_acc)
    ta.fwd(p, dev["q"], dev["k"], dev["v"], scale, o=o, lse=lse)
    ta.bwd_accum(p, dev["q"], dev["k"], dev["v"], o, lse, dev["do"], scale, dk_acc, dv_acc, dq=dq)
    torch.cuda.synchronize()
    p.close()
    ref = oracle.tree_attention_subset(x.q, x.k, x.v, x.do, t.parent, t.seg_start, t.seg_len,
                                       scale, qn)
    rows = ref["rows"]
    errs = {"o": rel_l2(_host(o)[rows], ref["o"][rows]),
            "dq": rel_l2(_host(dq)[rows], ref["dq"][rows]),
            "dk": rel_l2(_host(dk_acc), ref["dk"]),
            "dv": rel_l2(_host(dv_acc), ref["dv"]),
            "lse": float(np.abs(_host(lse)[:, rows] - ref["lse"][:, rows]).max())}
    print("errors:", errs, flush=True)
    for k in ("o", "dq", "dk", "dv"):
        assert errs[k] <= REL_L2, (k, errs)
    assert errs["lse"] <= LSE_ABS
    # rows outside the subset stay as they were
    assert not bool(o[torch.from_numpy(~rows).cuda()].any())
