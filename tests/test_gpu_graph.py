"""The forward, backward, accumulating backward, cast and linear-attention
calls enqueue only kernels on the caller's stream (no allocation, host
synchronisation or memset once the plan exists), so a training loop may
capture them in a HIP graph.  Each case captures a pass, replays it several times with eager work
and synchronisations between the replays, and checks every replay bit for
bit against the eager pass: the kernels take the same inputs in the same
order, so the results must not differ in a single bit.
"""

import numpy as np
import pytest

from tree_inputs import binary_tree, random_tree, star_tree
from gpu_util import device_inputs, make

pytestmark = pytest.mark.gpu

CASES = {
    "binary-ragged-bf16": (binary_tree(129, 97, 3), 4, 2, 128, "bf16"),
    "star-key-parts-bf16": (star_tree(3200, 3, 200), 4, 2, 128, "bf16"),
    "forest-d64-fp32": (random_tree(np.random.default_rng(7), 8, max_len=200, n_roots=2),
                        2, 1, 64, "fp32"),
}


def _capture_and_replay(fn, outs, reps=3):
    """Eager pass, capture, then `reps` replays, each against the eager
    result; the outputs are overwritten before every replay and the eager
    pass runs again between replays."""
    import torch
    fn()
    torch.cuda.synchronize()
    ref = [a.clone() for a in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    for rep in range(reps):
        for a in outs:
            a.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, ref)):
            assert torch.equal(a, b), (rep, i)
        fn()  # the program's own eager work between replays
        torch.cuda.synchronize()
        for a, b in zip(outs, ref):
            assert torch.equal(a, b)
    del g


@pytest.mark.parametrize("name", list(CASES))
def test_one_call_pass_in_a_graph(name):
    import torch
    import prefix_shared_tree_attn_amd as ta
    t, hq, hkv, d, dtype = CASES[name]
    print(f"case {name}: N={t.num_tokens} nodes={t.num_nodes}", flush=True)
    x = make(t, hq, hkv, d, dtype, do_std=1.0 if dtype == "fp32" else 1e-2)
    dev = device_inputs(x, dtype)
    n, scale = t.num_tokens, 1.0 / np.sqrt(d)
    p = ta.plan(t.parent, t.seg_start, t.seg_len, n, hq, hkv, d, dtype)
    ws_f, ws_b = ta.workspace(p, "fwd"), ta.workspace(p, "bwd")
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    o = torch.empty_like(q)
    lse = torch.empty((hq, n), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

    def step():
        ta.fwd(p, q, k, v, scale, o=o, lse=lse, ws=ws_f)
        ta.bwd(p, q, k, v, o, lse, do, scale, dq=dq, dk=dk, dv=dv, ws=ws_b)

    _capture_and_replay(step, [o, lse, dq, dk, dv])
    p.close()


@pytest.mark.parametrize("name", list(CASES))
def test_walk_in_a_graph(name):
    import torch
    import prefix_shared_tree_attn_amd as ta
    t, hq, hkv, d, dtype = CASES[name]
    x = make(t, hq, hkv, d, dtype, do_std=1.0 if dtype == "fp32" else 1e-2)
    dev = device_inputs(x, dtype)
    n, scale = t.num_tokens, 1.0 / np.sqrt(d)
    calls = ta.walk_runs(t.parent, t.seg_len)
    print(f"case {name}: N={n} nodes={t.num_nodes} calls={len(calls)}", flush=True)
    plans = [ta.plan(t.parent, t.seg_start, t.seg_len, n, hq, hkv, d, dtype, query_nodes=c)
             for c in calls]
    ws_f = torch.empty(max(1, max(p.workspace_size()[0] for p in plans)), dtype=torch.uint8,
                       device="cuda")
    ws_b = torch.empty(max(1, max(p.workspace_size()[1] for p in plans)), dtype=torch.uint8,
                       device="cuda")
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    o = torch.empty_like(q)
    lse = torch.empty((hq, n), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    acc = torch.empty((2, n, hkv, d), dtype=torch.float32, device="cuda")

    def walk():
        acc.zero_()  # a fill kernel, not a memset node
        for p in plans:
            ta.fwd(p, q, k, v, scale, o=o, lse=lse, ws=ws_f)
        for p in reversed(plans):
            ta.bwd_accum(p, q, k, v, o, lse, do, scale, acc[0], acc[1], dq=dq, ws=ws_b)
        ta.accum_cast(acc[0], dtype, out=dk)
        ta.accum_cast(acc[1], dtype, out=dv)

    _capture_and_replay(walk, [o, lse, dq, dk, dv])
    for p in plans:
        p.close()


@pytest.mark.parametrize("name", ["binary-ragged-bf16", "star-key-parts-bf16"])
def test_linear_pass_in_a_graph(name):
    import torch
    import prefix_shared_tree_attn_amd as ta
    t, hq, hkv, d, dtype = CASES[name]
    x = make(t, hq, hkv, d, dtype)
    dev = device_inputs(x, dtype)
    n, scale = t.num_tokens, 1.0 / np.sqrt(d)
    p = ta.plan(t.parent, t.seg_start, t.seg_len, n, hq, hkv, d, dtype)
    print(f"case {name}: N={n} pieces={p.stats()['lin_pieces']}", flush=True)
    ws = ta.lin_workspace(p, "bwd")  # the backward's workspace covers the forward's
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    o = torch.empty_like(q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

    def step():
        ta.lin_fwd(p, q, k, v, scale, o=o, ws=ws)
        ta.lin_bwd(p, q, k, v, do, scale, dq=dq, dk=dk, dv=dv, ws=ws)

    _capture_and_replay(step, [o, dq, dk, dv])
    p.close()
