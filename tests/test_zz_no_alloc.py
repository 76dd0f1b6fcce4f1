"""tree_attn_bwd_noalloc: the backward pass with the library's fixed scratch.

GPU: two calls in a row through the C ABI, the second on a smaller tree,
each checked against tree_attn_bwd with a caller workspace (same kernels and
plan, so the results must agree bit for bit) and against the fp64 oracle at
the parity bar; then a plan whose query tiles are cut into key parts, whose
partial dQ also lives in the fixed scratch.  CPU: the size, plan-kind and null checks
that run before any device work.
"""

import ctypes

import numpy as np
import pytest

import oracle
import prefix_shared_tree_attn_amd as ta
from prefix_shared_tree_attn_amd import _ffi
from tree_inputs import binary_tree, chain_tree, star_tree
from gpu_util import LSE_ABS, REL_L2, device_inputs, make, rel_l2

STATIC_BYTES = 64 << 20
WORKSPACE, INVALID_ARG, NO_DEVICE_PLAN = 5, 1, 7


def _noalloc_raw(handle):
    null = ctypes.c_void_p(0)
    return _ffi.lib().tree_attn_bwd_noalloc(handle, *([null] * 6), ctypes.c_float(0.1),
                                           null, null, null, null)


def test_noalloc_rejects_before_any_device_work():
    # a plan whose backward scratch exceeds the fixed array: WORKSPACE
    big = star_tree(2048, 16, 1024)
    p = ta.plan_host(big.parent, big.seg_start, big.seg_len, big.num_tokens, 8, 2, 128, "bf16")
    assert p.workspace_size()[1] > STATIC_BYTES
    assert _noalloc_raw(p.handle) == WORKSPACE
    assert b"fixed" in _ffi.lib().tree_attn_last_error()
    # a plan that fits but has no device arrays: NO_DEVICE_PLAN
    small = binary_tree(129, 97, 3)
    p2 = ta.plan_host(small.parent, small.seg_start, small.seg_len, small.num_tokens, 4, 2,
                      128, "bf16")
    assert 0 < p2.workspace_size()[1] <= STATIC_BYTES
    assert _noalloc_raw(p2.handle) == NO_DEVICE_PLAN
    # null plan
    assert _noalloc_raw(ctypes.c_void_p(0)) == INVALID_ARG
    p.close()
    p2.close()


def _one_call(t, hq, hkv, d, dtype, check_oracle):
    import torch
    scale = 1.0 / np.sqrt(d)
    x = make(t, hq, hkv, d, dtype)
    dev = device_inputs(x, dtype)
    p = ta.plan(t.parent, t.seg_start, t.seg_len, t.num_tokens, hq, hkv, d, dtype)
    need = p.workspace_size()[1]
    print(f"case: N={t.num_tokens} nodes={t.num_nodes} hq={hq} hkv={hkv} d={d} {dtype} "
          f"scratch={need} slots={p.stats()['bwd_slots']}", flush=True)
    assert 0 < need <= STATIC_BYTES
    o, lse = ta.fwd(p, dev["q"], dev["k"], dev["v"], scale)
    ref_dev = ta.bwd(p, dev["q"], dev["k"], dev["v"], o, lse, dev["do"], scale)
    got_dev = ta.bwd_noalloc(p, dev["q"], dev["k"], dev["v"], o, lse, dev["do"], scale)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got_dev, ref_dev):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b), name
    if check_oracle:
        ref = oracle.tree_attention(x.q, x.k, x.v, x.do, t.parent, t.seg_start, t.seg_len,
                                    scale)
        got = {"o": o, "lse": lse, "dq": got_dev[0], "dk": got_dev[1], "dv": got_dev[2]}
        got = {k: v.float().cpu().numpy().astype(np.float64) for k, v in got.items()}
        errs = {k: rel_l2(got[k], ref[k]) for k in ("o", "dq", "dk", "dv")}
        errs["lse"] = float(np.abs(got["lse"] - ref["lse"]).max())
        print("errors:", errs, flush=True)
        for k in ("o", "dq", "dk", "dv"):
            assert errs[k] <= REL_L2, (k, errs)
        assert errs["lse"] <= LSE_ABS, errs
    p.close()


@pytest.mark.gpu
def test_noalloc_two_calls_second_smaller():
    # first: a 1024-token prompt whose key tiles are split into slots
    _one_call(star_tree(1024, 16, 64), 4, 2, 128, "bf16", check_oracle=True)
    # second: a smaller, ragged tree on the same (now dirty) scratch
    _one_call(binary_tree(129, 97, 3), 4, 2, 128, "bf16", check_oracle=True)


@pytest.mark.gpu
def test_noalloc_with_key_parts():
    t = chain_tree([3500, 300])
    p = ta.plan(t.parent, t.seg_start, t.seg_len, t.num_tokens, 4, 2, 128, "bf16")
    assert p.stats()["fwd_split_tiles"] > 0
    p.close()
    _one_call(t, 4, 2, 128, "bf16", check_oracle=True)
