"""GPU tests of the passes either side of tree attention, through the C ABI,
against oracle/prefix_tree.py: the gather is bit-exact, the scatter-sum and
the rotary embedding are compared in fp64 (fp32: relative error <= 1e-5;
bf16: relative L2 <= 1e-2, the bf16 bar of the attention path)."""

import numpy as np
import pytest

import oracle
from oracle import prefix_tree as opt
from tree_inputs import config_tree

pytestmark = pytest.mark.gpu


def _rel(a, b):
    return float(np.linalg.norm((np.asarray(a, np.float64) - b).ravel())
                 / max(np.linalg.norm(np.asarray(b, np.float64).ravel()), 1e-300))


@pytest.mark.parametrize("shape,dtype", [((300, 64), "bf16"), ((300, 3), "fp32"),
                                          ((300,), "bf16"), ((300,), "fp32"),
                                          ((300, 4, 128), "bf16")])
def test_gather_bit_exact(shape, dtype):
    import torch
    import prefix_shared_tree_attn_amd as ta
    rng = np.random.default_rng(1)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    src = torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(tdt).cuda()
    idx_np = rng.integers(0, shape[0], 777).astype(np.int32)
    idx = torch.from_numpy(idx_np).cuda()
    print(f"gather case {shape} {dtype}", flush=True)
    out = ta.gather_rows(src, idx)
    torch.cuda.synchronize()
    ref = opt.gather_rows(src.float().cpu().numpy(), idx_np)
    np.testing.assert_array_equal(out.float().cpu().numpy(), ref)


def _trajectories(cfg):
    t = config_tree(cfg)
    return [p.tolist() for p in oracle.root_to_leaf_paths(t.parent, t.seg_start, t.seg_len)]


@pytest.mark.parametrize("cfg,width,dtype", [(1, 64, "fp32"), (1, 1, "fp32"), (2, 96, "fp32"),
                                             (2, 128, "bf16"), (4, 16, "bf16"), (1, 5, "bf16"),
                                             (1, 3, "fp32")])
def test_scatter_sum_matches_oracle(cfg, width, dtype):
    import torch
    import prefix_shared_tree_attn_amd as ta
    tree = ta.build_tree(_trajectories(cfg))
    total = tree.traj_index.shape[0]
    rng = np.random.default_rng(2)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    src = torch.from_numpy(rng.standard_normal((total, width)).astype(np.float32)).to(tdt).cuda()
    print(f"scatter case cfg{cfg} T={total} N={tree.num_tokens} w={width} {dtype}", flush=True)
    off = torch.from_numpy(tree.inv_offsets).cuda()
    pos = torch.from_numpy(tree.inv_positions).cuda()
    out = ta.scatter_sum_rows(src, off, pos, tree.num_tokens)
    out2 = ta.scatter_sum_rows(src, off, pos, tree.num_tokens)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)  # fixed summation order
    ref = opt.scatter_sum_rows(src.float().cpu().numpy(), tree.traj_index, tree.num_tokens)
    err = _rel(out.float().cpu().numpy(), ref)
    print("rel error", err, flush=True)
    assert err <= (1e-5 if dtype == "fp32" else 1e-2)


@pytest.mark.parametrize("d,theta,dtype,inverse", [(128, 1e4, "fp32", False), (64, 5e5, "fp32", True),
                                                    (128, 1e4, "bf16", False), (128, 1e4, "bf16", True)])
def test_rope_matches_oracle_at_tree_depth(d, theta, dtype, inverse):
    import torch
    import prefix_shared_tree_attn_amd as ta
    t = config_tree(5)  # long trunk: positions up to ~34.7K
    p = ta.plan(t.parent, t.seg_start, t.seg_len, t.num_tokens, 2, 1, 128)
    _, pos = ta.positions(p)
    rng = np.random.default_rng(3)
    rows = np.sort(rng.choice(t.num_tokens, 3000, replace=False))
    h = 3
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    x = torch.from_numpy(rng.standard_normal((t.num_tokens, h, d)).astype(np.float32)).to(tdt).cuda()
    x0 = x[torch.from_numpy(rows).cuda()].float().cpu().numpy()
    print(f"rope case d={d} theta={theta} {dtype} inverse={inverse}", flush=True)
    ta.rope(x, pos, theta=theta, inverse=inverse)
    torch.cuda.synchronize()
    got = x[torch.from_numpy(rows).cuda()].float().cpu().numpy()
    ref = opt.rope(x0, pos.cpu().numpy()[rows], theta=theta, inverse=inverse)
    err = _rel(got, ref)
    print("rel error", err, flush=True)
    assert err <= (1e-5 if dtype == "fp32" else 1e-2)
    p.close()


@pytest.mark.parametrize("d,dtype", [(6, "fp32"), (6, "bf16"), (10, "fp32")])
def test_rope_scalar_path(d, dtype):
    """Head sizes whose half is not a multiple of 4 take the one-pair path."""
    import torch
    import prefix_shared_tree_attn_amd as ta
    rng = np.random.default_rng(6)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    x = torch.from_numpy(rng.standard_normal((257, 3, d)).astype(np.float32)).to(tdt).cuda()
    pos_np = rng.integers(0, 40000, 257).astype(np.int32)
    x0 = x.float().cpu().numpy()
    ta.rope(x, torch.from_numpy(pos_np).cuda())
    torch.cuda.synchronize()
    err = _rel(x.float().cpu().numpy(), opt.rope(x0, pos_np))
    assert err <= (1e-5 if dtype == "fp32" else 1e-2), err


def test_rope_round_trip_fp32():
    import torch
    import prefix_shared_tree_attn_amd as ta
    rng = np.random.default_rng(4)
    x = torch.from_numpy(rng.standard_normal((500, 2, 64)).astype(np.float32)).cuda()
    pos = torch.from_numpy(rng.integers(0, 40000, 500).astype(np.int32)).cuda()
    y = x.clone()
    ta.rope(y, pos)
    ta.rope(y, pos, inverse=True)
    torch.cuda.synchronize()
    assert _rel(y.cpu().numpy(), x.cpu().numpy()) <= 1e-6


def test_end_to_end_trajectories_to_unique_dout():
    """Per-trajectory dO rows summed onto unique tokens equal, for every
    unique token, the oracle's sum over the trajectory positions of its
    prefix (the dO contract of tree_attn_bwd)."""
    import torch
    import prefix_shared_tree_attn_amd as ta
    trajs = _trajectories(2)
    tree = ta.build_tree(trajs)
    ref_tree = opt.build_tree(trajs)
    np.testing.assert_array_equal(tree.traj_index, ref_tree["traj_index"])
    rng = np.random.default_rng(5)
    total = tree.traj_index.shape[0]
    hq, d = 4, 128
    do_traj = torch.from_numpy(rng.standard_normal((total, hq, d)).astype(np.float32)).cuda()
    do_u = ta.scatter_sum_rows(do_traj, torch.from_numpy(tree.inv_offsets).cuda(),
                               torch.from_numpy(tree.inv_positions).cuda(), tree.num_tokens)
    back = ta.gather_rows(do_u, torch.from_numpy(tree.traj_index).cuda())
    torch.cuda.synchronize()
    ref = opt.scatter_sum_rows(do_traj.cpu().numpy().reshape(total, -1), ref_tree["traj_index"],
                               tree.num_tokens).reshape(tree.num_tokens, hq, d)
    assert _rel(do_u.cpu().numpy(), ref) <= 1e-5
    np.testing.assert_array_equal(back.cpu().numpy(), do_u.cpu().numpy()[tree.traj_index])
