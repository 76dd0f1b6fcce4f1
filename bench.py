"""Benchmark: prefix-shared tree attention forward + backward on one MI355X.

One step is one pass of the whole path over one batch: build the plan for
the tree (host planning + upload of its work arrays), the per-token position
pass, the forward pass and the backward pass (preprocess, main, reductions).  Throughput is unique
tokens per second and TFLOP/s counted on the deduplicated tree work,
14 * D * Hq * sum_t (d(t) + 1) per step (forward 4, backward 10, in the
usual attention convention with the backward's recomputation).

Prints one JSON line.  Default workload: the long-trunk agentic tree, the
largest of the five (a 32,768-token trunk with 64 branches of 2,048 tokens
attached at seeded trunk positions, 163,840 unique tokens; 64 query / 8 kv
heads, head dim 128, bf16).  ``--config`` selects another of the five
workload trees.  The host baseline times the fp64 oracle on a bounded sample
(whole root-to-leaf paths, one query head) and scales it; the line says so.  ``--workload linear`` times the chunkwise linear-attention pass over
the same tree instead (plan + linear forward + linear backward per step),
with its own metric line.  ``--workload dfs`` runs the same softmax
attention as a depth-first walk of the tree (forward calls in preorder,
accumulating backward calls in reverse), with the calls' plans built before
the timed region, and reports it beside the one-call pass: by default each
call takes a run of consecutive preorder nodes whose root paths fit in the
longest root-to-leaf path (tree_attn_walk_runs), with ``--walk node`` one
node per call.  Only one
GPU is used; ``--gpus`` above 1 is refused.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CUs x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
PEAK_FP32_TFLOPS = 157.3    # dense fp32 matrix peak
PEAK_HBM_GBS = 8000.0
METRIC = "tree-attn fwd+bwd unique tokens/s and TFLOP/s (% of bf16 MFMA peak), 1 GPU"
DFS_METRIC = ("tree-attn fwd+bwd unique tokens/s, depth-first walk (query-subset calls, "
              "accumulated K/V gradients), 1 GPU")
LIN_METRIC = "tree linear-attn fwd+bwd unique tokens/s (chunkwise, state handoffs), 1 GPU"
LIN_CHUNK = 64


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def _args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=5, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip timing the oracle on the host")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run a plain device copy of this size (counter calibration)")
    ap.add_argument("--workload", choices=["softmax", "linear", "dfs"], default="softmax",
                    help="softmax tree attention (default), chunkwise linear attention, or "
                         "softmax tree attention as a depth-first walk")
    ap.add_argument("--walk", choices=["runs", "node"], default="runs",
                    help="depth-first walk: runs of preorder nodes within the deepest path's "
                         "rows per call (default), or one node per call")
    return ap.parse_args()


def _inputs_sha256(t, x, dtype: str) -> str:
    """SHA-256 over the node table (parent, seg_start, seg_len as int32) and
    the Q, K, V, dO tensors exactly as uploaded (bf16 bit patterns, or fp32),
    so that a run's inputs can be checked against a regeneration from the
    seeds."""
    h = hashlib.sha256()
    for a in (t.parent, t.seg_start, t.seg_len):
        h.update(np.ascontiguousarray(a, np.int32).tobytes())
    for name in ("q", "k", "v", "do"):
        a = x.bits[name] if dtype == "bf16" else getattr(x, name)
        h.update(memoryview(np.ascontiguousarray(a)).cast("B"))
    return h.hexdigest()


def _traffic_from_profile(kernel: str, workload: str):
    """HBM bytes per launch of a kernel from the committed counter summary,
    if it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("sources_sha256") != _sources_sha():
        return None
    return rec.get("bytes_per_launch")


def _sources_sha() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "prefix_shared_tree_attn_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h", ".cpp")):
            h.update(name.encode())
            h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()


def _host_threads():
    """Cores this process may run on, and the BLAS library behind NumPy."""
    from threadpoolctl import threadpool_info
    cores = len(os.sched_getaffinity(0))
    libs = [p for p in threadpool_info() if p.get("user_api") == "blas"]
    blas = ", ".join(f"{p.get('internal_api', '?')} {p.get('version', '?')}" for p in libs)
    return cores, blas or "none found"


def _sample_paths(t, d: int, budget_flop: float = 1.0e12):
    """Root-to-leaf paths (leaves in node order) taken for the host timing
    sample: as many as fit a dense fp64 fwd+bwd budget of one query head
    (12 D FLOP per (query, key) pair of each path, the oracle keeping P),
    at least one."""
    import oracle
    paths = oracle.root_to_leaf_paths(t.parent, t.seg_start, t.seg_len)
    chosen, work = [], 0.0
    for p in paths:
        w = 12.0 * d * len(p) * (len(p) + 1) / 2
        if chosen and work + w > budget_flop:
            break
        chosen.append(p)
        work += w
    return chosen


def cpu_baseline(t, spec, sample):
    """Times the unmodified fp64 oracle on the host's cores over a bounded
    sample of the workload and scales it to unique tokens/s of the whole
    workload.  ``sample`` is (rows of each sampled path, q, k, v, dO of query
    head 0 and kv head 0 on those rows).  The sampled paths run through the
    oracle as a forest of independent chains (each path is its own
    trajectory), which is exactly the dense per-path work the oracle does for
    them in the whole tree; the result is scaled by the ratio of the whole
    workload's dense per-path work (every path, every query head) to the
    sample's."""
    import oracle
    from threadpoolctl import threadpool_limits
    from tree_inputs import NodeTable, tree_stats
    lens, q, k, v, do = sample
    m = len(lens)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int32)
    forest = NodeTable(np.full(m, -1, np.int32), starts, np.asarray(lens, np.int32),
                       int(sum(lens)))
    cores, blas = _host_threads()
    with threadpool_limits(limits=cores, user_api="blas"):
        t0 = time.perf_counter()
        oracle.tree_attention(q, k, v, do, forest.parent, forest.seg_start, forest.seg_len,
                              spec["scale"])
        dt = time.perf_counter() - t0
    hq = spec["heads_q"]
    whole = tree_stats(t)["dense_pairs"] * hq
    part = sum(int(x) * (int(x) + 1) // 2 for x in lens)
    factor = whole / part
    return {
        "value": t.num_tokens / (dt * factor),
        "unit": "unique tokens/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"{m} of the tree's root-to-leaf paths ({int(sum(lens))} tokens), query "
                   f"head 0 of {hq}, fwd+bwd in fp64: {dt:.2f} s on {cores} cores; scaled by "
                   f"{factor:.1f}, the whole workload's dense per-path work over the sample's"),
        "blas": blas,
        "scaled": True,
        "sample_seconds": dt,
        "scale_factor": factor,
    }


def _baseline_sample(t, x, d):
    """Rows and head-0 inputs of the paths ``cpu_baseline`` times, copied out
    before the full host inputs are released."""
    paths = _sample_paths(t, d)
    idx = np.concatenate(paths)
    lens = [len(p) for p in paths]
    return (lens, x.q[idx, 0:1].copy(), x.k[idx, 0:1].copy(), x.v[idx, 0:1].copy(),
            x.do[idx, 0:1].copy())


def cpu_baseline_linear(t, spec):
    """Times the fp64 linear-attention oracle on the host over one kv-head
    group of the same workload and scales it to unique tokens/s."""
    import oracle
    from tree_inputs import make_inputs
    from threadpoolctl import threadpool_info
    hq, hkv, d = spec["heads_q"], spec["heads_kv"], spec["head_dim"]
    x = make_inputs(t.num_tokens, hq, hkv, d, dtype=spec["dtype"], do_std=spec["do_std"])
    t0 = time.perf_counter()
    oracle.tree_linear_attention(x.q, x.k, x.v, x.do, t.parent, t.seg_start, t.seg_len,
                                 spec["scale"], kv_heads=[0])
    dt = time.perf_counter() - t0
    threads = sum(int(p.get("num_threads", 0)) for p in threadpool_info()
                  if p.get("user_api") == "blas") or 1
    return {
        "value": t.num_tokens / (dt * hkv),
        "unit": "unique tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"kv-head group 0 of {hkv} ({hq // hkv} query heads), full tree, linear "
                   f"attention fwd+bwd in fp64 by path expansion: {dt:.2f} s, scaled by "
                   f"{hkv} groups"),
    }


def main_linear(args) -> int:
    """Chunkwise linear attention over the tree: plan + forward + backward."""
    import torch
    import prefix_shared_tree_attn_amd as ta
    from tree_inputs import config_spec, config_tree, make_inputs, tree_stats

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    cfg = args.config
    t = config_tree(cfg)
    spec = config_spec(cfg)
    if spec["dtype"] != "bf16":
        print("the linear-attention pass takes bf16 tensors; choose a bf16 workload",
              file=sys.stderr)
        return 2
    st = tree_stats(t)
    hq, hkv, d = spec["heads_q"], spec["heads_kv"], spec["head_dim"]
    scale = spec["scale"]
    n = t.num_tokens
    log(f"linear workload {spec['name']}: N={n} nodes={t.num_nodes} hq={hq} hkv={hkv} d={d}")
    x = make_inputs(n, hq, hkv, d, dtype="bf16", do_std=spec["do_std"])

    def up(name):
        return torch.from_numpy(x.bits[name].view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v, do = up("q"), up("k"), up("v"), up("do")
    o = torch.empty_like(q)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    probe = ta.plan(t.parent, t.seg_start, t.seg_len, n, hq, hkv, d, "bf16")
    ws = ta.lin_workspace(probe, "bwd")
    pstats = probe.stats()
    probe.close()
    del x
    plans = []

    def step():
        p = ta.plan(t.parent, t.seg_start, t.seg_len, n, hq, hkv, d, "bf16")
        ta.lin_fwd(p, q, k, v, scale, o=o, ws=ws)
        ta.lin_bwd(p, q, k, v, do, scale, dq=dq, dk=dk, dv=dv, ws=ws)
        plans.append(p)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    for p in plans:
        p.close()
    plans.clear()
    log(f"warmup done ({args.warmup} steps)")
    ta.timing_read(reset=True)
    ta.timing_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ta.timing_enable(False)
    kt = ta.timing_read(reset=True)
    for p in plans:
        p.close()
    plans.clear()
    log(f"timed {args.steps} steps: {wall:.3f} s")
    # the same steps again without the per-kernel events (a few microseconds
    # per launch), for reference
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall_plain = time.perf_counter() - t0
    for p in plans:
        p.close()
    plans.clear()
    if args.copy_probe_mib > 0:
        nb = args.copy_probe_mib << 20
        a = torch.ones(nb // 4, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        torch.mul(a, 1.0, out=b)
        torch.cuda.synchronize()
        log(f"copy probe: {nb} bytes read + {nb} bytes written")

    ms_step = 1e3 * wall / args.steps
    P, M, C, E = pstats["lin_pieces"], t.num_nodes, LIN_CHUNK, 2
    sb = P * hkv * d * d * E            # bf16 piece states (or deltas)
    eb = M * hkv * d * d * 4            # fp32 node-boundary states
    tq = n * hq * d * E                 # one [N, Hq, D] bf16 tensor
    tk = n * hkv * d * E                # one [N, Hkv, D] bf16 tensor
    # algorithmic HBM bytes per launch (each operand read once, each result
    # written once)
    kern_bytes = {
        "lin_kv": 2 * tk + sb,          # K, V -> per-piece K^T V
        "lin_scan": 2 * sb + eb,        # deltas -> states (+ node ends)
        "lin_out": sb + tq + 2 * tk + tq,
        "lin_qdo": 2 * tq + sb,
        "lin_rscan": 2 * sb + eb,
        "lin_dq": sb + tq + 2 * tk + tq,
        "lin_dkdv": sb + 2 * tq + 4 * tk,  # R, Q, dO, K, V -> dK, dV
    }
    # matrix-core work as executed (chunks padded to 64 tokens)
    f_in = 2.0 * C * d * d               # one chunk x state product
    f_att = 4.0 * C * C * d               # masked chunk products
    kern_flop = {
        "lin_kv": P * hkv * f_in, "lin_scan": 0.0, "lin_out": P * hq * (f_in + f_att),
        "lin_qdo": P * hq * f_in, "lin_rscan": 0.0, "lin_dq": P * hq * (f_in + f_att),
        "lin_dkdv": 2 * (P * hkv * f_in + P * hq * f_att),
    }
    step_flop = (2 * kern_flop["lin_kv"] + kern_flop["lin_out"] + kern_flop["lin_qdo"]
                 + kern_flop["lin_dq"] + kern_flop["lin_dkdv"])

    def avg_ms(kind):
        r = kt[kind]
        return r["total_ms"] / max(r["launches"], 1)

    kinds = [kk for kk in kern_bytes if kt[kk]["launches"]]
    kname = {"lin_kv": "lin_outer_kernel", "lin_scan": "lin_scan_kernel",
             "lin_out": "lin_chunk_kernel<128, 0>", "lin_qdo": "lin_outer_kernel",
             "lin_rscan": "lin_scan_kernel", "lin_dq": "lin_chunk_kernel<128, 1>",
             "lin_dkdv": "lin_dkdv_kernel<128>"}

    def roof(kind):
        ach = kern_bytes[kind] / (avg_ms(kind) * 1e-3) / 1e9
        return {"bound": "hbm", "kernel": kname[kind], "achieved": ach, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": ach / PEAK_HBM_GBS, "bytes_per_launch": kern_bytes[kind],
                "avg_ms": avg_ms(kind)}

    dominant = max(kinds, key=avg_ms)
    main_roof = roof(dominant)
    main_roof["traffic"] = _traffic_from_profile(dominant, spec["name"] + "-linear")
    result = {
        "metric": LIN_METRIC,
        "value": n / (ms_step * 1e-3),
        "unit": "unique tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "ms_per_step_without_events": 1e3 * wall_plain / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{spec['name']} tree, chunkwise linear attention (chunk {C})",
            "unique_tokens": n, "nodes": t.num_nodes, "pieces": P, "heads_q": hq,
            "heads_kv": hkv, "head_dim": d, "scale": scale, "global_batch": 1,
            "seq_len": st["max_path"], "parallelism": "none (1 GPU)",
        },
        "tflops": step_flop / (ms_step * 1e-3) / 1e12,
        "kernels_ms": {kk: avg_ms(kk) for kk in kinds},
        "roofline": main_roof,
        "roofline_kernels": {kk: roof(kk) for kk in kinds},
    }
    if not args.no_cpu_baseline:
        log("timing the linear-attention oracle on the host (cpu baseline)")
        result["cpu_baseline"] = cpu_baseline_linear(t, spec)
    print(json.dumps(result), flush=True)
    return 0


def main_dfs(args) -> int:
    """Softmax tree attention as a depth-first walk: per step, zero the fp32
    K/V gradient accumulators, one forward call per node in preorder, one
    accumulating backward call per node in reverse preorder, and the casts
    of the accumulators.  The one-call pass (plan built beforehand) is timed
    in the same run for comparison."""
    import torch
    import prefix_shared_tree_attn_amd as ta
    from tree_inputs import config_spec, config_tree, dfs_preorder, make_inputs, tree_stats

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    cfg = args.config
    t = config_tree(cfg)
    spec = config_spec(cfg)
    st = tree_stats(t)
    hq, hkv, d, dtype = spec["heads_q"], spec["heads_kv"], spec["head_dim"], spec["dtype"]
    scale = spec["scale"]
    n = t.num_tokens
    log(f"dfs workload {spec['name']}: N={n} nodes={t.num_nodes} hq={hq} hkv={hkv} d={d}")
    x = make_inputs(n, hq, hkv, d, dtype=dtype, do_std=spec["do_std"])

    def up(name):
        if dtype == "bf16":
            a = torch.from_numpy(x.bits[name].view(np.int16)).view(torch.bfloat16)
        else:
            a = torch.from_numpy(getattr(x, name))
        return a.to(dev)

    q, k, v, do = up("q"), up("k"), up("v"), up("do")
    sample = None if args.no_cpu_baseline else _baseline_sample(t, x, d)
    del x
    o = torch.empty_like(q)
    lse = torch.empty((hq, n), dtype=torch.float32, device=dev)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    acc = torch.empty((2, n, hkv, d), dtype=torch.float32, device=dev)
    if args.walk == "node":
        calls = [[i] for i in dfs_preorder(t.parent)]
    else:
        calls = ta.walk_runs(t.parent, t.seg_len)
    log(f"walk: {len(calls)} calls ({args.walk})")
    t0 = time.perf_counter()
    plans = [ta.plan(t.parent, t.seg_start, t.seg_len, n, hq, hkv, d, dtype, query_nodes=c)
             for c in calls]
    torch.cuda.synchronize()
    plan_ms = 1e3 * (time.perf_counter() - t0)
    has_limit = any(bool((p.export()["bwd_entries"][:, 3] < 0).any()) for p in plans)
    ws = torch.empty(max(p.workspace_size()[1] for p in plans), dtype=torch.uint8, device=dev)
    # split query tiles keep their key parts' partial results here
    ws_f = torch.empty(max(1, max(p.workspace_size()[0] for p in plans)), dtype=torch.uint8,
                       device=dev)
    whole = ta.plan(t.parent, t.seg_start, t.seg_len, n, hq, hkv, d, dtype)
    ws_whole = ta.workspace(whole, "bwd")
    ws_whole_f = ta.workspace(whole, "fwd")

    def walk():
        acc.zero_()
        for p in plans:
            ta.fwd(p, q, k, v, scale, o=o, lse=lse, ws=ws_f)
        for p in reversed(plans):
            ta.bwd_accum(p, q, k, v, o, lse, do, scale, acc[0], acc[1], dq=dq, ws=ws)
        ta.accum_cast(acc[0], dtype, out=dk)
        ta.accum_cast(acc[1], dtype, out=dv)

    def one_call():
        ta.fwd(whole, q, k, v, scale, o=o, lse=lse, ws=ws_whole_f)
        ta.bwd(whole, q, k, v, o, lse, do, scale, dq=dq, dk=dk, dv=dv, ws=ws_whole)

    def timed(fn, steps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        return 1e3 * (time.perf_counter() - t0) / steps

    for _ in range(args.warmup):
        walk()
        one_call()
    # both passes timed without per-kernel events (each event pair costs a
    # few microseconds per launch, which a walk of many small calls would
    # feel); the per-kernel split comes from a second, instrumented walk
    ms_one = timed(one_call, args.steps)
    log(f"one call: {ms_one:.3f} ms")
    ms_step = timed(walk, args.steps)
    log(f"walk: {ms_step:.3f} ms")
    ta.timing_read(reset=True)
    ta.timing_enable(True)
    ms_events = timed(walk, args.steps)
    ta.timing_enable(False)
    kt = ta.timing_read(reset=True)
    log(f"walk with per-kernel events: {ms_events:.3f} ms")
    for p in plans + [whole]:
        p.close()

    pairs = st["pairs"]
    peak = PEAK_BF16_TFLOPS if dtype == "bf16" else PEAK_FP32_TFLOPS
    step_flop = 14.0 * d * hq * pairs
    # over a whole walk the kernels do the whole tree's work
    kern_flop = {"fwd": 4.0 * d * hq * pairs, "bwd_dkdv": 8.0 * d * hq * pairs,
                 "bwd_dq": 2.0 * d * hq * pairs}
    kern_exec = {"fwd": 1.0, "bwd_dkdv": 1.0, "bwd_dq": 3.0}
    pipe = dtype == "bf16"
    # key-limit entries (key tiles crossing from a parent into the child
    # stored after it) need the pipelined kernel's other variant
    kern_name = {"fwd": f"tree_attn_fwd_kernel<{'bf16' if pipe else 'float'}, {d}>",
                 "bwd_dkdv": (f"tree_attn_dkdv_pipe_kernel<{d}, {str(has_limit).lower()}>"
                              if pipe
                              else f"tree_attn_dkdv_kernel<float, {d}>"),
                 "bwd_dq": f"tree_attn_dq_kernel<{'bf16' if pipe else 'float'}, {d}>"}

    def roof(kind):
        r = kt[kind]
        walk_ms = r["total_ms"] / args.steps  # every launch of one walk
        ach = kern_flop[kind] / (walk_ms * 1e-3) / 1e12
        return {"bound": "mfma", "kernel": kern_name[kind], "achieved": ach, "peak": peak,
                "unit": "TFLOP/s", "frac": ach / peak,
                "executed_over_counted": kern_exec[kind],
                "flop_per_launch": kern_flop[kind] / len(plans),
                "avg_ms": r["total_ms"] / max(r["launches"], 1), "launches_per_step": len(plans),
                "ms_per_step": walk_ms}

    dominant = max(("fwd", "bwd_dkdv", "bwd_dq"), key=lambda kk: kt[kk]["total_ms"])
    main_roof = roof(dominant)
    main_roof["traffic"] = None
    result = {
        "metric": DFS_METRIC,
        "value": n / (ms_step * 1e-3),
        "unit": "unique tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{spec['name']} tree, depth-first walk, " + (
                "one node per call" if args.walk == "node" else
                f"{len(calls)} calls of preorder runs within the deepest path's rows"),
            "unique_tokens": n, "nodes": t.num_nodes, "pairs": pairs, "heads_q": hq,
            "heads_kv": hkv, "head_dim": d, "softmax_scale": scale, "global_batch": 1,
            "seq_len": st["max_path"], "parallelism": "none (1 GPU)",
        },
        "tflops": step_flop / (ms_step * 1e-3) / 1e12,
        "frac_of_peak": step_flop / (ms_step * 1e-3) / 1e12 / peak,
        "one_call_ms": ms_one,
        "walk_over_one_call": ms_step / ms_one,
        "ms_per_step_with_events": ms_events,
        "plans_ms_host": plan_ms,
        "kernels_ms_per_step": {kk: kt[kk]["total_ms"] / args.steps for kk in kt
                                if kt[kk]["launches"]},
        "roofline": main_roof,
        "roofline_kernels": {kk: roof(kk) for kk in ("fwd", "bwd_dkdv", "bwd_dq")},
    }
    if not args.no_cpu_baseline:
        log("timing the oracle on the host (cpu baseline)")
        result["cpu_baseline"] = cpu_baseline(t, spec, sample)
    print(json.dumps(result), flush=True)
    return 0


def _passes_around_attention(ta, torch, t, o, q, k, pos_id, do, hq, hkv, d, reps=5):
    """The steps either side of the attention call, on the same workload:
    prefix compression of the tree's root-to-leaf trajectories (host), the
    gather of O rows to every trajectory position, the fixed-order sum of
    per-trajectory dO rows onto unique tokens, and rotary embeddings of Q
    and K at tree depth.  Not part of the timed step; rates are HBM bytes
    moved (each row read and written once) per second."""
    n = t.num_tokens
    # trajectories: root-to-leaf paths, token id = unique row
    parent, start, length = t.parent, t.seg_start, t.seg_len
    kids = np.zeros(t.num_nodes, bool)
    kids[parent[parent >= 0]] = True
    trajs = []
    for leaf in np.nonzero(~kids)[0]:
        chain, node = [], int(leaf)
        while node >= 0:
            chain.append(node)
            node = int(parent[node])
        trajs.append(np.concatenate([np.arange(start[c], start[c] + length[c]) for c in chain[::-1]]))
    t0 = time.perf_counter()
    tree = ta.build_tree(trajs)
    build_ms = 1e3 * (time.perf_counter() - t0)
    total = tree.traj_index.shape[0]
    dev = q.device
    tidx = torch.from_numpy(tree.traj_index).to(dev)
    off = torch.from_numpy(tree.inv_offsets).to(dev)
    pos = torch.from_numpy(tree.inv_positions).to(dev)
    row = hq * d * o.element_size()
    o_traj = torch.empty((total, hq, d), dtype=o.dtype, device=dev)
    do_traj = do[tidx]  # per-trajectory upstream gradients (input of the sum)
    do_u = torch.empty_like(do)
    qr, kr = q.clone(), k.clone()

    def passes():
        ta.gather_rows(o, tidx, out=o_traj)
        ta.scatter_sum_rows(do_traj, off, pos, n, out=do_u)
        ta.rope(qr, pos_id)
        ta.rope(kr, pos_id)

    for _ in range(2):  # warm-up: first touch of the new buffers
        passes()
    torch.cuda.synchronize()
    ta.timing_read(reset=True)
    ta.timing_enable(True)
    for _ in range(reps):
        passes()
    torch.cuda.synchronize()
    ta.timing_enable(False)
    kt = ta.timing_read(reset=True)

    def ms(kind):
        r = kt[kind]
        return r["total_ms"] / max(r["launches"], 1)

    rope_bytes = (2 * n * hq * d + 2 * n * hkv * d) * q.element_size() / 2  # per launch, averaged
    return {
        "trajectories": len(trajs), "trajectory_tokens": int(total), "unique_tokens": n,
        "build_tree_ms_host": build_ms,
        "gather_o_GBps": 2 * total * row / (ms("gather") * 1e-3) / 1e9,
        "scatter_sum_do_GBps": (total + n) * row / (ms("scatter_sum") * 1e-3) / 1e9,
        "rope_qk_GBps": rope_bytes / (ms("rope") * 1e-3) / 1e9,
        "ms": {"gather": ms("gather"), "scatter_sum": ms("scatter_sum"), "rope": ms("rope")},
        "peak_GBps": PEAK_HBM_GBS,
    }


def main() -> int:
    args = _args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the path is single-GPU; multi-GPU sharding is design-only)", file=sys.stderr)
        return 2
    if args.workload == "linear":
        return main_linear(args)
    if args.workload == "dfs":
        return main_dfs(args)
    import torch
    import prefix_shared_tree_attn_amd as ta
    from tree_inputs import config_spec, config_tree, make_inputs, tree_stats
    from tree_inputs.tensors import SEEDS as INPUT_SEEDS

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    cfg = args.config
    t = config_tree(cfg)
    spec = config_spec(cfg)
    st = tree_stats(t)
    hq, hkv, d, dtype = spec["heads_q"], spec["heads_kv"], spec["head_dim"], spec["dtype"]
    scale = spec["scale"]
    n = t.num_tokens
    log(f"workload {spec['name']}: N={n} nodes={t.num_nodes} pairs={st['pairs']} "
        f"hq={hq} hkv={hkv} d={d} {dtype}")

    x = make_inputs(n, hq, hkv, d, dtype=dtype, do_std=spec["do_std"])
    log("inputs generated")
    inputs_sha = _inputs_sha256(t, x, dtype)

    def up(name):
        if dtype == "bf16":
            a = torch.from_numpy(x.bits[name].view(np.int16)).view(torch.bfloat16)
        else:
            a = torch.from_numpy(getattr(x, name))
        return a.to(dev)

    q, k, v, do = up("q"), up("k"), up("v"), up("do")
    tdt = q.dtype
    o = torch.empty((n, hq, d), dtype=tdt, device=dev)
    lse = torch.empty((hq, n), dtype=torch.float32, device=dev)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    probe = ta.plan(t.parent, t.seg_start, t.seg_len, n, hq, hkv, d, dtype)
    ws = ta.workspace(probe, "bwd")
    ws_f = ta.workspace(probe, "fwd")  # key parts of split query tiles (small trees)
    pstats = probe.stats()
    # the dK/dV kernel variant with key-limit masks runs when the plan has them
    has_limit = bool((probe.export()["bwd_entries"][:, 3] < 0).any())
    probe.close()
    sample = None if args.no_cpu_baseline else _baseline_sample(t, x, d)
    del x
    log("device buffers ready")

    plans = []

    node_id = torch.empty((n,), dtype=torch.int32, device=dev)
    pos_id = torch.empty((n,), dtype=torch.int32, device=dev)

    def step():
        p = ta.plan(t.parent, t.seg_start, t.seg_len, n, hq, hkv, d, dtype)
        ta.positions(p, node_id=node_id, pos_id=pos_id)
        ta.fwd(p, q, k, v, scale, o=o, lse=lse, ws=ws_f)
        ta.bwd(p, q, k, v, o, lse, do, scale, dq=dq, dk=dk, dv=dv, ws=ws)
        plans.append(p)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    for p in plans:
        p.close()
    plans.clear()
    log(f"warmup done ({args.warmup} steps)")

    ta.timing_read(reset=True)
    ta.timing_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ta.timing_enable(False)
    kt = ta.timing_read(reset=True)
    for p in plans:
        p.close()
    plans.clear()
    log(f"timed {args.steps} steps: {wall:.3f} s")
    # the same steps again without the per-kernel events (a few microseconds
    # per launch), for reference
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall_plain = time.perf_counter() - t0
    for p in plans:
        p.close()
    plans.clear()

    if args.copy_probe_mib > 0:
        # a plain elementwise kernel of known traffic, to calibrate HBM byte
        # counters: reads nb bytes and writes nb bytes
        nb = args.copy_probe_mib << 20
        a = torch.ones(nb // 4, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        torch.mul(a, 1.0, out=b)
        torch.cuda.synchronize()
        log(f"copy probe: {nb} bytes read + {nb} bytes written")

    ms_step = 1e3 * wall / args.steps
    pairs = st["pairs"]
    fwd_flop = 4.0 * d * hq * pairs
    bwd_flop = 10.0 * d * hq * pairs
    step_flop = fwd_flop + bwd_flop
    tflops = step_flop / (ms_step * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if dtype == "bf16" else PEAK_FP32_TFLOPS

    def avg_ms(kind):
        r = kt[kind]
        return r["total_ms"] / max(r["launches"], 1)

    esize = 2 if dtype == "bf16" else 4
    # Algorithmic work of each kernel, 2 D FLOP per (query, key, head) pair
    # and product, counted on the method's own work: the forward forms S and
    # O (4 D); the backward's 10 D split into S, dP, dV and dK in the dK/dV
    # kernel (8 D) and dQ (2 D).  The dQ kernel executes 6 D, because it
    # recomputes S and dP rather than receiving dS through an atomic
    # reduction; the recomputation is reported as executed_over_counted and
    # earns no credit.
    kern_flop = {"fwd": 4.0 * d * hq * pairs, "bwd_dkdv": 8.0 * d * hq * pairs,
                 "bwd_dq": 2.0 * d * hq * pairs}
    kern_exec = {"fwd": 1.0, "bwd_dkdv": 1.0, "bwd_dq": 3.0}
    pipe = dtype == "bf16"
    kern_name = {"fwd": f"tree_attn_fwd_kernel<{'bf16' if pipe else 'float'}, {d}>",
                 "bwd_dkdv": (f"tree_attn_dkdv_pipe_kernel<{d}, {str(has_limit).lower()}>"
                              if pipe else f"tree_attn_dkdv_kernel<float, {d}>"),
                 "bwd_dq": f"tree_attn_dq_kernel<{'bf16' if pipe else 'float'}, {d}>"}

    def roof(kind):
        ach = kern_flop[kind] / (avg_ms(kind) * 1e-3) / 1e12
        return {"bound": "mfma", "kernel": kern_name[kind], "achieved": ach, "peak": peak,
                "unit": "TFLOP/s", "frac": ach / peak, "flop_per_launch": kern_flop[kind],
                "executed_over_counted": kern_exec[kind],
                "executed_frac": ach * kern_exec[kind] / peak, "avg_ms": avg_ms(kind)}

    dominant = max(("fwd", "bwd_dkdv", "bwd_dq"), key=avg_ms)
    main_roof = roof(dominant)
    main_roof["traffic"] = _traffic_from_profile(dominant, spec["name"])
    # HBM-bound passes: the position pass writes node and position ids; the
    # preprocess reads O, dO and LSE and writes -D and -LSE log2 e; the
    # reduction reads the fp32 partial slots and writes the split tiles' dK
    # and dV
    pre_bytes = n * hq * d * 2 * esize + 3 * n * hq * 4
    red_bytes = 2 * pstats["bwd_slots"] * 128 * d * 4 + 2 * pstats["bwd_split_tiles"] * 128 * d * esize
    workload = spec["name"]
    result = {
        "metric": METRIC,
        "value": n / (ms_step * 1e-3),
        "unit": "unique tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "ms_per_step_without_events": 1e3 * wall_plain / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{workload}: " + {
                1: "binary tree, root 32 + 3 levels of 16-token segments",
                2: "GRPO star, 1024-token prompt + 16 x 2048-token responses",
                3: "irregular 8-level agent tree, ~32K tokens",
                4: "segment search tree, 512-token segments, 6 binary levels",
                5: "32768-token trunk + 64 x 2048-token branches"}[cfg],
            "unique_tokens": n, "nodes": t.num_nodes, "pairs": pairs,
            "heads_q": hq, "heads_kv": hkv, "head_dim": d, "softmax_scale": scale,
            "global_batch": 1, "seq_len": st["max_path"], "parallelism": "none (1 GPU)",
        },
        "inputs": {"tensor_seeds": dict(INPUT_SEEDS), "tree_seed": 0,
                   "sha256": inputs_sha},
        "tflops": tflops,
        "frac_of_peak": tflops / peak,
        "dense_per_path_flop_ratio": st["dense_ratio"],
        "kernels_ms": {kk: avg_ms(kk) for kk in kt if kt[kk]["launches"]},
        "roofline": main_roof,
        "roofline_kernels": {k: roof(k) for k in ("fwd", "bwd_dkdv", "bwd_dq")},
        "hbm_passes_GBps": {
            "positions": 8 * n / (avg_ms("positions") * 1e-3) / 1e9,
            # bf16: the dQ kernel computes the row terms (no separate launch)
            "bwd_pre": (pre_bytes / (avg_ms("bwd_pre") * 1e-3) / 1e9
                        if kt["bwd_pre"]["launches"] else None),
            "bwd_reduce": (red_bytes / (avg_ms("bwd_reduce") * 1e-3) / 1e9
                           if kt["bwd_reduce"]["launches"] else None),
            "peak": PEAK_HBM_GBS,
        },
        "plan": {k: pstats[k] for k in ("fwd_tiles", "bwd_items", "bwd_split_tiles", "bwd_slots")},
    }
    result["next_rows"] = _passes_around_attention(ta, torch, t, o, q, k, pos_id, do, hq, hkv, d)
    if not args.no_cpu_baseline:
        log("timing the oracle on the host (cpu baseline)")
        result["cpu_baseline"] = cpu_baseline(t, spec, sample)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
