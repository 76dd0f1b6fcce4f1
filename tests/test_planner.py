"""Host-side tests of libtree_attn.so: exports, validation and the planner.

These run without a GPU: tree_attn_plan_host validates and plans on the CPU
and the plan's work arrays are exported and checked here against the
ancestor relation computed independently in Python.
"""

import ctypes
import os
import re

import numpy as np
import pytest

import prefix_shared_tree_attn_amd as ta
from prefix_shared_tree_attn_amd import _ffi
from tree_inputs import (NodeTable, binary_tree, caterpillar_tree, chain_tree, config_tree,
                         dfs_preorder, random_tree, star_tree, tree_stats)

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "tree_attn.h")


def test_library_exports_every_declared_symbol():
    text = open(HEADER).read()
    declared = set(re.findall(r"\b(tree_attn_[a-z_]+)\s*\(", text))
    assert declared == set(_ffi.EXPORTS)
    lib = _ffi.lib()
    for name in declared:
        assert hasattr(lib, name), name


def _visible(t: NodeTable):
    """Set of (q, key) pairs: key is in an ancestor node of q's node, or in
    q's node at or before q (built from parent pointers directly)."""
    m = t.num_nodes
    node_of = np.empty(t.num_tokens, np.int64)
    for i in range(m):
        node_of[t.seg_start[i]:t.seg_start[i] + t.seg_len[i]] = i
    anc = [set() for _ in range(m)]
    for i in range(m):
        a = int(t.parent[i])
        while a >= 0:
            anc[i].add(a)
            a = int(t.parent[a])
    vis = set()
    for q in range(t.num_tokens):
        n = int(node_of[q])
        for a in anc[n]:
            for key in range(int(t.seg_start[a]), int(t.seg_start[a] + t.seg_len[a])):
                vis.add((q, key))
        for key in range(int(t.seg_start[n]), q + 1):
            vis.add((q, key))
    return vis


def _fwd_pairs(ex, hq, hkv):
    pairs = {}
    for q0, q1, rb, re_ in ex["fwd_tiles"]:
        for k0, k1, causal, _ in ex["fwd_ranges"][rb:re_]:
            for q in range(q0, q1):
                for key in range(k0, k1):
                    if causal and key > q:
                        continue
                    pairs[(q, key)] = pairs.get((q, key), 0) + 1
    return pairs


def _bwd_triples(ex):
    trip = {}
    for it in ex["bwd_items"]:
        k0, k1, g, eb, ee = it[:5]
        for h, q0, q1, mask in ex["bwd_entries"][eb:ee]:
            # mask 1: causal (key <= row); 0: every key; -(limit + 1): keys < limit
            klim = -int(mask) - 1 if mask < 0 else k1
            for q in range(q0, q1):
                for key in range(k0, min(k1, klim)):
                    if mask == 1 and key > q:
                        continue
                    trip[(q, key, h)] = trip.get((q, key, h), 0) + 1
    return trip


def _trees():
    rng = np.random.default_rng(0)
    out = [chain_tree([5]), chain_tree([130, 1, 200]), star_tree(100, 3, 150),
           binary_tree(40, 70, 3), config_tree(1)]
    for seed in range(6):
        r = np.random.default_rng(seed)
        out.append(random_tree(r, int(r.integers(1, 14)), max_len=300,
                               n_roots=int(r.integers(1, 3))))
    return out


@pytest.mark.parametrize("idx", range(11))
def test_plan_covers_every_visible_pair_once(idx):
    t = _trees()[idx]
    hq, hkv = 4, 2
    p = ta.plan_host(t.parent, t.seg_start, t.seg_len, t.num_tokens, hq, hkv, 64, "bf16",
                     num_cus=4)
    ex = p.export()
    vis = _visible(t)
    fp = _fwd_pairs(ex, hq, hkv)
    assert set(fp) == vis and set(fp.values()) == {1}
    bt = _bwd_triples(ex)
    want = {(q, key, h) for (q, key) in vis for h in range(hq)}
    assert set(bt) == want and set(bt.values()) == {1}
    # every backward item's heads belong to its kv head
    for it in ex["bwd_items"]:
        hs = ex["bwd_entries"][it[3]:it[4], 0]
        assert np.all(hs // (hq // hkv) == it[2])
    st = p.stats()
    assert st["pairs"] == tree_stats(t)["pairs"] == len(vis)


def test_forward_block_mapping_covers_tiles_and_heads_once():
    """The forward launch maps workgroup b to (tile, head) as: slot = b / 8,
    group = (slot / G) * 8 + b % 8, tile = group / Hkv, head = (group % Hkv) * G
    + slot % G; every (tile, head) must come up exactly once."""
    t = binary_tree(100, 90, 3)
    for hq, hkv in ((28, 4), (8, 8), (3, 1)):
        p = ta.plan_host(t.parent, t.seg_start, t.seg_len, t.num_tokens, hq, hkv, 128)
        st = p.stats()
        gs = hq // hkv
        ngroups = st["fwd_tiles"] * hkv
        seen = {}
        for b in range(st["fwd_blocks"]):
            slot = b // 8
            gi = (slot // gs) * 8 + b % 8
            if gi >= ngroups:
                continue
            key = (gi // hkv, (gi % hkv) * gs + slot % gs)
            seen[key] = seen.get(key, 0) + 1
        assert set(seen) == {(ti, h) for ti in range(st["fwd_tiles"]) for h in range(hq)}
        assert set(seen.values()) == {1}


def test_item_placement_and_split_heavy_tiles():
    t = config_tree(2)  # star: the prompt's key tiles are seen by every response
    p = ta.plan_host(t.parent, t.seg_start, t.seg_len, t.num_tokens, 32, 8, 128)
    ex = p.export()
    st = p.stats()
    assert st["bwd_split_tiles"] > 0 and st["bwd_slots"] > 0
    items, ent = ex["bwd_items"], ex["bwd_entries"]
    load = np.zeros(8)
    queues = [[] for _ in range(8)]
    for b, it in enumerate(items):
        if it[3] == it[4]:  # padding: no work, no slot
            assert it[5] == -1 and it[6] == -1
            continue
        assert it[6] == b % 8  # workgroup b runs on XCD b % 8
        rows = int((ent[it[3]:it[4], 2] - ent[it[3]:it[4], 1]).sum())
        load[b % 8] += rows * int(it[1] - it[0])
        queues[b % 8].append(it)
    assert load.max() <= 1.05 * load.mean()
    # the key tiles of one response node and kv head read the same rows: they
    # all sit on one XCD
    prompt = int(t.seg_len[0])
    where = {}
    for x, q in enumerate(queues):
        for it in q:
            if it[0] >= prompt:
                where.setdefault((int((it[0] - prompt) // 2048), int(it[2])), set()).add(x)
    assert len(where) == 16 * 8 and all(len(xs) == 1 for xs in where.values())
    fcost = []
    for q0, q1, rb, re_ in ex["fwd_tiles"]:
        keys = sum(int(k1 - k0) for k0, k1, _, _ in ex["fwd_ranges"][rb:re_])
        fcost.append((q1 - q0) * keys)
    assert all(a >= b for a, b in zip(fcost, fcost[1:]))
    # split chunks of one key tile carry distinct slots; unsplit items use -1
    slots = ex["bwd_items"][:, 5]
    assert len(set(slots[slots >= 0])) == st["bwd_slots"]


def test_workspace_size():
    t = config_tree(2)
    p = ta.plan_host(t.parent, t.seg_start, t.seg_len, t.num_tokens, 32, 8, 128)
    f, b = p.workspace_size()
    st = p.stats()
    n = t.num_tokens
    al = lambda x: (x + 255) // 256 * 256
    slot = st["bwd_slots"] * 128 * 128 * 4
    assert f == 0
    assert b == 2 * al(n * 32 * 4) + 2 * al(slot)


def test_empty_tree():
    p = ta.plan_host([], [], [], 0, 2, 1, 64)
    st = p.stats()
    assert st["num_tokens"] == 0 and st["fwd_tiles"] == 0 and st["bwd_items"] == 0
    assert p.workspace_size() == (0, 0)


@pytest.mark.parametrize("parent,start,length,n,hq,hkv,d,dtype,status", [
    ([-1, 5], [0, 4], [4, 4], 8, 1, 1, 64, "bf16", "BAD_TREE"),      # parent out of range
    ([-1, 1], [0, 4], [4, 4], 8, 1, 1, 64, "bf16", "BAD_TREE"),      # self loop
    ([2, 0, 1], [0, 4, 8], [4, 4, 4], 12, 1, 1, 64, "bf16", "BAD_TREE"),  # cycle
    ([-1, 0], [0, 3], [4, 4], 8, 1, 1, 64, "bf16", "LAYOUT"),        # overlap
    ([-1, 0], [0, 5], [4, 4], 9, 1, 1, 64, "bf16", "LAYOUT"),        # gap
    ([-1, 0], [0, 4], [4, 0], 8, 1, 1, 64, "bf16", "LAYOUT"),        # empty segment
    ([-1, 0], [0, 4], [4, 4], 9, 1, 1, 64, "bf16", "LAYOUT"),        # uncovered tail
    ([-1, 0], [0, 4], [4, 5], 8, 1, 1, 64, "bf16", "LAYOUT"),        # past the end
    ([-1], [0], [4], 4, 3, 2, 64, "bf16", "UNSUPPORTED"),            # Hq % Hkv
    ([-1], [0], [4], 4, 2, 1, 96, "bf16", "UNSUPPORTED"),            # head_dim
    ([-1], [0], [4], 4, 0, 1, 64, "bf16", "UNSUPPORTED"),            # no heads
    ([], [], [], 4, 1, 1, 64, "bf16", "LAYOUT"),                     # tokens, no nodes
])
def test_validation_errors(parent, start, length, n, hq, hkv, d, dtype, status):
    with pytest.raises(ta.TreeAttnError) as ei:
        ta.plan_host(parent, start, length, n, hq, hkv, d, dtype)
    assert ei.value.status == status
    assert len(str(ei.value)) > len(status) + 10  # carries a detail message


def test_raw_abi_rejects_null_and_negative():
    lib = _ffi.lib()
    h = ctypes.c_void_p(0)
    st = lib.tree_attn_plan_host(None, None, None, 2, 8, 1, 1, 64, 0, 0, ctypes.byref(h))
    assert _ffi.STATUS[st] == "INVALID_ARG"
    one = (ctypes.c_int32 * 1)(0)
    st = lib.tree_attn_plan_host(one, one, one, -1, 8, 1, 1, 64, 0, 0, ctypes.byref(h))
    assert _ffi.STATUS[st] == "INVALID_ARG"
    st = lib.tree_attn_plan_host(one, one, one, 1, 8, 1, 1, 64, 7, 0, ctypes.byref(h))
    assert _ffi.STATUS[st] == "UNSUPPORTED"
    assert lib.tree_attn_workspace_size(None, None, None) == 1
    assert lib.tree_attn_status_string(3) == b"invalid segment layout"
    lib.tree_attn_plan_destroy(None)  # ignored


def test_host_plan_rejected_by_fwd():
    t = chain_tree([8])
    p = ta.plan_host(t.parent, t.seg_start, t.seg_len, 8, 1, 1, 64)
    lib = _ffi.lib()
    # well-formed arguments (addresses that are never dereferenced: the
    # device check fails first) reach the device check
    a = [ctypes.c_void_p(0x10000 + 0x1000 * i) for i in range(5)]
    st = lib.tree_attn_fwd(p.handle, a[0], a[1], a[2], ctypes.c_float(1.0), a[3], a[4], None, 0,
                           None)
    assert _ffi.STATUS[st] == "NO_DEVICE_PLAN"
    st = lib.tree_attn_positions(p.handle, None, None, None)
    assert _ffi.STATUS[st] == "NO_DEVICE_PLAN"


def _fake(n, misaligned=()):
    """n distinct fake device addresses, 16-byte aligned except the listed
    positions (8 bytes off).  Argument checks reject them before any device
    work, so they are never dereferenced."""
    return [ctypes.c_void_p(0x100000 + 0x1000 * i + (8 if i in misaligned else 0))
            for i in range(n)]


@pytest.mark.parametrize("bad", range(5))
def test_fwd_rejects_misaligned_tensors_before_any_launch(bad):
    t = chain_tree([8])
    p = ta.plan_host(t.parent, t.seg_start, t.seg_len, 8, 1, 1, 64)
    lib = _ffi.lib()
    a = _fake(5, misaligned=(bad,))
    st = lib.tree_attn_fwd(p.handle, a[0], a[1], a[2], ctypes.c_float(0.125), a[3], a[4], None,
                           0, None)
    assert _ffi.STATUS[st] == "INVALID_ARG"
    assert b"16-byte" in lib.tree_attn_last_error()


@pytest.mark.parametrize("bad", range(9))
def test_bwd_rejects_misaligned_tensors_before_any_launch(bad):
    t = chain_tree([8])
    p = ta.plan_host(t.parent, t.seg_start, t.seg_len, 8, 1, 1, 64)
    lib = _ffi.lib()
    a = _fake(9, misaligned=(bad,))  # q, k, v, o, lse, dout, dq, dk, dv
    ws = ctypes.c_void_p(0x900000)
    st = lib.tree_attn_bwd(p.handle, a[0], a[1], a[2], a[3], a[4], a[5], ctypes.c_float(0.125),
                           a[6], a[7], a[8], ws, 1 << 20, None)
    assert _ffi.STATUS[st] == "INVALID_ARG"
    assert b"16-byte" in lib.tree_attn_last_error()
    good = _fake(9)
    st = lib.tree_attn_bwd(p.handle, good[0], good[1], good[2], good[3], good[4], good[5],
                           ctypes.c_float(0.125), good[6], good[7], good[8], ws, 1 << 20, None)
    assert _ffi.STATUS[st] == "NO_DEVICE_PLAN"


@pytest.mark.parametrize("scale", [0.0, -0.125, float("inf"), float("nan"), -0.0])
def test_softmax_scale_must_be_positive(scale):
    """Scores are masked with -inf and scaled afterwards, and the forward's
    row max is taken on unscaled scores: a scale <= 0 or not finite is
    rejected by the forward, the backward and the accumulating backward."""
    t = chain_tree([8])
    lib = _ffi.lib()
    p = ta.plan_host(t.parent, t.seg_start, t.seg_len, 8, 1, 1, 64)
    a = _fake(9)
    st = lib.tree_attn_fwd(p.handle, a[0], a[1], a[2], ctypes.c_float(scale), a[3], a[4], None,
                           0, None)
    assert _ffi.STATUS[st] == "INVALID_ARG"
    ws = ctypes.c_void_p(0x900000)
    st = lib.tree_attn_bwd(p.handle, a[0], a[1], a[2], a[3], a[4], a[5], ctypes.c_float(scale),
                           a[6], a[7], a[8], ws, 1 << 20, None)
    assert _ffi.STATUS[st] == "INVALID_ARG"
    ps = ta.plan_host(t.parent, t.seg_start, t.seg_len, 8, 1, 1, 64, query_nodes=[0])
    st = lib.tree_attn_bwd_accum(ps.handle, a[0], a[1], a[2], a[3], a[4], a[5],
                                 ctypes.c_float(scale), a[6], a[7], a[8], ws, 1 << 20, None)
    assert _ffi.STATUS[st] == "INVALID_ARG"
    assert b"softmax_scale" in lib.tree_attn_last_error()


def test_config_plans_build_quickly():
    for i in (1, 2, 3, 4, 5):
        t = config_tree(i)
        from tree_inputs import config_spec
        sp = config_spec(i)
        p = ta.plan_host(t.parent, t.seg_start, t.seg_len, t.num_tokens, sp["heads_q"],
                         sp["heads_kv"], sp["head_dim"], sp["dtype"])
        st = p.stats()
        assert st["pairs"] == tree_stats(t)["pairs"]
        assert st["fwd_tiles"] > 0 and st["bwd_items"] > 0


# ------------------------------------------------ query-subset plans (depth-first walk)

def _row_nodes(t):
    node_of = np.empty(t.num_tokens, np.int64)
    for i in range(t.num_nodes):
        node_of[t.seg_start[i]:t.seg_start[i] + t.seg_len[i]] = i
    return node_of


@pytest.mark.parametrize("idx", range(11))
def test_subset_plan_covers_its_query_pairs_once(idx):
    t = _trees()[idx]
    hq, hkv = 4, 2
    rng = np.random.default_rng(40 + idx)
    node_of = _row_nodes(t)
    vis = _visible(t)
    subsets = [[int(rng.integers(t.num_nodes))],
               list(rng.choice(t.num_nodes, size=max(1, t.num_nodes // 2), replace=False)),
               list(range(t.num_nodes)), []]
    for qn in subsets:
        p = ta.plan_host(t.parent, t.seg_start, t.seg_len, t.num_tokens, hq, hkv, 64, "bf16",
                         num_cus=4, query_nodes=qn + qn[:1])  # a repeat is ignored
        ex = p.export()
        want = {(q, key) for (q, key) in vis if node_of[q] in set(qn)}
        fp = _fwd_pairs(ex, hq, hkv)
        assert set(fp) == want and set(fp.values()) <= {1}
        bt = _bwd_triples(ex)
        assert set(bt) == {(q, key, h) for (q, key) in want for h in range(hq)}
        assert set(bt.values()) <= {1}
        st = p.stats()
        assert st["subset"] == 1
        assert st["pairs"] == len(want)
        assert st["query_rows"] == int(sum(t.seg_len[i] for i in set(qn)))
        # every working item writes fp32 slots (the reduction adds them into
        # the caller's accumulators); slots are distinct
        work = ex["bwd_items"][ex["bwd_items"][:, 3] < ex["bwd_items"][:, 4]]
        assert np.all(work[:, 5] >= 0)
        assert len(set(work[:, 5].tolist())) == len(work) == st["bwd_slots"]
        assert st["bwd_split_tiles"] == len({(int(a), int(g)) for a, g in work[:, [0, 2]]})


def test_whole_tree_plan_is_not_a_subset():
    t = binary_tree(40, 70, 3)
    st = ta.plan_host(t.parent, t.seg_start, t.seg_len, t.num_tokens, 4, 2, 64).stats()
    assert st["subset"] == 0 and st["query_rows"] == t.num_tokens


def test_subset_plan_rejects_bad_nodes():
    t = binary_tree(10, 10, 2)
    for bad in ([t.num_nodes], [-1]):
        with pytest.raises(ta.TreeAttnError) as ei:
            ta.plan_host(t.parent, t.seg_start, t.seg_len, t.num_tokens, 2, 1, 64,
                         query_nodes=bad)
        assert ei.value.status == "INVALID_ARG"
    lib = _ffi.lib()
    h = ctypes.c_void_p(0)
    par = np.ascontiguousarray(t.parent, np.int32)
    ss = np.ascontiguousarray(t.seg_start, np.int32)
    sl = np.ascontiguousarray(t.seg_len, np.int32)
    P = ctypes.POINTER(ctypes.c_int32)
    st = lib.tree_attn_plan_host_subset(par.ctypes.data_as(P), ss.ctypes.data_as(P),
                                        sl.ctypes.data_as(P), t.num_nodes, t.num_tokens, 2, 1,
                                        64, 0, None, 3, 0, ctypes.byref(h))
    assert _ffi.STATUS[st] == "INVALID_ARG"


def test_subset_plan_calls_are_checked_on_the_host():
    """A host-only subset plan still reaches the argument checks of the
    accumulating backward and the cast, which need no GPU to fail."""
    lib = _ffi.lib()
    assert _ffi.STATUS[lib.tree_attn_accum_cast(None, None, -1, 0, None)] == "INVALID_ARG"
    assert _ffi.STATUS[lib.tree_attn_accum_cast(None, None, 0, 0, None)] == "OK"
    assert _ffi.STATUS[lib.tree_attn_accum_cast(None, None, 4, 0, None)] == "INVALID_ARG"
    t = chain_tree([8])
    p = ta.plan_host(t.parent, t.seg_start, t.seg_len, 8, 1, 1, 64, query_nodes=[0])
    st = lib.tree_attn_bwd_accum(p.handle, *([None] * 6), ctypes.c_float(1.0), None, None, None,
                                 None, 0, None)
    assert _ffi.STATUS[st] == "INVALID_ARG"  # null tensors, before the device check
    a = _fake(9)
    st = lib.tree_attn_bwd_accum(p.handle, a[0], a[1], a[2], a[3], a[4], a[5],
                                 ctypes.c_float(1.0), a[6], a[7], a[8], ctypes.c_void_p(0x900000),
                                 1 << 20, None)
    assert _ffi.STATUS[st] == "NO_DEVICE_PLAN"


def test_key_and_query_tiles_cross_node_boundaries_inside_runs():
    """A first child stored right after its parent continues the parent's
    run: query tiles and key tiles tile the run, not each node, and the
    parent's other children get key-limit entries for the tile that crosses
    the boundary."""
    t = star_tree(300, 5, 257)  # prompt 300, first response stored at 300
    hq, hkv = 2, 1
    p = ta.plan_host(t.parent, t.seg_start, t.seg_len, t.num_tokens, hq, hkv, 128, num_cus=4)
    ex = p.export()
    run = 300 + 257
    qt = [tuple(x) for x in ex["fwd_tiles"][:, :2].tolist()]
    assert sum(1 for q0, q1 in qt if q1 <= run) == -(-run // 128)
    assert (256, 384) in qt  # one query tile spans the prompt's end
    work = ex["bwd_items"][ex["bwd_items"][:, 3] < ex["bwd_items"][:, 4]]
    kt = {(int(a), int(b)) for a, b in work[:, :2]}
    assert sum(1 for k0, k1 in kt if k1 <= run) == -(-run // 128)
    assert (256, 384) in kt
    lim = ex["bwd_entries"][ex["bwd_entries"][:, 3] < 0]
    assert len(lim) > 0 and set((-lim[:, 3] - 1).tolist()) == {300}
    # those rows are the other four responses (stored after the first)
    assert int(lim[:, 1].min()) >= run and int(lim[:, 2].max()) <= t.num_tokens


def test_caterpillar_tiles_span_many_nodes():
    """A trunk of 1-3 token nodes, each with a leaf: one key tile spans dozens
    of trunk nodes and carries a key-limit entry per leaf below them; every
    (query, key, head) is still covered exactly once."""
    rng = np.random.default_rng(4)
    t = caterpillar_tree([int(x) for x in rng.integers(1, 4, 150)], 5)
    hq, hkv = 2, 1
    p = ta.plan_host(t.parent, t.seg_start, t.seg_len, t.num_tokens, hq, hkv, 64, num_cus=4)
    ex = p.export()
    vis = _visible(t)
    fp = _fwd_pairs(ex, hq, hkv)
    assert set(fp) == vis and set(fp.values()) == {1}
    bt = _bwd_triples(ex)
    assert set(bt) == {(q, key, h) for (q, key) in vis for h in range(hq)}
    assert set(bt.values()) == {1}
    trunk = int(t.seg_len[:150].sum())
    # the deepest leaf is stored right after the trunk and continues its run;
    # every other leaf is a run of its own
    assert len(ex["fwd_tiles"]) == -(-(trunk + 5) // 128) + 149
    assert int((ex["bwd_entries"][:, 3] < 0).sum()) > 100


def _key_intervals(ex, tiles):
    """(k0, k1, causal) intervals of the given forward tiles, sorted, with
    adjacent intervals of equal causality merged."""
    iv = sorted((int(k0), int(k1), int(c)) for i in tiles
                for k0, k1, c, _ in ex["fwd_ranges"][ex["fwd_tiles"][i][2]:ex["fwd_tiles"][i][3]])
    out = []
    for k0, k1, c in iv:
        if out and out[-1][1] == k0 and out[-1][2] == c:
            out[-1] = (out[-1][0], k1, c)
        else:
            out.append((k0, k1, c))
    return out


SPLIT_TREES = {
    "chain": chain_tree([3500, 300]),
    "star": star_tree(3200, 3, 200),
    "binary": binary_tree(2000, 400, 3),
    "caterpillar": caterpillar_tree([1200, 1100, 1000, 900], 150),
}


@pytest.mark.parametrize("name", list(SPLIT_TREES))
@pytest.mark.parametrize("subset", [False, True])
def test_split_forward_tiles(name, subset):
    """A plan whose (query tile, head) workgroups would leave CUs idle
    cuts the keys of its long query tiles into parts of at least
    kFwdMinPartSteps steps: each split query tile's parts are the tiles with
    its rows and its consecutive slots, together they hold exactly the keys of
    the unsplit tile (the plan for a one-CU chip, which never splits), the
    parts share the tile's key steps evenly, and the forward and backward
    workspaces hold the parts' fp32 partial results."""
    t = SPLIT_TREES[name]
    hq, hkv, d = 2, 1, 64
    qn = [t.num_nodes - 1] if subset else None
    p = ta.plan_host(t.parent, t.seg_start, t.seg_len, t.num_tokens, hq, hkv, d, "bf16",
                     query_nodes=qn)
    whole = ta.plan_host(t.parent, t.seg_start, t.seg_len, t.num_tokens, hq, hkv, d, "bf16",
                         num_cus=1, query_nodes=qn)
    ex, st = p.export(), p.stats()
    ew = whole.export()
    assert st["fwd_split_tiles"] > 0 and whole.stats()["fwd_split_tiles"] == 0
    part, comb = ex["fwd_part"], ex["fwd_combine"]
    assert comb.shape == (st["fwd_split_tiles"], 4)
    assert sorted(part[part >= 0].tolist()) == list(range(st["fwd_slots"]))
    by_rows = {tuple(int(x) for x in ew["fwd_tiles"][i][:2]): i
               for i in range(len(ew["fwd_tiles"]))}
    split_rows = set()
    for q0, q1, s0, ns in comb:
        assert ns >= 2
        idx_t = np.nonzero((part >= s0) & (part < s0 + ns))[0]
        assert len(idx_t) == ns
        assert all(tuple(ex["fwd_tiles"][i][:2]) == (q0, q1) for i in idx_t)
        assert _key_intervals(ex, idx_t) == _key_intervals(ew, [by_rows[(int(q0), int(q1))]])
        steps = []
        for i in idx_t:
            rb, re_ = ex["fwd_tiles"][i][2:]
            steps.append(sum((k1 - k0 + 63) // 64 for k0, k1, _, _ in ex["fwd_ranges"][rb:re_]))
        assert min(steps) >= 16 and max(steps) - min(steps) <= 1
        split_rows.add((int(q0), int(q1)))
    # the unsplit tiles are the whole plan's other tiles, unchanged
    rest = sorted(tuple(int(x) for x in ex["fwd_tiles"][i][:2]) for i in np.nonzero(part < 0)[0])
    assert rest == sorted(r for r in by_rows if r not in split_rows)
    for i in np.nonzero(part < 0)[0]:
        r = tuple(int(x) for x in ex["fwd_tiles"][i][:2])
        assert _key_intervals(ex, [i]) == _key_intervals(ew, [by_rows[r]])
    f, b = p.workspace_size()
    al = lambda x: (x + 255) // 256 * 256
    rows = st["fwd_slots"] * hq * 128
    assert f == al(rows * d * 4) + al(rows * 2 * 4)
    n = t.num_tokens
    slot = st["bwd_slots"] * 128 * d * 4
    assert b == 2 * al(n * hq * 4) + 2 * al(slot) + al(rows * d * 4)


def test_large_plans_do_not_split_forward_tiles():
    for cfg, hq, hkv in ((2, 32, 8), (4, 28, 4)):
        t = config_tree(cfg)
        p = ta.plan_host(t.parent, t.seg_start, t.seg_len, t.num_tokens, hq, hkv, 128)
        ex, st = p.export(), p.stats()
        assert st["fwd_split_tiles"] == 0 and st["fwd_slots"] == 0
        assert np.all(ex["fwd_part"] == -1)
        assert p.workspace_size()[0] == 0


# ---- runs of a memory-bounded depth-first walk (tree_attn_walk_runs)

def _root_path(parent, v):
    s = set()
    while v >= 0:
        s.add(int(v))
        v = int(parent[v])
    return s


def _greedy_runs(parent, seg_len, budget):
    """The cut written out with sets: walk the preorder, keep the union of
    the current run's root paths, and open a new run when the next node's
    path would take it past the budget."""
    order = dfs_preorder(parent)
    tok = lambda nodes: sum(int(seg_len[u]) for u in nodes)
    if budget <= 0:
        budget = max((tok(_root_path(parent, v)) for v in order), default=0)
    runs, cur, res = [], [], set()
    for v in order:
        grown = res | _root_path(parent, v)
        if cur and tok(grown) > budget:
            runs.append(cur)
            cur, res = [v], _root_path(parent, v)
        else:
            cur.append(v)
            res = grown
    if cur:
        runs.append(cur)
    return runs, budget


def _walk_trees():
    rng = np.random.default_rng(77)
    trees = [("chain", chain_tree([5, 1, 9])), ("star", star_tree(300, 5, 257)),
             ("binary", binary_tree(129, 97, 3)),
             ("caterpillar", caterpillar_tree([1 + (7 * i) % 3 for i in range(40)], 5))]
    for i in range(12):
        trees.append((f"random-{i}", random_tree(rng, int(rng.integers(1, 40)),
                                                 max_len=int(rng.choice([3, 50, 400])), min_len=1,
                                                 n_roots=int(rng.integers(1, 4)),
                                                 shuffle=bool(i % 2))))
    trees += [(f"config-{c}", config_tree(c)) for c in (2, 3, 4, 5)]
    return trees


WALK_TREES = _walk_trees()


@pytest.mark.parametrize("idx", range(len(WALK_TREES)))
def test_walk_runs_follow_the_greedy_cut(idx):
    name, t = WALK_TREES[idx]
    seg = np.asarray(t.seg_len)
    longest = max(sum(int(seg[u]) for u in _root_path(t.parent, v)) for v in range(t.num_nodes))
    for budget in (0, 1, longest // 2, longest, 3 * longest, 1 << 40):
        got = ta.walk_runs(t.parent, t.seg_len, budget)
        want, used = _greedy_runs(t.parent, t.seg_len, budget)
        assert got == want, (name, budget)
        # a partition of the preorder into consecutive runs
        assert [v for r in got for v in r] == dfs_preorder(t.parent)
        for r in got:
            res = set().union(*(_root_path(t.parent, v) for v in r))
            rt = sum(int(seg[u]) for u in res)
            # within the budget, or one node whose own path is longer
            assert rt <= used or len(r) == 1, (name, budget, r)
        # no two neighbouring runs could have been one
        for a, b in zip(got, got[1:]):
            res = set().union(*(_root_path(t.parent, v) for v in a + b[:1]))
            assert sum(int(seg[u]) for u in res) > used
    # the default budget keeps a run's resident rows within the deepest path
    assert _greedy_runs(t.parent, t.seg_len, 0)[1] == longest
    assert len(ta.walk_runs(t.parent, t.seg_len, 1)) == t.num_nodes
    assert len(ta.walk_runs(t.parent, t.seg_len, 1 << 40)) == 1


def test_walk_runs_on_the_grpo_star():
    """Prompt and first response fill the deepest path; every later
    response shares the prompt and runs on its own."""
    t = config_tree(2)
    runs = ta.walk_runs(t.parent, t.seg_len)
    assert runs[0] == [0, 1] and all(len(r) == 1 for r in runs[1:])
    assert len(runs) == t.num_nodes - 1


@pytest.mark.parametrize("parent,seg_len,status", [
    ([1, 0], [2, 3], "BAD_TREE"),        # a cycle
    ([-1, 5], [2, 3], "BAD_TREE"),       # parent out of range
    ([-1, 1], [2, 3], "BAD_TREE"),       # its own parent
    ([-2, 0], [2, 3], "BAD_TREE"),
    ([-1, 0], [2, 0], "LAYOUT"),         # an empty segment
])
def test_walk_runs_rejects_bad_tables(parent, seg_len, status):
    with pytest.raises(ta.TreeAttnError) as ei:
        ta.walk_runs(parent, seg_len)
    assert ei.value.status == status


def test_walk_runs_raw_abi():
    lib = _ffi.lib()
    two = (ctypes.c_int32 * 2)(-1, 0)
    lens = (ctypes.c_int32 * 2)(4, 4)
    order = (ctypes.c_int32 * 2)()
    starts = (ctypes.c_int32 * 3)()
    runs = ctypes.c_int32(-1)
    st = lib.tree_attn_walk_runs(None, lens, 2, 0, order, starts, ctypes.byref(runs))
    assert _ffi.STATUS[st] == "INVALID_ARG"
    st = lib.tree_attn_walk_runs(two, lens, -1, 0, order, starts, ctypes.byref(runs))
    assert _ffi.STATUS[st] == "INVALID_ARG"
    st = lib.tree_attn_walk_runs(two, lens, 2, 0, order, starts, None)
    assert _ffi.STATUS[st] == "INVALID_ARG"
    st = lib.tree_attn_walk_runs(two, lens, 2, 0, order, starts, ctypes.byref(runs))
    assert _ffi.STATUS[st] == "OK" and runs.value == 1
    assert list(order) == [0, 1] and list(starts)[:2] == [0, 2]
    # an empty table: no runs
    st = lib.tree_attn_walk_runs(None, None, 0, 0, None, starts, ctypes.byref(runs))
    assert _ffi.STATUS[st] == "OK" and runs.value == 0 and starts[0] == 0
    assert ta.walk_runs([], []) == []


# ---- randomised coverage: forests, query subsets, CU counts

def _visible_matrix(t: NodeTable, rows_mask):
    """V[q, key] = 1 where query row q (a row of a listed node) sees key."""
    n = t.num_tokens
    node_of = np.empty(n, np.int64)
    for i in range(t.num_nodes):
        node_of[t.seg_start[i]:t.seg_start[i] + t.seg_len[i]] = i
    v = np.zeros((n, n), np.int32)
    for q in np.nonzero(rows_mask)[0]:
        nd = int(node_of[q])
        a = int(t.parent[nd])
        while a >= 0:
            v[q, t.seg_start[a]:t.seg_start[a] + t.seg_len[a]] = 1
            a = int(t.parent[a])
        v[q, t.seg_start[nd]:q + 1] = 1
    return v


def _check_cover(t: NodeTable, hq, hkv, num_cus, query_nodes):
    n = t.num_tokens
    p = ta.plan_host(t.parent, t.seg_start, t.seg_len, n, hq, hkv, 64, "bf16", num_cus=num_cus,
                     query_nodes=query_nodes)
    ex = p.export()
    rows = np.zeros(n, bool)
    for i in (range(t.num_nodes) if query_nodes is None else query_nodes):
        rows[t.seg_start[i]:t.seg_start[i] + t.seg_len[i]] = True
    vis = _visible_matrix(t, rows)
    fwd = np.zeros((n, n), np.int32)
    for q0, q1, rb, re_ in ex["fwd_tiles"]:
        for k0, k1, causal, _ in ex["fwd_ranges"][rb:re_]:
            blk = np.ones((q1 - q0, k1 - k0), np.int32)
            if causal:
                blk = (np.arange(k0, k1)[None, :] <= np.arange(q0, q1)[:, None]).astype(np.int32)
            fwd[q0:q1, k0:k1] += blk
    assert np.array_equal(fwd, vis), np.argwhere(fwd != vis)[:5]
    bwd = np.zeros((hq, n, n), np.int32)
    for it in ex["bwd_items"]:
        k0, k1, g, eb, ee = it[:5]
        for h, q0, q1, mask in ex["bwd_entries"][eb:ee]:
            assert h // (hq // hkv) == g
            ke = min(k1, -int(mask) - 1) if mask < 0 else k1
            if ke <= k0 or q1 <= q0:
                continue
            blk = np.ones((q1 - q0, ke - k0), np.int32)
            if mask == 1:
                blk = (np.arange(k0, ke)[None, :] <= np.arange(q0, q1)[:, None]).astype(np.int32)
            bwd[h, q0:q1, k0:ke] += blk
    for h in range(hq):
        assert np.array_equal(bwd[h], vis), (h, np.argwhere(bwd[h] != vis)[:5])
    split = p.stats()["fwd_split_tiles"]
    assert p.stats()["pairs"] == int(vis.sum())
    p.close()
    return split


@pytest.mark.parametrize("seed", range(4))
def test_random_plans_cover_every_visible_pair_once(seed):
    """Seeded random forests and caterpillars (packed depth first or in a
    random order), 1-24 query heads on 1-4 kv heads, 1-256 CUs, and the
    whole tree, no node or a random set of query nodes: every (query row,
    key) pair that a listed row sees is in exactly one forward tile (key
    parts of split tiles included) and, for every head, in exactly one
    backward item, and in no other."""
    rng = np.random.default_rng(900 + seed)
    for _ in range(60):
        if rng.random() < 0.15:
            t = caterpillar_tree([int(x) for x in rng.integers(1, 30, int(rng.integers(2, 30)))],
                                 int(rng.integers(1, 150)))
        else:
            t = random_tree(rng, int(rng.integers(1, 25)),
                            max_len=int(rng.choice([5, 60, 300])), min_len=1,
                            n_roots=int(rng.integers(1, 4)), shuffle=bool(rng.random() < 0.5))
        hkv = int(rng.choice([1, 2, 4]))
        hq = hkv * int(rng.choice([1, 2, 3, 6]))
        r = rng.random()
        qn = None if r < 0.3 else [] if r < 0.4 else sorted(
            set(int(x) for x in rng.integers(0, t.num_nodes, int(rng.integers(1, t.num_nodes + 1)))))
        _check_cover(t, hq, hkv, int(rng.choice([1, 4, 16, 256])), qn)


@pytest.mark.parametrize("t,query_nodes", [
    (chain_tree([3500, 300]), None),
    (chain_tree([3300]), [0]),
    (star_tree(3200, 3, 200), [0, 2]),
    (caterpillar_tree([1200, 1100, 1000, 900], 150), None),
])
def test_key_parts_cover_every_visible_pair_once(t, query_nodes):
    """Few query tiles for 256 CUs, long enough to be cut into key parts: the
    parts' key ranges together still cover each visible pair exactly once."""
    assert _check_cover(t, 2, 1, 256, query_nodes) > 0


# ---- longest-first order and the split cap

def _fwd_costs(ex):
    """Cost of each forward tile in launch order: rows x keys of its ranges
    (the causal range counted whole), the planner's sort key."""
    out = []
    for q0, q1, rb, re_ in ex["fwd_tiles"]:
        keys = sum(int(k1 - k0) for k0, k1, _, _ in ex["fwd_ranges"][rb:re_])
        out.append(int(q1 - q0) * keys)
    return np.array(out, np.int64)


def _bwd_costs(ex):
    """Cost of each backward item in launch order (rows x keys over its
    entries); XCD of each item (-1 for the empty items that pad queues)."""
    cost, xcd = [], []
    for it in ex["bwd_items"]:
        k0, k1, g, eb, ee, slot, x = (int(v) for v in it[:7])
        cost.append(sum(int(q1 - q0) * (k1 - k0) for _, q0, q1, _ in ex["bwd_entries"][eb:ee]))
        xcd.append(x)
    return np.array(cost, np.int64), np.array(xcd)


@pytest.mark.parametrize("t", [config_tree(c) for c in (2, 3, 4, 5)] +
                         [random_tree(np.random.default_rng(s), 30, max_len=700, n_roots=2)
                          for s in range(3)])
def test_longest_first_order_and_split_cap(t):
    """Forward tiles run longest first.  No backward item exceeds the split
    cap, max(total / (8 num_cus), 128 * 32 * 64), by more than the 32-row
    rounding of its last chunk.  Items go to XCD b % 8 in launch order, and
    the last 40% of each XCD's work runs longest first, so that every XCD
    ends on its shortest items."""
    hq, hkv, ncus = 8, 2, 256
    p = ta.plan_host(t.parent, t.seg_start, t.seg_len, t.num_tokens, hq, hkv, 128, "bf16",
                     num_cus=ncus)
    ex = p.export()
    fc = _fwd_costs(ex)
    if p.stats()["fwd_split_tiles"] == 0:
        assert np.all(fc[:-1] >= fc[1:])
    bc, xcd = _bwd_costs(ex)
    total = int(bc.sum())
    cap = max(total // (8 * ncus), 128 * 32 * 64)
    assert int(bc.max()) <= cap + 32 * 128
    assert np.array_equal(xcd[xcd >= 0], (np.arange(len(xcd)) % 8)[xcd >= 0])
    for x in range(8):
        q = bc[xcd == x]
        load = int(q.sum())
        acc = np.cumsum(q)
        cut = int(np.argmax(acc * 100 >= load * 60)) + 1 if load else len(q)
        tail = q[cut:]
        assert np.all(tail[:-1] >= tail[1:]), x
    p.close()


def _two_token_chain(m, shuffle):
    parent = np.arange(-1, m - 1, dtype=np.int32)
    seg_len = np.full(m, 2, np.int32)
    order = np.random.default_rng(5).permutation(m) if shuffle else np.arange(m)
    seg_start = np.empty(m, np.int32)
    seg_start[order] = 2 * np.arange(m, dtype=np.int32)
    return parent, seg_start, seg_len, 2 * m


def test_deep_tree_stored_out_of_order_is_refused_before_planning():
    """A 40,000-node chain stored depth first plans in milliseconds; the same
    chain in a shuffled order would need about 10^9 key-range entries (its
    depth per tile) and is refused with UNSUPPORTED from an O(M) count,
    before any list is built.  A 3,000-node shuffled chain is still
    planned, and covered exactly (quadratic, but within the limit)."""
    import time
    par, st, ln, n = _two_token_chain(40000, False)
    p = ta.plan_host(par, st, ln, n, 8, 2, 128, "bf16")
    p.close()
    par, st, ln, n = _two_token_chain(40000, True)
    t0 = time.perf_counter()
    with pytest.raises(ta.TreeAttnError) as ei:
        ta.plan_host(par, st, ln, n, 8, 2, 128, "bf16")
    assert ei.value.status == "UNSUPPORTED" and "depth-first" in str(ei.value)
    assert time.perf_counter() - t0 < 5.0
    par, st, ln, n = _two_token_chain(300, True)
    _check_cover(NodeTable(par, st, ln, n, "shuffled-chain"), 2, 1, 256, None)
    par, st, ln, n = _two_token_chain(3000, True)
    p = ta.plan_host(par, st, ln, n, 2, 1, 128, "bf16")
    p.close()
