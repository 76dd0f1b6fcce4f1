"""Prefix-shared tree attention on MI355X: Python binding of libtree_attn.so.

Argument marshalling only: every step of planning and of the forward and
backward passes runs in the C++/HIP library (include/tree_attn.h).  PyTorch
provides device memory and the current HIP stream.  Importing the package
does not need a GPU; calling ``fwd``/``bwd`` needs the built library and a
GPU, and fails loudly otherwise.
"""

from __future__ import annotations

import ctypes
from typing import Optional, Tuple

import numpy as np

from . import _ffi
from ._ffi import TreeAttnError, PlanStats  # noqa: F401

__all__ = ["Plan", "plan", "plan_host", "fwd", "bwd", "bwd_noalloc", "bwd_accum", "accum_cast", "positions",
           "workspace",
           "TreeAttnError", "timing_enable", "timing_read", "PrefixTree", "build_tree",
           "gather_rows", "scatter_sum_rows", "rope", "lin_fwd", "lin_bwd", "lin_workspace",
           "walk_runs"]


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _stream_handle(stream) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


class Plan:
    """An immutable work plan for one tree and one head configuration."""

    def __init__(self, handle: int, num_tokens: int, hq: int, hkv: int, head_dim: int,
                 dtype: str, device: Optional[int]):
        self._h = ctypes.c_void_p(handle)
        self.num_tokens, self.hq, self.hkv, self.head_dim = num_tokens, hq, hkv, head_dim
        self.dtype = dtype
        self.device = device

    @property
    def handle(self) -> ctypes.c_void_p:
        if not self._h:
            raise ValueError("plan already destroyed")
        return self._h

    def close(self) -> None:
        if self._h:
            _ffi.lib().tree_attn_plan_destroy(self._h)
            self._h = ctypes.c_void_p(0)

    def __del__(self):  # pragma: no cover - interpreter shutdown order
        try:
            self.close()
        except Exception:
            pass

    def workspace_size(self) -> Tuple[int, int]:
        f, b = ctypes.c_size_t(0), ctypes.c_size_t(0)
        _ffi.check(_ffi.lib().tree_attn_workspace_size(self.handle, ctypes.byref(f),
                                                       ctypes.byref(b)), "workspace_size")
        return int(f.value), int(b.value)

    def lin_workspace_size(self) -> Tuple[int, int]:
        f, b = ctypes.c_size_t(0), ctypes.c_size_t(0)
        _ffi.check(_ffi.lib().tree_attn_lin_workspace_size(self.handle, ctypes.byref(f),
                                                           ctypes.byref(b)), "lin_workspace_size")
        return int(f.value), int(b.value)

    def lin_export(self) -> dict:
        """Linear-attention piece table: ``pieces [P, 8]`` and ``succ``, and the
        state scans' order: ``chains``, ``chain_nodes`` and ``phases``."""
        st = self.stats()
        out = {"pieces": np.zeros((st["lin_pieces"], 8), np.int32),
               "succ": np.zeros((st["lin_succ"],), np.int32)}
        _ffi.check(_ffi.lib().tree_attn_lin_plan_export(
            self.handle, _ptr(out["pieces"]), _ptr(out["succ"])), "lin_plan_export")
        out["chains"] = np.zeros((st["lin_chains"], 4), np.int32)
        out["chain_nodes"] = np.zeros((st["lin_nodes"],), np.int32)
        out["phases"] = np.zeros((st["lin_phases"], 4), np.int32)
        _ffi.check(_ffi.lib().tree_attn_lin_plan_export_chains(
            self.handle, _ptr(out["chains"]), _ptr(out["chain_nodes"]), _ptr(out["phases"])),
            "lin_plan_export_chains")
        return out

    def stats(self) -> dict:
        s = PlanStats()
        _ffi.check(_ffi.lib().tree_attn_plan_stats(self.handle, ctypes.byref(s)), "plan_stats")
        return {name: int(getattr(s, name)) for name, _ in PlanStats._fields_}

    def export(self) -> dict:
        st = self.stats()
        out = {
            "fwd_tiles": np.zeros((st["fwd_tiles"], 4), np.int32),
            "fwd_ranges": np.zeros((st["fwd_ranges"], 4), np.int32),
            "bwd_items": np.zeros((st["bwd_items"], 8), np.int32),
            "bwd_entries": np.zeros((st["bwd_entries"], 4), np.int32),
        }
        _ffi.check(_ffi.lib().tree_attn_plan_export(
            self.handle, _ptr(out["fwd_tiles"]), _ptr(out["fwd_ranges"]),
            _ptr(out["bwd_items"]), _ptr(out["bwd_entries"])), "plan_export")
        out["fwd_part"] = np.zeros((st["fwd_tiles"],), np.int32)
        out["fwd_combine"] = np.zeros((st["fwd_split_tiles"], 4), np.int32)
        _ffi.check(_ffi.lib().tree_attn_plan_export_split(
            self.handle, _ptr(out["fwd_part"]), _ptr(out["fwd_combine"])), "plan_export_split")
        return out


def _plan_args(parent, seg_start, seg_len, num_tokens, hq, hkv, head_dim, dtype):
    par, st, ln = _i32(parent), _i32(seg_start), _i32(seg_len)
    if not (par.shape == st.shape == ln.shape) or par.ndim != 1:
        raise ValueError("parent, seg_start and seg_len must be 1-D of equal length")
    if dtype not in _ffi.DTYPES:
        raise ValueError(f"dtype must be one of {list(_ffi.DTYPES)}")
    return par, st, ln, int(par.shape[0])


def plan(parent, seg_start, seg_len, num_tokens: int, hq: int, hkv: int, head_dim: int,
         dtype: str = "bf16", stream=None, query_nodes=None) -> Plan:
    """Validates the node table and builds a device plan (tree_attn_plan), or
    with ``query_nodes`` a query-subset plan (tree_attn_plan_subset)."""
    import torch
    par, st, ln, m = _plan_args(parent, seg_start, seg_len, num_tokens, hq, hkv, head_dim, dtype)
    h = ctypes.c_void_p(0)
    L = _ffi.lib()
    common = (_ptr(par), _ptr(st), _ptr(ln), m, int(num_tokens), int(hq), int(hkv),
              int(head_dim), _ffi.DTYPES[dtype])
    sp = ctypes.c_void_p(_stream_handle(stream))
    if query_nodes is None:
        _ffi.check(L.tree_attn_plan(*common, sp, ctypes.byref(h)), "plan")
    else:
        qn = _i32(query_nodes).reshape(-1)
        _ffi.check(L.tree_attn_plan_subset(*common, _ptr(qn), int(qn.shape[0]), sp,
                                           ctypes.byref(h)), "plan_subset")
    return Plan(h.value, int(num_tokens), hq, hkv, head_dim, dtype, torch.cuda.current_device())


def plan_host(parent, seg_start, seg_len, num_tokens: int, hq: int, hkv: int, head_dim: int,
              dtype: str = "bf16", num_cus: int = 256, query_nodes=None) -> Plan:
    """Host-only plan (tree_attn_plan_host / tree_attn_plan_host_subset):
    validation, inspection, sizing."""
    par, st, ln, m = _plan_args(parent, seg_start, seg_len, num_tokens, hq, hkv, head_dim, dtype)
    h = ctypes.c_void_p(0)
    L = _ffi.lib()
    common = (_ptr(par), _ptr(st), _ptr(ln), m, int(num_tokens), int(hq), int(hkv),
              int(head_dim), _ffi.DTYPES[dtype])
    if query_nodes is None:
        _ffi.check(L.tree_attn_plan_host(*common, int(num_cus), ctypes.byref(h)), "plan_host")
    else:
        qn = _i32(query_nodes).reshape(-1)
        _ffi.check(L.tree_attn_plan_host_subset(*common, _ptr(qn), int(qn.shape[0]),
                                                int(num_cus), ctypes.byref(h)),
                   "plan_host_subset")
    return Plan(h.value, int(num_tokens), hq, hkv, head_dim, dtype, None)


_TORCH_DTYPES = {"bf16": "bfloat16", "fp32": "float32"}


def _check_tensor(x, name: str, shape, p: Plan):
    import torch
    fp32 = name in ("lse", "dk_acc", "dv_acc")
    want = torch.float32 if fp32 else getattr(torch, _TORCH_DTYPES[p.dtype])
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if x.device.type != "cuda" or x.device.index != p.device:
        raise ValueError(f"{name} must live on cuda:{p.device}")
    if x.dtype != want:
        raise TypeError(f"{name} must be {want}, got {x.dtype}")
    if tuple(x.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(x.shape)}")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(x.data_ptr())


def workspace(p: Plan, which: str = "bwd"):
    """Allocates a device workspace of the size the plan asks for."""
    import torch
    f, b = p.workspace_size()
    n = b if which == "bwd" else f
    return torch.empty(max(n, 1), dtype=torch.uint8, device=f"cuda:{p.device}")


def fwd(p: Plan, q, k, v, scale: float, o=None, lse=None, ws=None, stream=None):
    """tree_attn_fwd: returns (o [N,Hq,D], lse [Hq,N] fp32)."""
    import torch
    n, hq, hkv, d = p.num_tokens, p.hq, p.hkv, p.head_dim
    if o is None:
        o = torch.empty((n, hq, d), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((hq, n), dtype=torch.float32, device=q.device)
    args = [_check_tensor(q, "q", (n, hq, d), p), _check_tensor(k, "k", (n, hkv, d), p),
            _check_tensor(v, "v", (n, hkv, d), p)]
    po = _check_tensor(o, "o", (n, hq, d), p)
    pl = _check_tensor(lse, "lse", (hq, n), p)
    if ws is None and p.workspace_size()[0] > 0:
        ws = workspace(p, "fwd")
    wptr, wbytes = (ctypes.c_void_p(ws.data_ptr()), ws.numel()) if ws is not None else (None, 0)
    _ffi.check(_ffi.lib().tree_attn_fwd(p.handle, *args, ctypes.c_float(scale), po, pl, wptr,
                                        wbytes, ctypes.c_void_p(_stream_handle(stream))), "fwd")
    return o, lse


def bwd(p: Plan, q, k, v, o, lse, do, scale: float, dq=None, dk=None, dv=None, ws=None,
        stream=None):
    """tree_attn_bwd: returns (dq, dk, dv)."""
    import torch
    n, hq, hkv, d = p.num_tokens, p.hq, p.hkv, p.head_dim
    if dq is None:
        dq = torch.empty((n, hq, d), dtype=q.dtype, device=q.device)
    if dk is None:
        dk = torch.empty((n, hkv, d), dtype=q.dtype, device=q.device)
    if dv is None:
        dv = torch.empty((n, hkv, d), dtype=q.dtype, device=q.device)
    if ws is None:
        ws = workspace(p, "bwd")
    args = [_check_tensor(q, "q", (n, hq, d), p), _check_tensor(k, "k", (n, hkv, d), p),
            _check_tensor(v, "v", (n, hkv, d), p), _check_tensor(o, "o", (n, hq, d), p),
            _check_tensor(lse, "lse", (hq, n), p), _check_tensor(do, "do", (n, hq, d), p)]
    outs = [_check_tensor(dq, "dq", (n, hq, d), p), _check_tensor(dk, "dk", (n, hkv, d), p),
            _check_tensor(dv, "dv", (n, hkv, d), p)]
    _ffi.check(_ffi.lib().tree_attn_bwd(
        p.handle, *args[:5], args[5], ctypes.c_float(scale), *outs,
        ctypes.c_void_p(ws.data_ptr()), ws.numel(),
        ctypes.c_void_p(_stream_handle(stream))), "bwd")
    return dq, dk, dv


def bwd_noalloc(p: Plan, q, k, v, o, lse, do, scale: float, dq=None, dk=None, dv=None,
                stream=None):
    """tree_attn_bwd_noalloc: tree_attn_bwd with the library's fixed scratch
    instead of a caller workspace; returns (dq, dk, dv).  Outputs that are
    not passed in are allocated here, by torch, before the call."""
    import torch
    n, hq, hkv, d = p.num_tokens, p.hq, p.hkv, p.head_dim
    if dq is None:
        dq = torch.empty((n, hq, d), dtype=q.dtype, device=q.device)
    if dk is None:
        dk = torch.empty((n, hkv, d), dtype=q.dtype, device=q.device)
    if dv is None:
        dv = torch.empty((n, hkv, d), dtype=q.dtype, device=q.device)
    args = [_check_tensor(q, "q", (n, hq, d), p), _check_tensor(k, "k", (n, hkv, d), p),
            _check_tensor(v, "v", (n, hkv, d), p), _check_tensor(o, "o", (n, hq, d), p),
            _check_tensor(lse, "lse", (hq, n), p), _check_tensor(do, "do", (n, hq, d), p)]
    outs = [_check_tensor(dq, "dq", (n, hq, d), p), _check_tensor(dk, "dk", (n, hkv, d), p),
            _check_tensor(dv, "dv", (n, hkv, d), p)]
    _ffi.check(_ffi.lib().tree_attn_bwd_noalloc(
        p.handle, *args, ctypes.c_float(scale), *outs,
        ctypes.c_void_p(_stream_handle(stream))), "bwd_noalloc")
    return dq, dk, dv


def bwd_accum(p: Plan, q, k, v, o, lse, do, scale: float, dk_acc, dv_acc, dq=None, ws=None,
              stream=None):
    """tree_attn_bwd_accum on a query-subset plan: writes dQ of the query
    rows and adds the K/V gradients into the fp32 ``dk_acc``/``dv_acc``
    [N,Hkv,D].  Returns dq."""
    import torch
    n, hq, hkv, d = p.num_tokens, p.hq, p.hkv, p.head_dim
    if dq is None:
        dq = torch.empty((n, hq, d), dtype=q.dtype, device=q.device)
    if ws is None:
        ws = workspace(p, "bwd")
    args = [_check_tensor(q, "q", (n, hq, d), p), _check_tensor(k, "k", (n, hkv, d), p),
            _check_tensor(v, "v", (n, hkv, d), p), _check_tensor(o, "o", (n, hq, d), p),
            _check_tensor(lse, "lse", (hq, n), p), _check_tensor(do, "do", (n, hq, d), p)]
    outs = [_check_tensor(dq, "dq", (n, hq, d), p),
            _check_tensor(dk_acc, "dk_acc", (n, hkv, d), p),
            _check_tensor(dv_acc, "dv_acc", (n, hkv, d), p)]
    _ffi.check(_ffi.lib().tree_attn_bwd_accum(
        p.handle, *args, ctypes.c_float(scale), *outs, ctypes.c_void_p(ws.data_ptr()),
        ws.numel(), ctypes.c_void_p(_stream_handle(stream))), "bwd_accum")
    return dq


def accum_cast(acc, dtype: str = "bf16", out=None, stream=None):
    """tree_attn_accum_cast: fp32 accumulator -> tensor of ``dtype``."""
    import torch
    _dev_check(acc, "acc", torch.float32)
    if not acc.is_contiguous():
        raise ValueError("acc must be contiguous")
    if out is None:
        out = torch.empty(acc.shape, dtype=getattr(torch, _TORCH_DTYPES[dtype]),
                          device=acc.device)
    _dev_check(out, "out", getattr(torch, _TORCH_DTYPES[dtype]))
    if out.numel() != acc.numel() or not out.is_contiguous():
        raise ValueError("out must be contiguous with as many elements as acc")
    _ffi.check(_ffi.lib().tree_attn_accum_cast(
        ctypes.c_void_p(acc.data_ptr()), ctypes.c_void_p(out.data_ptr()), acc.numel(),
        _ffi.DTYPES[dtype], ctypes.c_void_p(_stream_handle(stream))), "accum_cast")
    return out


def lin_workspace(p: Plan, which: str = "bwd"):
    """Allocates the device workspace of the linear-attention pass."""
    import torch
    f, b = p.lin_workspace_size()
    n = b if which == "bwd" else f
    return torch.empty(max(n, 1), dtype=torch.uint8, device=f"cuda:{p.device}")


def lin_fwd(p: Plan, q, k, v, scale: float, o=None, ws=None, stream=None):
    """tree_attn_lin_fwd: chunkwise linear attention over the tree; returns o."""
    import torch
    n, hq, hkv, d = p.num_tokens, p.hq, p.hkv, p.head_dim
    if o is None:
        o = torch.empty((n, hq, d), dtype=q.dtype, device=q.device)
    if ws is None:
        ws = lin_workspace(p, "fwd")
    args = [_check_tensor(q, "q", (n, hq, d), p), _check_tensor(k, "k", (n, hkv, d), p),
            _check_tensor(v, "v", (n, hkv, d), p)]
    po = _check_tensor(o, "o", (n, hq, d), p)
    _ffi.check(_ffi.lib().tree_attn_lin_fwd(
        p.handle, *args, ctypes.c_float(scale), po, ctypes.c_void_p(ws.data_ptr()), ws.numel(),
        ctypes.c_void_p(_stream_handle(stream))), "lin_fwd")
    return o


def lin_bwd(p: Plan, q, k, v, do, scale: float, dq=None, dk=None, dv=None, ws=None,
            stream=None):
    """tree_attn_lin_bwd: returns (dq, dk, dv)."""
    import torch
    n, hq, hkv, d = p.num_tokens, p.hq, p.hkv, p.head_dim
    if dq is None:
        dq = torch.empty((n, hq, d), dtype=q.dtype, device=q.device)
    if dk is None:
        dk = torch.empty((n, hkv, d), dtype=q.dtype, device=q.device)
    if dv is None:
        dv = torch.empty((n, hkv, d), dtype=q.dtype, device=q.device)
    if ws is None:
        ws = lin_workspace(p, "bwd")
    args = [_check_tensor(q, "q", (n, hq, d), p), _check_tensor(k, "k", (n, hkv, d), p),
            _check_tensor(v, "v", (n, hkv, d), p), _check_tensor(do, "do", (n, hq, d), p)]
    outs = [_check_tensor(dq, "dq", (n, hq, d), p), _check_tensor(dk, "dk", (n, hkv, d), p),
            _check_tensor(dv, "dv", (n, hkv, d), p)]
    _ffi.check(_ffi.lib().tree_attn_lin_bwd(
        p.handle, *args, ctypes.c_float(scale), *outs, ctypes.c_void_p(ws.data_ptr()),
        ws.numel(), ctypes.c_void_p(_stream_handle(stream))), "lin_bwd")
    return dq, dk, dv


def positions(p: Plan, node_id=None, pos_id=None, stream=None):
    """tree_attn_positions: returns (node_id [N] int32, pos_id [N] int32)."""
    import torch
    n = p.num_tokens
    dev = f"cuda:{p.device}"
    if node_id is None:
        node_id = torch.empty((n,), dtype=torch.int32, device=dev)
    if pos_id is None:
        pos_id = torch.empty((n,), dtype=torch.int32, device=dev)
    for name, x in (("node_id", node_id), ("pos_id", pos_id)):
        if (x.dtype != torch.int32 or tuple(x.shape) != (n,) or not x.is_contiguous()
                or x.device.type != "cuda" or x.device.index != p.device):
            raise ValueError(f"{name} must be a contiguous int32 [{n}] tensor on {dev}")
    _ffi.check(_ffi.lib().tree_attn_positions(
        p.handle, ctypes.c_void_p(node_id.data_ptr()), ctypes.c_void_p(pos_id.data_ptr()),
        ctypes.c_void_p(_stream_handle(stream))), "positions")
    return node_id, pos_id


class PrefixTree:
    """Result of tree_attn_build_tree (host numpy int32 arrays)."""

    def __init__(self, parent, seg_start, seg_len, unique_tokens, traj_index, mult, inv_offsets,
                 inv_positions):
        self.parent, self.seg_start, self.seg_len = parent, seg_start, seg_len
        self.unique_tokens, self.traj_index, self.mult = unique_tokens, traj_index, mult
        self.inv_offsets, self.inv_positions = inv_offsets, inv_positions

    @property
    def num_nodes(self) -> int:
        return int(self.parent.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.unique_tokens.shape[0])


def walk_runs(parent, seg_len, budget: int = 0):
    """tree_attn_walk_runs: the query-node lists of a memory-bounded
    depth-first walk's calls, in preorder (budget <= 0: the longest
    root-to-leaf path's token count)."""
    parent, seg_len = _i32(parent).reshape(-1), _i32(seg_len).reshape(-1)
    m = parent.shape[0]
    if seg_len.shape[0] != m:
        raise ValueError("parent and seg_len differ in length")
    order = np.zeros(max(m, 1), np.int32)
    starts = np.zeros(m + 1, np.int32)
    runs = ctypes.c_int32(0)
    _ffi.check(_ffi.lib().tree_attn_walk_runs(_ptr(parent), _ptr(seg_len), m, int(budget),
                                              _ptr(order), _ptr(starts), ctypes.byref(runs)),
               "walk_runs")
    r = runs.value
    return [order[starts[i]:starts[i + 1]].tolist() for i in range(r)]


def build_tree(trajectories) -> PrefixTree:
    """tree_attn_build_tree over a list of token-id sequences."""
    seqs = [np.asarray(t, dtype=np.int32).ravel() for t in trajectories]
    b = len(seqs)
    offsets = np.zeros(b + 1, np.int64)
    if b:
        offsets[1:] = np.cumsum([s.shape[0] for s in seqs])
    total = int(offsets[-1])
    tokens = np.ascontiguousarray(np.concatenate(seqs) if total else np.zeros(0, np.int32))
    cap = max(2 * b, 1)
    parent = np.zeros(cap, np.int32)
    seg_start = np.zeros(cap, np.int32)
    seg_len = np.zeros(cap, np.int32)
    uniq = np.zeros(max(total, 1), np.int32)
    tidx = np.zeros(max(total, 1), np.int32)
    mult = np.zeros(max(total, 1), np.int32)
    inv_off = np.zeros(total + 1, np.int32)
    inv_pos = np.zeros(max(total, 1), np.int32)
    m, n = ctypes.c_int32(0), ctypes.c_int32(0)
    _ffi.check(_ffi.lib().tree_attn_build_tree(
        _ptr(tokens), offsets.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), b,
        _ptr(parent), _ptr(seg_start), _ptr(seg_len), _ptr(uniq), _ptr(tidx), _ptr(mult),
        _ptr(inv_off), _ptr(inv_pos), ctypes.byref(m), ctypes.byref(n)), "build_tree")
    m, n = m.value, n.value
    return PrefixTree(parent[:m].copy(), seg_start[:m].copy(), seg_len[:m].copy(),
                      uniq[:n].copy(), tidx[:total].copy(), mult[:n].copy(),
                      inv_off[:n + 1].copy(), inv_pos[:total].copy())


def _dev_check(x, name, dtype=None):
    import torch
    if not isinstance(x, torch.Tensor) or x.device.type != "cuda" or not x.is_contiguous():
        raise ValueError(f"{name} must be a contiguous CUDA tensor")
    if dtype is not None and x.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {x.dtype}")
    return ctypes.c_void_p(x.data_ptr())


def gather_rows(src, index, out=None, stream=None):
    """tree_attn_gather_rows: out[i] = src[index[i]] (rows = leading dimension)."""
    import torch
    rows = int(index.shape[0])
    if out is None:
        out = torch.empty((rows,) + tuple(src.shape[1:]), dtype=src.dtype, device=src.device)
    if tuple(out.shape[1:]) != tuple(src.shape[1:]) or out.dtype != src.dtype or out.shape[0] != rows:
        raise ValueError("out must have index.shape[0] rows shaped like src's rows")
    row_bytes = int(np.prod(src.shape[1:])) * src.element_size()
    _ffi.check(_ffi.lib().tree_attn_gather_rows(
        _dev_check(src, "src"), _dev_check(out, "out"), _dev_check(index, "index", torch.int32),
        rows, row_bytes, ctypes.c_void_p(_stream_handle(stream))), "gather_rows")
    return out


def scatter_sum_rows(src, inv_offsets, inv_positions, num_rows: int, out=None, stream=None):
    """tree_attn_scatter_sum_rows: out[u] = sum of src rows mapped to u (fp32, fixed order)."""
    import torch
    dt = {torch.bfloat16: "bf16", torch.float32: "fp32"}.get(src.dtype)
    if dt is None:
        raise TypeError("src must be bfloat16 or float32")
    if out is None:
        out = torch.empty((num_rows,) + tuple(src.shape[1:]), dtype=src.dtype, device=src.device)
    if tuple(out.shape) != (num_rows,) + tuple(src.shape[1:]) or out.dtype != src.dtype:
        raise ValueError("out must be [num_rows] + src row shape in src's dtype")
    row_elems = int(np.prod(src.shape[1:])) if src.dim() > 1 else 1
    _ffi.check(_ffi.lib().tree_attn_scatter_sum_rows(
        _dev_check(src, "src"), _dev_check(out, "out"),
        _dev_check(inv_offsets, "inv_offsets", torch.int32),
        _dev_check(inv_positions, "inv_positions", torch.int32), int(num_rows), row_elems,
        _ffi.DTYPES[dt], ctypes.c_void_p(_stream_handle(stream))), "scatter_sum_rows")
    return out


def rope(x, pos_id, theta: float = 10000.0, inverse: bool = False, stream=None):
    """tree_attn_rope: rotates x [N, H, D] in place at positions pos_id [N]."""
    import torch
    dt = {torch.bfloat16: "bf16", torch.float32: "fp32"}.get(x.dtype)
    if dt is None or x.dim() != 3:
        raise TypeError("x must be a 3-D bfloat16 or float32 tensor [N, H, D]")
    n, h, d = (int(v) for v in x.shape)
    if tuple(pos_id.shape) != (n,):
        raise ValueError(f"pos_id must have shape ({n},)")
    _ffi.check(_ffi.lib().tree_attn_rope(
        _dev_check(x, "x"), _dev_check(pos_id, "pos_id", torch.int32), n, h, d,
        ctypes.c_float(theta), 1 if inverse else 0, _ffi.DTYPES[dt],
        ctypes.c_void_p(_stream_handle(stream))), "rope")
    return x


def timing_enable(enable: bool = True) -> None:
    """Brackets every library kernel with HIP events (tree_attn_timing_enable)."""
    _ffi.check(_ffi.lib().tree_attn_timing_enable(1 if enable else 0), "timing_enable")


def timing_read(reset: bool = True) -> dict:
    """Per kernel kind: launches and summed milliseconds (tree_attn_timing_read)."""
    t = _ffi.Timing()
    _ffi.check(_ffi.lib().tree_attn_timing_read(ctypes.byref(t), 1 if reset else 0),
               "timing_read")
    return {k: {"launches": int(t.launches[i]), "total_ms": float(t.total_ms[i])}
            for i, k in enumerate(_ffi.TIMING_KINDS)}
