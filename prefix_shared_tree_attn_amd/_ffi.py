"""ctypes declarations of libtree_attn.so (include/tree_attn.h)."""

from __future__ import annotations

import ctypes
import os

# TREE_ATTN_LIBRARY selects another build of the same library (the host
# sanitizer build that the CPU tests run the planner tests against).
LIB_PATH = os.environ.get("TREE_ATTN_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libtree_attn.so")

STATUS = {
    0: "OK", 1: "INVALID_ARG", 2: "BAD_TREE", 3: "LAYOUT", 4: "UNSUPPORTED",
    5: "WORKSPACE", 6: "HIP", 7: "NO_DEVICE_PLAN",
}
DTYPES = {"bf16": 0, "fp32": 1}

# every symbol include/tree_attn.h declares
EXPORTS = (
    "tree_attn_plan", "tree_attn_plan_host", "tree_attn_plan_destroy",
    "tree_attn_workspace_size", "tree_attn_fwd", "tree_attn_bwd",
    "tree_attn_plan_stats", "tree_attn_plan_export", "tree_attn_status_string",
    "tree_attn_last_error", "tree_attn_timing_enable", "tree_attn_timing_read",
    "tree_attn_positions", "tree_attn_build_tree", "tree_attn_gather_rows",
    "tree_attn_scatter_sum_rows", "tree_attn_rope", "tree_attn_lin_workspace_size",
    "tree_attn_lin_fwd", "tree_attn_lin_bwd", "tree_attn_lin_plan_export",
    "tree_attn_plan_subset", "tree_attn_plan_host_subset", "tree_attn_bwd_accum",
    "tree_attn_accum_cast", "tree_attn_bwd_noalloc", "tree_attn_plan_export_split",
    "tree_attn_lin_plan_export_chains", "tree_attn_walk_runs",
)


class PlanStats(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int64) for name in (
        "num_tokens", "num_nodes", "num_q_heads", "num_kv_heads", "head_dim", "pairs",
        "fwd_tiles", "fwd_ranges", "fwd_blocks", "bwd_items", "bwd_entries",
        "bwd_split_tiles", "bwd_slots", "fwd_tile_rows", "fwd_tile_keys", "bwd_tile_keys",
        "bwd_block_rows", "lin_pieces", "lin_succ", "lin_chunk", "subset", "query_rows",
        "fwd_split_tiles", "fwd_slots", "lin_chains", "lin_phases", "lin_nodes")]


class Timing(ctypes.Structure):
    _fields_ = [("launches", ctypes.c_int64 * 16), ("total_ms", ctypes.c_double * 16)]


TIMING_KINDS = ("fwd", "bwd_pre", "bwd_dkdv", "bwd_reduce", "bwd_dq", "positions", "gather",
                "scatter_sum", "rope", "lin_kv", "lin_scan", "lin_out", "lin_qdo", "lin_rscan",
                "lin_dq", "lin_dkdv")


class TreeAttnError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = STATUS.get(status, str(status))
        super().__init__(f"{where}: {self.status}: {detail}")


_lib = None


def lib() -> ctypes.CDLL:
    """Loads the HIP library; fails loudly when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m prefix_shared_tree_attn_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    i32p = ctypes.POINTER(ctypes.c_int32)
    vp = ctypes.c_void_p
    L.tree_attn_plan.argtypes = [i32p, i32p, i32p] + [ctypes.c_int32] * 5 + [
        ctypes.c_int, vp, ctypes.POINTER(vp)]
    L.tree_attn_plan_host.argtypes = [i32p, i32p, i32p] + [ctypes.c_int32] * 5 + [
        ctypes.c_int, ctypes.c_int32, ctypes.POINTER(vp)]
    L.tree_attn_plan_destroy.argtypes = [vp]
    L.tree_attn_plan_destroy.restype = None
    L.tree_attn_workspace_size.argtypes = [vp, ctypes.POINTER(ctypes.c_size_t),
                                           ctypes.POINTER(ctypes.c_size_t)]
    L.tree_attn_fwd.argtypes = [vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, ctypes.c_size_t, vp]
    L.tree_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, vp,
                                ctypes.c_size_t, vp]
    L.tree_attn_plan_stats.argtypes = [vp, ctypes.POINTER(PlanStats)]
    L.tree_attn_plan_export.argtypes = [vp, i32p, i32p, i32p, i32p]
    L.tree_attn_plan_export_split.argtypes = [vp, i32p, i32p]
    L.tree_attn_lin_plan_export_chains.argtypes = [vp, i32p, i32p, i32p]
    L.tree_attn_status_string.argtypes = [ctypes.c_int]
    L.tree_attn_status_string.restype = ctypes.c_char_p
    L.tree_attn_last_error.argtypes = []
    L.tree_attn_last_error.restype = ctypes.c_char_p
    L.tree_attn_positions.argtypes = [vp, vp, vp, vp]
    i64p = ctypes.POINTER(ctypes.c_int64)
    L.tree_attn_build_tree.argtypes = [i32p, i64p, ctypes.c_int32] + [i32p] * 10
    L.tree_attn_walk_runs.argtypes = [i32p, i32p, ctypes.c_int32, ctypes.c_int64, i32p, i32p,
                                      i32p]
    L.tree_attn_gather_rows.argtypes = [vp, vp, vp, ctypes.c_int64, ctypes.c_int64, vp]
    L.tree_attn_scatter_sum_rows.argtypes = [vp, vp, vp, vp, ctypes.c_int64, ctypes.c_int64,
                                             ctypes.c_int, vp]
    L.tree_attn_rope.argtypes = [vp, vp, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                 ctypes.c_float, ctypes.c_int32, ctypes.c_int, vp]
    L.tree_attn_lin_workspace_size.argtypes = [vp, ctypes.POINTER(ctypes.c_size_t),
                                               ctypes.POINTER(ctypes.c_size_t)]
    L.tree_attn_lin_fwd.argtypes = [vp, vp, vp, vp, ctypes.c_float, vp, vp, ctypes.c_size_t, vp]
    L.tree_attn_lin_bwd.argtypes = [vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, vp,
                                    ctypes.c_size_t, vp]
    L.tree_attn_lin_plan_export.argtypes = [vp, i32p, i32p]
    L.tree_attn_plan_subset.argtypes = [i32p, i32p, i32p] + [ctypes.c_int32] * 5 + [
        ctypes.c_int, i32p, ctypes.c_int32, vp, ctypes.POINTER(vp)]
    L.tree_attn_plan_host_subset.argtypes = [i32p, i32p, i32p] + [ctypes.c_int32] * 5 + [
        ctypes.c_int, i32p, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(vp)]
    L.tree_attn_bwd_accum.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp,
                                      vp, ctypes.c_size_t, vp]
    L.tree_attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp,
                                        vp]
    L.tree_attn_accum_cast.argtypes = [vp, vp, ctypes.c_int64, ctypes.c_int, vp]
    L.tree_attn_timing_enable.argtypes = [ctypes.c_int]
    L.tree_attn_timing_read.argtypes = [ctypes.POINTER(Timing), ctypes.c_int]
    for fn in ("tree_attn_timing_enable", "tree_attn_timing_read", "tree_attn_plan",
               "tree_attn_plan_host", "tree_attn_workspace_size", "tree_attn_fwd", "tree_attn_bwd",
               "tree_attn_plan_stats", "tree_attn_plan_export", "tree_attn_positions",
               "tree_attn_build_tree", "tree_attn_gather_rows", "tree_attn_scatter_sum_rows",
               "tree_attn_rope", "tree_attn_lin_workspace_size", "tree_attn_lin_fwd",
               "tree_attn_lin_bwd", "tree_attn_lin_plan_export", "tree_attn_plan_subset",
               "tree_attn_plan_host_subset", "tree_attn_bwd_accum", "tree_attn_accum_cast",
               "tree_attn_bwd_noalloc", "tree_attn_plan_export_split",
               "tree_attn_lin_plan_export_chains", "tree_attn_walk_runs"):
        getattr(L, fn).restype = ctypes.c_int
    _lib = L
    return L


def check(status: int, where: str) -> None:
    if status != 0:
        detail = lib().tree_attn_last_error().decode(errors="replace")
        raise TreeAttnError(status, where, detail)
