"""Helpers for GPU tests: move seeded inputs to the device, run the library,
compare with the oracle."""

from __future__ import annotations

import numpy as np

from tree_inputs import NodeTable, make_inputs

# Parity bar for this path: relative L2 error <= 1e-2 on O, dQ, dK, dV and
# max |LSE error| <= 1e-3 against the fp64 oracle.
REL_L2 = 1e-2
LSE_ABS = 1e-3
# fp32 inputs are computed in fp32 (fp32 MFMA products and accumulation,
# fp32 P and dS): measured errors are 2e-7 to 1.3e-6, i.e. a few to twenty
# units of fp32 rounding (2^-24 = 6e-8) from sums of up to a few thousand
# terms and the hardware exp2.  1e-5 leaves room for that and is a thousand
# times below what bf16 operands give (about 3e-3).
FP32_REL_L2 = 1e-5
FP32_LSE_ABS = 1e-5


def rel_l2(x: np.ndarray, ref: np.ndarray, zero_scale: float = 0.0) -> float:
    """||x - ref|| / ||ref||.  A reference that is exactly zero (a gradient
    whose terms cancel, such as dK of a lone token, where P = 1 and
    dP = D) has no size of its own: the error is then measured against
    `zero_scale`, the size of the terms that cancel (see cancel_scale)."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref.ravel())
    if den == 0.0:
        den = zero_scale
    return float(np.linalg.norm((x - ref).ravel()) / max(den, 1e-300))


def cancel_scale(other: np.ndarray, o: np.ndarray, do: np.ndarray, scale: float) -> float:
    """scale * ||D|| * ||other|| with D = rowwise dO . O: the size of the two
    terms P dP and P D whose difference dS forms dK (other = Q) and dQ
    (other = K); they cancel exactly when a row attends to one key."""
    d = np.einsum("thd,thd->th", np.asarray(do, np.float64), np.asarray(o, np.float64))
    return float(scale * np.linalg.norm(d) * np.linalg.norm(np.asarray(other, np.float64)))


def to_device(x, dtype: str):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def device_inputs(x, dtype: str):
    if dtype == "bf16":
        return {k: to_device(x.bits[k], "bf16") for k in ("q", "k", "v", "do")}
    return {k: to_device(getattr(x, k), "fp32") for k in ("q", "k", "v", "do")}


def run_library_device(t: NodeTable, x, hq: int, hkv: int, d: int, dtype: str,
                       scale: float, backward: bool = True):
    """Plans, runs fwd (and bwd) through the C ABI; returns device tensors
    (outputs and the device copies of the inputs)."""
    import torch
    import prefix_shared_tree_attn_amd as ta
    dev = device_inputs(x, dtype)
    p = ta.plan(t.parent, t.seg_start, t.seg_len, t.num_tokens, hq, hkv, d, dtype)
    o, lse = ta.fwd(p, dev["q"], dev["k"], dev["v"], scale)
    out = {"o": o, "lse": lse}
    if backward:
        dq, dk, dv = ta.bwd(p, dev["q"], dev["k"], dev["v"], o, lse, dev["do"], scale)
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    p.close()
    return out, dev


def run_library(t: NodeTable, x, hq: int, hkv: int, d: int, dtype: str, scale: float,
                backward: bool = True):
    """As run_library_device, returning host fp64 arrays of the outputs."""
    out, _ = run_library_device(t, x, hq, hkv, d, dtype, scale, backward)
    return {k: v.float().cpu().numpy().astype(np.float64) for k, v in out.items()}


def make(t: NodeTable, hq: int, hkv: int, d: int, dtype: str, do_std: float = 1e-2,
         seed_offset: int = 0):
    return make_inputs(t.num_tokens, hq, hkv, d, dtype=dtype, do_std=do_std,
                       seed_offset=seed_offset)
