"""Seeded random tensors for the packed unique-token layout.

Q and dO are ``[N, Hq, D]``, K and V are ``[N, Hkv, D]``.  Values are drawn in
fp32 from NumPy's PCG64 (``default_rng(seed)``, fixed seeds Q=1, K=2, V=3,
dO=4 plus an offset), scaled by a standard deviation, and for bf16 workloads
rounded once to bf16 with round-to-nearest-even.  Both the oracle and the GPU
consume exactly these rounded values, so input rounding is not part of any
comparison.  Large tensors are drawn in row chunks to bound host memory; the
chunking is fixed, so a given (seed, shape) always yields the same values.
"""

from __future__ import annotations

import dataclasses
import hashlib

import numpy as np

SEEDS = {"q": 1, "k": 2, "v": 3, "do": 4}
_CHUNK = 1 << 24  # elements per RNG draw


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even.
    Inputs are finite normals, so NaN handling is not needed."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_f32(seed: int, shape, std: float = 1.0) -> np.ndarray:
    """Standard normal fp32 draws, generated chunk by chunk from one stream."""
    rng = np.random.default_rng(seed)
    n = int(np.prod(shape))
    out = np.empty(n, np.float32)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        out[s:e] = rng.standard_normal(e - s, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out.reshape(shape)


@dataclasses.dataclass
class Inputs:
    """Host copies of one workload's inputs.

    ``f32`` holds the exact values (already bf16-rounded for bf16 workloads)
    as float32; ``bits`` holds the bf16 bit patterns (``None`` for fp32)."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    do: np.ndarray
    dtype: str
    bits: dict | None

    def sha256(self) -> str:
        h = hashlib.sha256()
        for name in ("q", "k", "v", "do"):
            a = self.bits[name] if self.bits is not None else getattr(self, name)
            h.update(np.ascontiguousarray(a).tobytes())
        return h.hexdigest()


def make_inputs(n_tokens: int, heads_q: int, heads_kv: int, head_dim: int,
                dtype: str = "bf16", do_std: float = 1e-2, seed_offset: int = 0,
                qkv_std: float = 1.0) -> Inputs:
    shapes = {"q": (n_tokens, heads_q, head_dim), "k": (n_tokens, heads_kv, head_dim),
              "v": (n_tokens, heads_kv, head_dim), "do": (n_tokens, heads_q, head_dim)}
    stds = {"q": qkv_std, "k": qkv_std, "v": qkv_std, "do": do_std}
    vals = {}
    bits = {} if dtype == "bf16" else None
    for name, shape in shapes.items():
        x = normal_f32(SEEDS[name] + seed_offset, shape, stds[name])
        if dtype == "bf16":
            b = bf16_round_bits(x)
            bits[name] = b
            x = bf16_bits_to_f32(b)
        elif dtype != "fp32":
            raise ValueError(dtype)
        vals[name] = x
    return Inputs(vals["q"], vals["k"], vals["v"], vals["do"], dtype, bits)
