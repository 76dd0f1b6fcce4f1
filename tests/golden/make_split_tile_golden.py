"""Writes the expected dK / dV of keys in heavily shared key tiles of the
full-size agent, segment-search and long-trunk trees (``split_tiles_cfg*.json``).

These keys belong to the most shared prefix rows of each tree: their
gradients are summed over every descendant branch (AReaL-DTA, abstract: the
prefix shared by many rollouts is computed once; Tree Training, in the HARTS
page's related list: shared-prefix work is reused in both passes).  In the
library their key tiles are split along the query rows for load balance and
summed from several partial slots.  The values come from the fp64 oracle
(``oracle.key_rows_by_row``) on the seeded workload inputs and nothing else;
the oracle takes minutes of host time on the long-trunk tree, which is why
the values are stored rather than recomputed inside the GPU test.

Usage: ``python tests/golden/make_split_tile_golden.py [config ...]``
(default 3 4 5).  Each file records an input fingerprint
(``input_fingerprint``) that the GPU test recomputes, so values from other
inputs are never compared.
"""

from __future__ import annotations

import hashlib
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from tree_inputs import config_spec, config_tree, make_inputs  # noqa: E402

# Key tiles (first row, 128 rows) and keys checked per tree: the root
# tile of the agent and segment-search trees (the heaviest in each), and a
# trunk tile of the long-trunk tree at 3/8 of the trunk (its oracle cost is
# about a quarter of the trunk's first tile; every trunk tile before the
# middle of the trunk is split).  Keys: first, an inner row, last of the tile.
SELECTION = {
    3: {"tile": 0, "keys": [0, 63, 127]},
    4: {"tile": 0, "keys": [0, 77, 127]},
    5: {"tile": 12288, "keys": [12288, 12338, 12415]},
}


def input_fingerprint(x) -> str:
    """SHA-256 over every 1009th bf16 pattern of Q, K, V and dO (cheap, and
    any change of the generator or its seeds changes it)."""
    h = hashlib.sha256()
    for name in ("q", "k", "v", "do"):
        h.update(np.ascontiguousarray(x.bits[name].reshape(-1)[::1009]).tobytes())
    return h.hexdigest()


def golden_path(cfg: int) -> str:
    return os.path.join(HERE, f"split_tiles_cfg{cfg}.json")


def make(cfg: int) -> dict:
    t = config_tree(cfg)
    sp = config_spec(cfg)
    hq, hkv, d = sp["heads_q"], sp["heads_kv"], sp["head_dim"]
    x = make_inputs(t.num_tokens, hq, hkv, d, dtype=sp["dtype"], do_std=sp["do_std"])
    sel = SELECTION[cfg]
    heads = [0, hkv - 1]
    out = {
        "source": ("fp64 oracle, oracle.key_rows_by_row, on the seeded workload inputs "
                   "(tree_inputs.make_inputs); written by tests/golden/make_split_tile_golden.py"),
        "cite": ("AReaL-DTA, abstract (a shared prefix computed once); Tree Training in the "
                 "HARTS page's related list (shared-prefix reuse in forward and backward)"),
        "config": cfg, "name": sp["name"], "num_tokens": int(t.num_tokens),
        "heads_q": hq, "heads_kv": hkv, "head_dim": d, "scale": sp["scale"],
        "tile_first_row": sel["tile"], "keys": sel["keys"], "kv_heads": heads,
        "input_fingerprint": input_fingerprint(x), "dk": {}, "dv": {},
    }
    for g in heads:
        t0 = time.perf_counter()
        dk, dv = oracle.key_rows_by_row(x.q, x.k, x.v, x.do, t.parent, t.seg_start, t.seg_len,
                                        sp["scale"], sel["keys"], g)
        print(f"config {cfg} kv head {g}: {time.perf_counter() - t0:.1f} s", flush=True)
        out["dk"][str(g)] = [[float(v) for v in row] for row in dk]
        out["dv"][str(g)] = [[float(v) for v in row] for row in dv]
    return out


def main(argv) -> int:
    cfgs = [int(a) for a in argv] or [3, 4, 5]
    for cfg in cfgs:
        rec = make(cfg)
        with open(golden_path(cfg), "w") as f:
            json.dump(rec, f, indent=0)
            f.write("\n")
        print(f"wrote {golden_path(cfg)}", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
