"""CPU checks of the stored split-tile values (no GPU): each file exists for
the agent, segment-search and long-trunk trees, names keys inside one
128-row tile, and its keys sit in key tiles the planner splits into several
partial slots for both kv heads it covers."""

import importlib.util
import json
import os

import numpy as np
import pytest

from tree_inputs import config_spec, config_tree

HERE = os.path.dirname(os.path.abspath(__file__))


def _gen():
    spec = importlib.util.spec_from_file_location(
        "make_split_tile_golden", os.path.join(HERE, "golden", "make_split_tile_golden.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


@pytest.mark.parametrize("cfg", [3, 4, 5])
def test_split_tile_golden_files(cfg):
    import prefix_shared_tree_attn_amd as ta
    gen = _gen()
    with open(gen.golden_path(cfg)) as f:
        rec = json.load(f)
    sp = config_spec(cfg)
    t = config_tree(cfg)
    assert rec["config"] == cfg and rec["num_tokens"] == t.num_tokens
    assert rec["keys"] == gen.SELECTION[cfg]["keys"]
    assert all(rec["tile_first_row"] <= k < rec["tile_first_row"] + 128 for k in rec["keys"])
    ex = ta.plan_host(t.parent, t.seg_start, t.seg_len, t.num_tokens, sp["heads_q"],
                      sp["heads_kv"], sp["head_dim"], sp["dtype"]).export()
    it = ex["bwd_items"]
    for g in rec["kv_heads"]:
        dk = np.asarray(rec["dk"][str(g)])
        dv = np.asarray(rec["dv"][str(g)])
        assert dk.shape == dv.shape == (len(rec["keys"]), sp["head_dim"])
        assert np.isfinite(dk).all() and np.isfinite(dv).all() and np.abs(dv).max() > 0
        for k in rec["keys"]:
            hit = it[(it[:, 0] <= k) & (k < it[:, 1]) & (it[:, 2] == g) & (it[:, 4] > it[:, 3])]
            assert int((hit[:, 5] >= 0).sum()) >= 2, (k, g)
