"""Seeded synthetic inputs shared by the oracle-side tests and the GPU path.

This package holds no attention arithmetic.  It only builds rollout prefix
trees (as node tables) and draws the random tensors that feed them.  Both the
fp64 oracle (``oracle/``) and the HIP library consume what it produces; it
imports neither of them.

Tree shapes follow the rollout trees the pages describe: a shared prompt or
history at the root and trajectories as root-to-leaf paths (AReaL-DTA,
abstract; HARTS, abstract), GRPO-style groups of stochastic rollouts (TreePO,
section 2, "16 stochastic rollouts") and fixed-length segment trees with
binary branching (TreePO, section 3, tree settings).
"""

from .trees import (  # noqa: F401
    NodeTable,
    CONFIGS,
    config_tree,
    config_spec,
    random_tree,
    chain_tree,
    star_tree,
    binary_tree,
    agent_tree,
    trunk_tree,
    tree_stats,
    dfs_preorder,
    caterpillar_tree,
)
from .tensors import (  # noqa: F401
    bf16_round_bits,
    bf16_bits_to_f32,
    normal_f32,
    make_inputs,
    Inputs,
)
