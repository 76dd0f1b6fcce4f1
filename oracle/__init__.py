"""fp64 CPU oracle for prefix-shared tree attention (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library never calls it, and it
shares no code with the HIP library: both consume the seeded inputs of
``tree_inputs`` and nothing else.

Parity status of each function is listed in ``oracle/path_expansion.py``
(softmax tree attention), ``oracle/linear_attention.py`` (linear attention
over the tree) and ``oracle/prefix_tree.py``.
"""

from .path_expansion import (  # noqa: F401
    root_to_leaf_paths,
    path_multiplicity,
    token_positions,
    causal_attention,
    tree_attention,
    tree_attention_subset,
    query_rows,
    key_rows,
    key_rows_by_row,
)
from .linear_attention import (  # noqa: F401,E402
    causal_linear_attention,
    tree_linear_attention,
    linear_query_rows,
    linear_key_rows,
)
from . import prefix_tree  # noqa: F401,E402
