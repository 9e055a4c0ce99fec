"""CPU float64 oracle for exact tiled attention — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The HIP library and its Python binding
never import it; the two share no code. Every function is pinned by the
``-m "not gpu"`` tests in ``tests/test_oracle.py`` (closed forms, invariants,
finite differences and an independent library routine).
"""
from .attention import (  # noqa: F401
    MASK_BLOCK_SPARSE,
    MASK_CAUSAL,
    MASK_NONE,
    backward,
    backward_head,
    backward_varlen,
    causal_offset,
    combine_partials,
    forward,
    forward_head,
    forward_varlen,
    online_forward_head,
    online_softmax_row,
    partial_head,
    probabilities_head,
    row_term_head,
    visible,
)
