"""CPU fp64 oracle for causal grouped-query attention -- TEST INFRASTRUCTURE ONLY.

Imported only by the test suite, the package smoke check and the benchmark's
CPU-baseline leg.  Shares no code with the HIP library.  Every function is
pinned by tests marked ``not gpu`` (worked example, closed forms, invariants,
finite differences and a PyTorch CPU cross-check).
"""

from .attention import (  # noqa: F401
    attention_weights,
    backward,
    backward_group,
    forward,
    forward_rows,
    kv_head,
    visible,
    visible_pairs_per_head,
)
