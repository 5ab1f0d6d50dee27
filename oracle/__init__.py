"""fp64 CPU oracle for block-sparse multi-draft verification attention.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may call it. It shares no code with the HIP library.
"""

from .sparse_verify import (  # noqa: F401
    num_blocks,
    block_representatives,
    budget_blocks,
    block_scores,
    select_blocks,
    draft_visibility,
    verify_attention,
    merge_partials,
    verify_layer,
)
from . import sparse_ffn  # noqa: F401,E402  (the threshold-pruned FFN; see its module)
