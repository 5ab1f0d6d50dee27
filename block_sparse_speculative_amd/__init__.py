"""Block-sparse multi-draft verification attention for MI355X (gfx950).

The hot path lives in libsv.so (HIP kernels behind the C ABI in include/sv.h);
this package is its thin ctypes binding plus device-buffer orchestration.
"""

from ._lib import (  # noqa: F401
    EXPORTS, LIB_PATH, SV_BF16, SV_F32, AttnPlan, Budget, Shape, SvError, abi_version,
    attn_num_splits, attn_plan, attn_workspace_bytes, block_repr, budget_blocks, lib,
    make_budget, make_shape, reuse_indices, select_and_attend, select_and_attend_static,
    select_and_attend_workspace_bytes, select_blocks, select_workspace_bytes,
    sparse_verify_attn, make_ffn_shape, sparse_ffn, sparse_ffn_workspace_bytes,
)
