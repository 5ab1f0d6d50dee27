"""Parity-test case definitions shared by the GPU tests and the CPU check that they
launch every attention build the library can pick.

A build is (dtype, head dim, tile tokens, padded rows, LDS ring, fused select): the
attention kernel is compiled once per such combination, and the library chooses one
from the shape, the split count and the grid size (sv_attn_plan_query reports which).
MATRIX holds one small workload per reachable (dtype, head dim, block size, rows)
class, each run at the library's split count, at one split, and at a split count that
puts more than 256 workgroups in the grid (the 64 KB-ring builds that share a CU),
through both the separate calls and the fused select-and-attend entry point.
"""

from __future__ import annotations

from block_sparse_speculative_amd import synth

W = synth.WORKLOADS

# ------------------------------------------------------------------ named small workloads

SMALL = {
    "tiny": W["tiny"],
    "llama_small": W["llama32k"].with_(num_seqs=2, num_q_heads=8, num_kv_heads=2, ctx=(8192, 6000)),
    "qwen_small": W["qwen128k"].with_(num_seqs=1, num_q_heads=16, num_kv_heads=2, ctx=(40000,)),
    "ragged_small": W["ragged"].with_(num_seqs=3, num_q_heads=8, num_kv_heads=2,
                                      ctx=(4096, 5000, 9000), ctx_range=None),
    "rows64": W["llama32k"].with_(num_q_heads=16, num_kv_heads=2, ctx=(7000,)),
    "d64_bs32": W["llama32k"].with_(head_dim=64, block_size=32, num_draft=2, num_q_heads=16,
                                    num_kv_heads=2, ctx=(3000,), budget=(0, 16, 100, 1, 1)),
    "fp32_d128": W["tiny"].with_(head_dim=128, block_size=64, ctx=(5000,),
                                 budget=(0, 12, 0, 1, 1), plant_count=4),
    "fp32_rows32_bs128": W["tiny"].with_(num_draft=8, block_size=128, ctx=(4500,),
                                         budget=(0, 8, 0, 1, 1)),
    # fp32 units of 64 and 128 rows (one workgroup per CU, 32-token tiles)
    "fp32_rows64_d64": W["tiny"].with_(num_q_heads=16, num_kv_heads=2, num_draft=8,
                                       ctx=(2500,)),
    "fp32_rows128_d128": W["tiny"].with_(num_q_heads=16, num_kv_heads=2, num_draft=16,
                                         head_dim=128, block_size=64, ctx=(3000,),
                                         budget=(0, 12, 0, 1, 1)),
    # more than 1024 blocks per row: LDS radix top-k, and the fused call's fallback
    "long_table": W["llama32k"].with_(num_seqs=1, num_q_heads=8, num_kv_heads=2, block_size=32,
                                      ctx=(40000,)),
}

EDGE = W["llama32k"].with_(num_seqs=4, num_q_heads=8, num_kv_heads=2, ctx=(0, 17, 200, 1000),
                           budget=(0, 2, 0, 1, 1))

TREES = {
    "llama_small": SMALL["llama_small"],
    "qwen_small": SMALL["qwen_small"],                  # T = 16: all 16 mask bits in use
    "fp32_rows32_bs128": SMALL["fp32_rows32_bs128"],
    "fp32_rows128_d128": SMALL["fp32_rows128_d128"],    # fp32, T = 16
    "edge": EDGE,                                       # ctx 0: the drafts alone
    "long_table": SMALL["long_table"],                  # > 1024 blocks: separate top-k
}

# ------------------------------------------------------------------ the build matrix

# (G, T) per row count: T * G rows of (draft token, query head) per unit.
ROWS = {16: (4, 4), 32: (4, 8), 64: (8, 8), 128: (8, 16)}

# Split count that puts more than 256 workgroups in the grid of a 16-unit workload
# (21 workgroups per unit: 336), with at most 32 per unit (the in-launch merge).
MANY_WG_SPLITS = 20


def matrix_workload(dtype: str, head_dim: int, block_size: int, rows: int) -> synth.Workload:
    """A small paged workload of 2 sequences x 8 KV heads (16 units) whose attention
    runs the build class (dtype, head_dim, block_size, rows). Contexts end inside a
    block (partly filled last tile) and keep 24 blocks per unit."""
    g, t = ROWS[rows]
    ctx = {32: (3000, 2100), 64: (5000, 3500), 128: (9000, 7000)}[block_size]
    base = W["tiny"] if dtype == "fp32" else W["llama32k"]
    return base.with_(name=f"m_{dtype}_d{head_dim}_bs{block_size}_r{rows}", num_seqs=2,
                      num_kv_heads=8, num_q_heads=8 * g, num_draft=t, head_dim=head_dim,
                      block_size=block_size, ctx=ctx, ctx_range=None, budget=(0, 24, 0, 1, 1),
                      plant_count=4, plant_percent=None, paged=True)


def matrix_classes():
    """(dtype, head_dim, block_size, rows) classes of the matrix."""
    out = []
    for d in (64, 128):
        for bs in (32, 64):
            for rows in (16, 32, 64, 128):
                out.append(("bf16", d, bs, rows))
        for rows in (32, 64, 128):          # bs 128: two 64-token tiles per block up to 64
            out.append(("bf16", d, 128, rows))   # rows, one 128-token tile above
        for rows in (16, 32, 64, 128):
            out.append(("fp32", d, 64, rows))
    return out


def matrix_cases():
    """(case id, workload, num_splits, fused) of every matrix run."""
    out = []
    for cls in matrix_classes():
        w = matrix_workload(*cls)
        for splits in (0, 1, MANY_WG_SPLITS):
            for fused in (False, True):
                out.append((f"{w.name}-s{splits}-{'fused' if fused else 'sep'}", w, splits,
                            fused))
    return out


def shape_of(w: synth.Workload):
    """sv_shape of a workload's instance (host arithmetic only; no device needed)."""
    from block_sparse_speculative_amd import _lib as L
    lens = synth.context_lengths(w, 0)
    table, P = synth.block_table(w, lens, 0)
    return L.make_shape(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size,
                        table.shape[1], P, w.num_draft, w.torch_dtype)


def k_max_of(w: synth.Workload) -> int:
    from block_sparse_speculative_amd import _lib as L
    budget = L.make_budget(*w.budget)
    return max([L.budget_blocks(budget, c, w.block_size) for c in synth.context_lengths(w, 0)]
               + [1])


def build_key(w: synth.Workload, num_splits: int, fused: bool):
    """The attention build a run of `w` launches: (dtype, D, tile tokens, padded rows,
    ring KB, fused select in the kernel)."""
    from block_sparse_speculative_amd import _lib as L
    shape = shape_of(w)
    plan = L.attn_plan(shape, k_max_of(w), num_splits)
    in_kernel_topk = fused and shape.max_blocks_per_seq <= 1024
    return (w.dtype, w.head_dim, plan["tile_tokens"], plan["padded_rows"], plan["ring_kb"],
            in_kernel_topk)
