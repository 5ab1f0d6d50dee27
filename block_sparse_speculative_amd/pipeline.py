"""Per-layer orchestration of the verification hot path on device buffers.

Everything here only allocates torch device buffers and calls the libsv entry
points; no step of the method is computed in Python.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import torch

from . import _lib as L


@dataclasses.dataclass
class Pool:
    """Paged KV pool of one layer (layouts as documented in include/sv.h)."""
    k: torch.Tensor       # [P, Hkv, bs, D]
    v: torch.Tensor       # [P, Hkv, bs, D]
    reps: torch.Tensor    # [P, Hkv, D] float32


def alloc_pool(shape: L.Shape, device="cuda", fill_nan: bool = False) -> Pool:
    P, Hkv, bs, D = shape.num_phys_blocks, shape.num_kv_heads, shape.block_size, shape.head_dim
    dt = torch.float32 if shape.dtype == L.SV_F32 else torch.bfloat16
    mk = torch.full if fill_nan else (lambda s, v, **kw: torch.empty(s, **kw))
    k = mk((P, Hkv, bs, D), float("nan"), dtype=dt, device=device)
    v = mk((P, Hkv, bs, D), float("nan"), dtype=dt, device=device)
    reps = mk((P, Hkv, D), float("nan"), dtype=torch.float32, device=device)
    return Pool(k, v, reps)


def append(shape: L.Shape, pool: Pool, k_new, v_new, n_new, ctx_before, block_table,
           ctx_after=None):
    """sv_block_repr over a batch of new tokens (k_new/v_new [B, n_max, Hkv, D]); with
    ctx_after the tokens rewrite cached positions of sequences of that length."""
    L.block_repr(shape, k_new, v_new, n_new, ctx_before, block_table, pool.k, pool.v, pool.reps,
                 ctx_after=ctx_after)


def fill_pool(shape: L.Shape, pool: Pool, k_ctx, v_ctx, ctx_lens, block_table, chunk: int = 0):
    """Write whole contexts into the pool (k_ctx/v_ctx [B, max_ctx, Hkv, D]).

    chunk > 0 appends in pieces of `chunk` tokens (as a decode loop would)."""
    B = shape.num_seqs
    dev = k_ctx.device
    lens = torch.as_tensor(ctx_lens, dtype=torch.int32, device=dev)
    max_ctx = int(k_ctx.shape[1])
    if chunk <= 0 or chunk >= max_ctx:
        append(shape, pool, k_ctx, v_ctx, lens, torch.zeros(B, dtype=torch.int32, device=dev),
               block_table)
        return
    for start in range(0, max_ctx, chunk):
        stop = min(max_ctx, start + chunk)
        n = (lens - start).clamp(min=0, max=stop - start).to(torch.int32)
        before = torch.minimum(lens, torch.full_like(lens, start)).to(torch.int32)
        append(shape, pool, k_ctx[:, start:stop].contiguous(), v_ctx[:, start:stop].contiguous(),
               n, before, block_table)


class Workspaces:
    """Caller-owned workspaces of the selection and attention entry points."""

    def __init__(self, shape: L.Shape, k_max: int, num_splits: int = 0, device="cuda"):
        self.sel = torch.empty(max(L.select_workspace_bytes(shape, k_max), 1), dtype=torch.uint8,
                               device=device)
        n = L.attn_workspace_bytes(shape, k_max, num_splits)
        # zero-filled once: the attention workspaces start with the merge words
        self.attn = torch.zeros(n, dtype=torch.uint8, device=device) if n else None
        self.fused = torch.zeros(L.select_and_attend_workspace_bytes(shape, k_max, num_splits),
                                 dtype=torch.uint8, device=device)
        self.num_splits = num_splits


def select(shape, budget, q, pool: Pool, block_table, ctx_lens, k_max, idx, cnt, ws: Workspaces,
           scores: Optional[torch.Tensor] = None):
    L.select_blocks(shape, budget, q, pool.reps, block_table, ctx_lens, k_max, idx, cnt,
                    scores=scores, ws=ws.sel)


def select_and_attend(shape, budget, q, k_draft, v_draft, pool: Pool, block_table, ctx_lens,
                      k_max, scale, idx, cnt, out, ws: Workspaces, lse=None, draft_mask=None):
    L.select_and_attend(shape, budget, q, pool.reps, k_draft, v_draft, pool.k, pool.v,
                        block_table, ctx_lens, k_max, scale, idx, cnt, out, lse=lse,
                        ws=ws.fused, num_splits=ws.num_splits, draft_mask=draft_mask)


def attend(shape, q, k_draft, v_draft, pool: Pool, block_table, ctx_lens, idx, cnt, k_max, scale,
           out, ws: Workspaces, lse=None, draft_mask=None):
    L.sparse_verify_attn(shape, q, k_draft, v_draft, pool.k, pool.v, block_table, ctx_lens, idx,
                         cnt, k_max, scale, out, lse=lse, ws=ws.attn, num_splits=ws.num_splits,
                         draft_mask=draft_mask)
