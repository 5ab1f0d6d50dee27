"""A resident instance of a workload: per-layer queries, draft K/V and paged KV pools
built on the device through sv_block_repr, plus the index/output buffers of a pass.

A verification pass over the instance runs, for every layer, either block selection
or inter-layer reuse, then the sparse multi-draft attention. Two ways to run it:
 - separate calls: sv_select_blocks or sv_reuse_indices (a copy of the previous
   layer's indices), then sv_sparse_verify_attn;
 - fused (the fast path): sv_select_and_attend on selecting layers, and on reuse
   layers sv_sparse_verify_attn reading the previous layer's index buffers
   themselves (the layer's idx / cnt ARE the previous layer's tensors).
"""

from __future__ import annotations

import dataclasses
from typing import List, Optional

import torch

from . import _lib as L
from . import pipeline as PL
from . import synth


@dataclasses.dataclass
class Layer:
    q: torch.Tensor
    k_draft: torch.Tensor
    v_draft: torch.Tensor
    pool: PL.Pool
    reuse: bool
    idx: torch.Tensor
    cnt: torch.Tensor
    out: torch.Tensor
    lse: Optional[torch.Tensor]


class Instance:
    def __init__(self, w: synth.Workload, seed: int = 0, device="cuda", num_layers: Optional[int] = None,
                 ctx_lens: Optional[List[int]] = None, paged: Optional[bool] = None,
                 num_splits: int = 0, with_lse: bool = True, nan_pool: bool = False,
                 k_max: Optional[int] = None, append_chunk: int = 0, progress=None,
                 fused: bool = False, layer_offset: int = 0, cap_selection: bool = False):
        if paged is not None:
            w = w.with_(paged=paged)
        self.w = w
        self.seed = seed
        # layer l of the instance is layer layer_offset + l of the workload (its inputs,
        # and whether it selects or reuses)
        self.layer_offset = layer_offset
        self.device = torch.device(device)
        self.ctx_lens = list(ctx_lens) if ctx_lens is not None else synth.context_lengths(w, seed)
        table, P = synth.block_table(w, self.ctx_lens, seed)
        self.table_host = table
        self.table = table.to(self.device)
        self.ctx = torch.tensor(self.ctx_lens, dtype=torch.int32, device=self.device)
        self.shape = L.make_shape(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                  w.block_size, table.shape[1], P, w.num_draft, w.torch_dtype)
        self.budget = L.make_budget(*w.budget)
        need = max([L.budget_blocks(self.budget, c, w.block_size) for c in self.ctx_lens] + [1])
        # k_max is at least every sequence's budget, unless cap_selection asks for the
        # given k_max as it is (below a budget it caps the selection)
        self.k_max = k_max if (cap_selection and k_max) else max(need, k_max or 0)
        self.scale = synth.softmax_scale(w)
        self.ws = PL.Workspaces(self.shape, self.k_max, num_splits, self.device)
        self.num_splits = L.attn_num_splits(self.shape, self.k_max, num_splits)
        self.plan = L.attn_plan(self.shape, self.k_max, num_splits)
        self.fused = fused
        # Draft tree (None: chain drafts) and its visibility bits on the device.
        self.parents = synth.draft_parents(w, seed)
        self.draft_mask = (None if self.parents is None else
                           synth.draft_mask(self.parents, w.num_draft).to(self.device))
        n_layers = w.num_layers if num_layers is None else num_layers
        B, T, Hq, Hkv, D = w.num_seqs, w.num_draft, w.num_q_heads, w.num_kv_heads, w.head_dim
        self.layers: List[Layer] = []
        for l in range(n_layers):
            x = synth.make_layer(w, seed, layer_offset + l, self.device, self.ctx_lens)
            pool = PL.alloc_pool(self.shape, self.device, fill_nan=nan_pool)
            PL.fill_pool(self.shape, pool, x["k_ctx"], x["v_ctx"], self.ctx_lens, self.table,
                         chunk=append_chunk)
            reuse = w.reuse_odd_layers and (layer_offset + l) % 2 == 1 and l > 0
            if reuse and fused:
                idx, cnt = self.layers[l - 1].idx, self.layers[l - 1].cnt
            else:
                idx = torch.full((B, Hkv, self.k_max), -7, dtype=torch.int32, device=self.device)
                cnt = torch.full((B, Hkv), -7, dtype=torch.int32, device=self.device)
            self.layers.append(Layer(
                q=x["q"], k_draft=x["k_draft"], v_draft=x["v_draft"], pool=pool, reuse=reuse,
                idx=idx, cnt=cnt,
                out=torch.empty((B, T, Hq, D), dtype=w.torch_dtype, device=self.device),
                lse=torch.empty((B, T, Hq), dtype=torch.float32, device=self.device)
                if with_lse else None))
            del x
            if progress is not None:
                progress(l + 1, n_layers)

    def logical(self, layer: int):
        """Regenerate the logical (unpaged) inputs of the instance's layer `layer` on the
        device."""
        return synth.make_layer(self.w, self.seed, self.layer_offset + layer, self.device,
                                self.ctx_lens)

    def select_or_reuse(self, l: int, scores: Optional[torch.Tensor] = None):
        ly = self.layers[l]
        if ly.reuse:
            prev = self.layers[l - 1]
            L.reuse_indices(self.shape, self.k_max, prev.idx, prev.cnt, ly.idx, ly.cnt)
        else:
            PL.select(self.shape, self.budget, ly.q, ly.pool, self.table, self.ctx, self.k_max,
                      ly.idx, ly.cnt, self.ws, scores=scores)

    def attend(self, l: int):
        ly = self.layers[l]
        PL.attend(self.shape, ly.q, ly.k_draft, ly.v_draft, ly.pool, self.table, self.ctx, ly.idx,
                  ly.cnt, self.k_max, self.scale, ly.out, self.ws, lse=ly.lse,
                  draft_mask=self.draft_mask)

    def run_layer(self, l: int):
        ly = self.layers[l]
        if not self.fused:
            self.select_or_reuse(l)
            self.attend(l)
        elif ly.reuse:
            self.attend(l)        # idx / cnt alias the previous layer's
        else:
            PL.select_and_attend(self.shape, self.budget, ly.q, ly.k_draft, ly.v_draft, ly.pool,
                                 self.table, self.ctx, self.k_max, self.scale, ly.idx, ly.cnt,
                                 ly.out, self.ws, lse=ly.lse, draft_mask=self.draft_mask)

    def step(self):
        for l in range(len(self.layers)):
            self.run_layer(l)

    # --------------------------------------------------------------- accounting
    def selected_tokens(self) -> int:
        return selected_tokens(self.w, self.ctx_lens, len(self.layers))

    def algorithmic_bytes(self) -> int:
        return algorithmic_bytes(self.w, self.ctx_lens, len(self.layers))

    def units(self) -> int:
        """Verified (draft token, query head) rows per pass, summed over layers."""
        return self.w.num_seqs * self.w.num_draft * self.w.num_q_heads * len(self.layers)


def _select_layers(w: synth.Workload, num_layers: int) -> int:
    return sum(1 for l in range(num_layers) if not (w.reuse_odd_layers and l % 2 == 1))


def selected_tokens(w: synth.Workload, ctx_lens, num_layers: int) -> int:
    """Context tokens attended in one pass, summed over layers, sequences and KV heads
    (host arithmetic on the budget and the context lengths)."""
    budget = L.make_budget(*w.budget)
    bs = w.block_size
    total = 0
    for c in ctx_lens:
        nb = -(-c // bs)
        k = L.budget_blocks(budget, c, bs)
        if k >= nb:
            toks = c
        else:
            # a sparse selection always holds the last (possibly partial) block
            toks = k * bs - (nb * bs - c if budget.keep_last else 0)
        total += toks
    return total * w.num_kv_heads * num_layers


def algorithmic_bytes(w: synth.Workload, ctx_lens, num_layers: int) -> int:
    """Bytes of selected K/V read plus representatives scored in one pass; sequences
    whose budget keeps every block are not scored."""
    esz = 4 if w.dtype == "fp32" else 2
    kv = selected_tokens(w, ctx_lens, num_layers) * w.head_dim * 2 * esz
    budget = L.make_budget(*w.budget)
    bs = w.block_size
    scored_blocks = 0
    for c in ctx_lens:
        nb = -(-c // bs)
        if L.budget_blocks(budget, c, bs) < nb:
            scored_blocks += nb
    reps = scored_blocks * w.num_kv_heads * w.head_dim * 4
    return kv + reps * _select_layers(w, num_layers)


def all_bytes(w: synth.Workload, ctx_lens, num_layers: int, k_max: int, splits: int) -> int:
    """Every byte one pass reads or writes, counted once each (host arithmetic): the
    algorithmic bytes, plus per layer the queries, draft K/V, outputs and block table
    read by the attention, the indices and counts (written on selecting layers, read on
    every layer), and with more than one split the fp32 partials (O, max, denominator)
    written and read back once; selecting layers add the first-draft queries and table
    read by the scoring and the block scores written and read once."""
    esz = 4 if w.dtype == "fp32" else 2
    B, T, Hq, Hkv, D = w.num_seqs, w.num_draft, w.num_q_heads, w.num_kv_heads, w.head_dim
    nb_max = max(max(-(-c // w.block_size) for c in ctx_lens), 1)
    units = B * Hkv
    rows = T * (Hq // Hkv)
    per_layer = (2 * B * T * Hq * D * esz          # queries in, outputs out
                 + 2 * B * T * Hkv * D * esz       # draft K and V
                 + B * nb_max * 4                  # block table
                 + units * (k_max + 1) * 4)        # indices and counts read
    if splits > 1:
        per_layer += 2 * (splits + 1) * units * rows * (D + 2) * 4
    per_select = (units * (k_max + 1) * 4          # indices and counts written
                  + B * Hq * D * esz               # first-draft queries for the scores
                  + B * nb_max * 4                 # block table for the scores
                  + 2 * units * nb_max * 4)        # scores written and read
    return (algorithmic_bytes(w, ctx_lens, num_layers) + num_layers * per_layer
            + _select_layers(w, num_layers) * per_select)
