"""Seeded synthetic inputs for verification attention.

This module only draws random tensors with the shapes, value distributions and
structure of the workloads (model head shapes, context lengths, paged block tables,
planted heavy blocks, correlated draft queries). It contains none of the method's
arithmetic: it never computes representatives, scores, selections or attention.
Both the HIP path and the CPU oracle consume exactly the tensors it returns.

Workload recipes (shapes follow Llama-3.1-8B and Qwen3-30B-A3B attention, the two
models evaluated on the tutorial page "Accelerate Speculative Decoding with Sparse
Computation in Verification", section "Experiments"; datasets are replaced by
seeded Gaussian data):

* tiny      1 seq, 8/2 heads, d 64, fp32, ctx 2048, block 32, T 4, budget 16 blocks,
            4 planted blocks (+2.0 * q_hat), iid queries.
* llama32k  1 seq, 32/8 heads, d 128, bf16, ctx 32768, block 64, T 8; dense if
            ctx <= 4096 else max(64, 5%); 3% planted (+1.5 * q_hat); drafts rho 0.8.
* ragged    16 seqs, ctx uniform in [4096, 65536] rounded down to 64, paged KV with
            a random block table, otherwise as llama32k.
* stack64k  32 layers, 4 seqs, ctx 65536, as llama32k; even layers select, odd layers
            reuse; the planted set of an odd layer keeps 80% of the previous layer's.
* qwen128k  2 seqs, 32/4 heads, d 128, bf16, ctx 131072, block 128, T 16;
            budget max(128, 3%), 2% planted (+1.5 * q_hat).

q_hat of KV head g is the unit vector along the sum of the first draft token's
queries of the heads in that GQA group (computed from the rounded queries).

Draft trees (any workload, draft_tree != "chain"): draft 0 is the root; in a
"random" tree the parent of draft t >= 1 is uniform over drafts 0..t-1, drawn per
sequence; in a "star" every draft t >= 1 hangs off the root.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional, Tuple

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str                     # "fp32" | "bf16"
    block_size: int
    num_draft: int
    num_layers: int
    ctx: Tuple[int, ...]           # fixed context per sequence (empty -> ctx_range)
    ctx_range: Optional[Tuple[int, int]]
    budget: Tuple[int, int, int, int, int]   # dense_ctx, min_blocks, frac_per_mille, keep_first, keep_last
    plant_count: Optional[int]     # fixed number of planted blocks per (seq, kv head)
    plant_percent: Optional[int]   # else round-half-up(percent * nb / 100)
    plant_alpha: float
    draft_rho: Optional[float]     # None -> iid draft queries
    paged: bool                    # random physical block table
    reuse_odd_layers: bool
    pair_overlap: float = 0.8
    draft_tree: str = "chain"      # "chain" | "random" | "star"

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 8, 2, 64, "fp32", 32, 4, 1, (2048,), None,
                     (0, 16, 0, 1, 1), 4, None, 2.0, None, False, False),
    "llama32k": Workload("llama32k", 1, 32, 8, 128, "bf16", 64, 8, 1, (32768,), None,
                         (4096, 64, 50, 1, 1), None, 3, 1.5, 0.8, False, False),
    "ragged": Workload("ragged", 16, 32, 8, 128, "bf16", 64, 8, 1, (), (4096, 65536),
                       (4096, 64, 50, 1, 1), None, 3, 1.5, 0.8, True, False),
    "stack64k": Workload("stack64k", 4, 32, 8, 128, "bf16", 64, 8, 32, (65536,) * 4, None,
                         (4096, 64, 50, 1, 1), None, 3, 1.5, 0.8, False, True),
    "qwen128k": Workload("qwen128k", 2, 32, 4, 128, "bf16", 128, 16, 1, (131072,) * 2, None,
                         (0, 128, 30, 1, 1), None, 2, 1.5, 0.8, False, False),
}


def _gen(seed: int, stream: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) * 1_000_003 + int(stream) * 7919 + 12345) % (2 ** 63 - 1))
    return g


def num_blocks(ctx: int, bs: int) -> int:
    return -(-ctx // bs)


def context_lengths(w: Workload, seed: int):
    """Per-sequence context lengths (host ints)."""
    if w.ctx:
        return [int(c) for c in w.ctx]
    lo, hi = w.ctx_range
    g = _gen(seed, 999_001, "cpu")
    u = torch.randint(lo, hi + 1, (w.num_seqs,), generator=g)
    return [int(x) // 64 * 64 for x in u.tolist()]


def block_table(w: Workload, ctx_lens, seed: int):
    """[B, max_nb] int32 logical->physical map and the pool size P.

    Unpaged workloads use the identity layout (sequence b owns rows b*max_nb..).
    Paged workloads scatter every sequence's blocks over a seeded permutation of
    P = sum(nb_b) physical blocks. Entries past a sequence's nb are 0 (never read).
    """
    bs = w.block_size
    nbs = [num_blocks(c, bs) for c in ctx_lens]
    max_nb = max(max(nbs), 1)
    table = torch.zeros((w.num_seqs, max_nb), dtype=torch.int32)
    if not w.paged:
        for b in range(w.num_seqs):
            table[b, : nbs[b]] = torch.arange(nbs[b], dtype=torch.int32) + b * max_nb
        return table, w.num_seqs * max_nb
    total = sum(nbs)
    perm = torch.randperm(total, generator=_gen(seed, 999_002, "cpu")).to(torch.int32)
    off = 0
    for b in range(w.num_seqs):
        table[b, : nbs[b]] = perm[off: off + nbs[b]]
        off += nbs[b]
    return table, max(total, 1)


def planted_count(w: Workload, nb: int) -> int:
    if w.plant_count is not None:
        return w.plant_count
    return (w.plant_percent * nb + 50) // 100


def planted_sets(w: Workload, ctx_lens, seed: int, layer: int):
    """Heavy blocks per (seq, kv head): list[B][Hkv] of sorted int lists.

    Drawn without replacement from the non-forced blocks 1..nb-2. For layer stacks
    with reuse, odd layer 2p+1 keeps round(overlap * n) blocks of layer 2p's set and
    adds fresh blocks outside it.
    """
    out = []
    base_layer = layer - (layer % 2) if w.reuse_odd_layers else layer
    g_base = _gen(seed, 1000 + base_layer, "cpu")
    g_odd = _gen(seed, 5000 + layer, "cpu")
    for b, ctx in enumerate(ctx_lens):
        nb = num_blocks(ctx, w.block_size)
        row = []
        for _ in range(w.num_kv_heads):
            n = min(planted_count(w, nb), max(nb - 2, 0))
            pool = torch.randperm(max(nb - 2, 0), generator=g_base) + 1
            base = pool[:n]
            if w.reuse_odd_layers and layer % 2 == 1 and n > 0:
                keep_n = int(math.floor(w.pair_overlap * n + 0.5))
                keep = base[torch.randperm(n, generator=g_odd)[:keep_n]]
                rest = pool[n:]
                fresh = rest[torch.randperm(rest.numel(), generator=g_odd)[: n - keep_n]]
                chosen = torch.cat([keep, fresh])
            else:
                chosen = base
            row.append(sorted(int(x) for x in chosen.tolist()))
        out.append(row)
    return out


def make_layer(w: Workload, seed: int, layer: int = 0, device="cpu", ctx_lens=None):
    """Draw one layer's inputs.

    Returns dict with
      q        [B, T, Hq, D]      (dtype)
      k_ctx    [B, max_ctx, Hkv, D] (dtype; tokens past ctx_b are zero)
      v_ctx    [B, max_ctx, Hkv, D]
      k_draft  [B, T, Hkv, D], v_draft likewise
      ctx_lens list[int], heavy list[B][Hkv]
    """
    dev = torch.device(device)
    if ctx_lens is None:
        ctx_lens = context_lengths(w, seed)
    B, T, Hq, Hkv, D, bs = (w.num_seqs, w.num_draft, w.num_q_heads, w.num_kv_heads,
                            w.head_dim, w.block_size)
    max_ctx = max(max(ctx_lens), 1)
    dt = w.torch_dtype
    g = _gen(seed, 2000 + layer, dev)

    q0 = torch.randn((B, 1, Hq, D), generator=g, device=dev)
    if T > 1:
        z = torch.randn((B, T - 1, Hq, D), generator=g, device=dev)
        if w.draft_rho is None:
            rest = z
        else:
            rho = w.draft_rho
            rest = rho * q0 + math.sqrt(1.0 - rho * rho) * z
        q = torch.cat([q0, rest], dim=1)
    else:
        q = q0
    q = q.to(dt)

    # Unit direction per (seq, kv head) along the group's summed first-draft query.
    qg = q[:, 0].float().reshape(B, Hkv, w.group, D).sum(dim=2)
    q_hat = qg / qg.norm(dim=-1, keepdim=True).clamp_min(1e-30)

    k = torch.randn((B, max_ctx, Hkv, D), generator=g, device=dev)
    heavy = planted_sets(w, ctx_lens, seed, layer)
    for b in range(B):
        for h in range(Hkv):
            blocks = heavy[b][h]
            if not blocks:
                continue
            tok = (torch.tensor(blocks, device=dev)[:, None] * bs
                   + torch.arange(bs, device=dev)[None, :]).reshape(-1)
            tok = tok[tok < ctx_lens[b]]
            k[b, tok, h, :] += w.plant_alpha * q_hat[b, h]
    k = k.to(dt)
    v = torch.randn((B, max_ctx, Hkv, D), generator=g, device=dev).to(dt)
    for b in range(B):
        if ctx_lens[b] < max_ctx:
            k[b, ctx_lens[b]:] = 0
            v[b, ctx_lens[b]:] = 0
    kd = torch.randn((B, T, Hkv, D), generator=g, device=dev).to(dt)
    vd = torch.randn((B, T, Hkv, D), generator=g, device=dev).to(dt)
    return dict(q=q, k_ctx=k, v_ctx=v, k_draft=kd, v_draft=vd, ctx_lens=list(ctx_lens),
                heavy=heavy)


def softmax_scale(w: Workload) -> float:
    return 1.0 / math.sqrt(w.head_dim)


def draft_parents(w: Workload, seed: int):
    """Parent draft of every draft token, per sequence ([B][T], -1 for the root), or
    None for chain drafts."""
    if w.draft_tree == "chain":
        return None
    T = w.num_draft
    if w.draft_tree == "star":
        return [[-1] + [0] * (T - 1) for _ in range(w.num_seqs)]
    if w.draft_tree != "random":
        raise ValueError(f"unknown draft tree {w.draft_tree!r}")
    g = _gen(seed, 7_000_001, "cpu")
    out = []
    for _ in range(w.num_seqs):
        par = [-1]
        for t in range(1, T):
            par.append(int(torch.randint(0, t, (1,), generator=g).item()))
        out.append(par)
    return out


def draft_mask(parents, num_draft: int) -> torch.Tensor:
    """The drafts each draft sees, as bits (int32 [B, T]): itself and its ancestors."""
    m = torch.zeros((len(parents), num_draft), dtype=torch.int32)
    for b, par in enumerate(parents):
        for t in range(num_draft):
            bits, x = 0, t
            while x >= 0:
                bits |= 1 << x
                x = par[x]
            m[b, t] = bits
    return m


# ---------------------------------------------------------------- sparse FFN inputs

@dataclasses.dataclass(frozen=True)
class FfnWorkload:
    """Inputs of the threshold-pruned FFN of one verification pass: the hidden states of
    the T draft tokens of one sequence (num_tokens rows) entering the FFN of one layer
    of Llama-3.1-8B's shape (d_model 4096, d_ffn 14336; the tutorial page's evaluated
    model), and the pruning threshold."""
    name: str
    num_tokens: int
    d_model: int
    d_ffn: int
    rho: float      # correlation of the draft tokens' hidden states (one shared component)
    tau: float      # pruning threshold on |SiLU(gate)|


FFN_WORKLOADS = {
    "ffn_llama8b": FfnWorkload("ffn_llama8b", 8, 4096, 14336, 0.9, 0.30),
}


def make_ffn(w: FfnWorkload, seed: int, device="cpu"):
    """Draw x [N, Dm] and the weights of one FFN layer, all rounded to bf16.

    x[t] = rho * x_shared + sqrt(1 - rho^2) * z_t with x_shared, z_t ~ N(0, I): the draft
    tokens of one sequence share most of their hidden state. w_gate and w_up ~
    N(0, 1/d_model) so a gate pre-activation is ~N(0, 1); w_down_t ~ N(0, 1/d_ffn).
    Returns dict(x, w_gate, w_up, w_down_t) of torch tensors on `device`."""
    dev = torch.device(device)
    g = _gen(seed, 3000, dev)
    n, dm, f = w.num_tokens, w.d_model, w.d_ffn
    shared = torch.randn((1, dm), generator=g, device=dev)
    z = torch.randn((n, dm), generator=g, device=dev)
    x = (w.rho * shared + math.sqrt(1.0 - w.rho * w.rho) * z).to(torch.bfloat16)
    wg = (torch.randn((f, dm), generator=g, device=dev) / math.sqrt(dm)).to(torch.bfloat16)
    wu = (torch.randn((f, dm), generator=g, device=dev) / math.sqrt(dm)).to(torch.bfloat16)
    wd = (torch.randn((f, dm), generator=g, device=dev) / math.sqrt(f)).to(torch.bfloat16)
    return dict(x=x, w_gate=wg, w_up=wu, w_down_t=wd)
