"""Plain, slow, fp64 reference for block-sparse multi-draft verification attention.

TEST INFRASTRUCTURE ONLY: used by ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``; never by the product path. It shares no
code, table or helper with the HIP library.

Sources (cited by short tag below):

* [TUT-T1]  Tutorial page "Accelerate Speculative Decoding with Sparse Computation in
  Verification" (agifrontier.github.io), section "Core technique 1: sparse attention
  for multiple tokens": blocks are chosen by the dot product of a draft query with a
  per-block representative value; a piecewise budget keeps many blocks for short
  contexts and sparsifies long ones; some layers reuse the previous layer's retrieval.
* [SS-F1]   sciencestack page for arXiv 2512.21911, Figure 1 caption: a KV block holds
  the key/value states of several prefix tokens; the selection uses the query of the
  FIRST draft token against each block's representative; all draft tokens share the
  selected set.
* [SS-ABS]  same page, Abstract: draft tokens are verified in one parallel pass; the
  framework reuses retrieval across draft tokens and across layers.
* [SPV-TREE] ebiotrade page on SpecPV, Introduction (the EAGLE-3 drafter searches and
  emits a tree of candidate tokens) and the excerpt on speculative decoding (SpecInfer
  organises the candidates as a token tree).

Readings taken where the pages leave a step open (each one is listed with its
justification in the design notes of the repository):

* R1 representative = arithmetic mean of the block's keys over its valid tokens.
* R2 the scorer is draft token t = 0 only.
* R3 one selection per KV head; its score sums the per-head dot products of the
  query heads in the GQA group.
* R4 unscaled dot product for scoring.
* R5 budget: k = nb if ctx <= dense_ctx_tokens, else min(nb, max(min_blocks,
  ceil(frac_per_mille * nb / 1000))).
* R6 first block and the block holding the last context token are forced in (when
  enabled) and count inside k.
* R7 ties go to the lower logical block index; NaN ranks as -inf.
* R8 selected indices are returned in ascending order.
* R9 softmax scale is an argument (1/sqrt(d) by convention).
* R10 draft token t sees every valid token of the selected blocks plus drafts 0..t.
* R11 a reuse layer takes the previous layer's selection unchanged.
* R17 draft trees: draft t has a parent draft (or none: it hangs off the context)
  that precedes it; draft t sees itself and its ancestors. The chain of R10 is the
  tree whose parent of t is t - 1. Selection still uses draft 0, the root.

All arithmetic is float64. Inputs may be float32 / bfloat16-valued arrays; they
are widened to float64 exactly.
"""

from __future__ import annotations

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def num_blocks(ctx_len: int, block_size: int) -> int:
    """Number of KV blocks covering ``ctx_len`` prefix tokens ([SS-F1]: a block holds
    several consecutive prefix tokens; the last one may be partly filled)."""
    return -(-int(ctx_len) // int(block_size))


def block_representatives(k_ctx, block_size: int):
    """Representative key of every block (reading R1; [TUT-T1], [SS-F1]).

    k_ctx: [ctx, Hkv, D] keys of one sequence in token order.
    Returns [nb, Hkv, D] float64: mean of the keys of the valid tokens of each block.
    """
    k = _f64(k_ctx)
    ctx = k.shape[0]
    nb = num_blocks(ctx, block_size)
    reps = np.zeros((nb, k.shape[1], k.shape[2]))
    for j in range(nb):
        lo = j * block_size
        hi = min(ctx, lo + block_size)
        reps[j] = k[lo:hi].sum(axis=0) / (hi - lo)
    return reps


def budget_blocks(ctx_len: int, block_size: int, dense_ctx_tokens: int,
                  min_blocks: int, frac_per_mille: int) -> int:
    """Piecewise block budget (reading R5; [TUT-T1] piecewise budget control).

    Short contexts (ctx <= dense_ctx_tokens) keep every block; longer ones keep
    max(min_blocks, ceil(frac * nb)) blocks, never more than nb.
    """
    nb = num_blocks(ctx_len, block_size)
    if ctx_len <= dense_ctx_tokens:
        return nb
    sparse = max(int(min_blocks), -(-int(frac_per_mille) * nb // 1000))
    return min(nb, sparse)


def block_scores(q_first, reps, group: int):
    """Importance score of every block for every KV head (readings R2-R4; [SS-F1]).

    q_first: [Hq, D] query of the first draft token; reps: [nb, Hkv, D].
    Query head h belongs to KV head h // group. Returns [Hkv, nb] float64 with
    score[g, j] = sum over heads h of group g of  q_first[h] . reps[j, g].
    """
    q = _f64(q_first)
    r = _f64(reps)
    hkv = r.shape[1]
    s = np.zeros((hkv, r.shape[0]))
    for g in range(hkv):
        for h in range(g * group, (g + 1) * group):
            s[g] += r[:, g, :] @ q[h]
    return s


def select_blocks(scores, k: int, keep_first: bool = True, keep_last: bool = True):
    """Top-k block selection of one KV head (readings R5-R8; [TUT-T1], [SS-F1]).

    scores: [nb]. Returns the ascending array of selected logical block indices.
    If k >= nb every block is kept. Otherwise the forced blocks (first, last) are
    kept and the remaining k - |forced| slots go to the highest-scoring other
    blocks, ties to the lower index, NaN treated as -inf.
    """
    s = _f64(scores)
    nb = s.shape[0]
    if k >= nb:
        return np.arange(nb, dtype=np.int64)
    forced = set()
    if keep_first:
        forced.add(0)
    if keep_last:
        forced.add(nb - 1)
    forced = sorted(forced)
    if k < len(forced):
        raise ValueError("budget smaller than the number of forced blocks")
    cand = np.array([j for j in range(nb) if j not in forced], dtype=np.int64)
    cs = s[cand]
    cs = np.where(np.isnan(cs), -np.inf, cs)
    # np.lexsort sorts by the LAST key first: descending score, then ascending index.
    order = np.lexsort((cand, -cs))
    chosen = cand[order[: k - len(forced)]]
    return np.sort(np.concatenate([np.array(forced, dtype=np.int64), chosen]))


def draft_visibility(parents, t_count: int):
    """The drafts each draft token attends to (readings R10, R17; [SPV-TREE]).

    parents: None for the chain, else a length-T sequence with parents[t] the parent
    draft of t (-1 for none); a parent must precede its child. Returns a list whose
    entry t is the ascending array of draft indices draft t sees: t and its ancestors.
    """
    if parents is None:
        return [np.arange(t + 1) for t in range(t_count)]
    par = [int(x) for x in parents]
    assert len(par) == t_count
    vis = []
    for t in range(t_count):
        seen = []
        x = t
        while x >= 0:
            assert x <= t and (x == t or x < seen[-1]), "a parent must precede its child"
            seen.append(x)
            x = par[x]
        vis.append(np.array(sorted(seen), dtype=np.int64))
    return vis


def verify_attention(q, k_ctx, v_ctx, k_draft, v_draft, selected, block_size: int,
                     scale: float, parents=None):
    """Multi-draft attention over the shared selected blocks (readings R9, R10, R17;
    [SS-F1] shared block set, [SS-ABS] parallel verification of draft tokens).

    q:        [T, Hq, D] draft-token queries
    k_ctx:    [ctx, Hkv, D] cached keys (token order), v_ctx likewise
    k_draft:  [T, Hkv, D] keys of the draft tokens themselves, v_draft likewise
    selected: sequence of length Hkv; selected[g] lists logical block indices
    parents:  None (chain) or the draft tree, as in draft_visibility
    Returns (out [T, Hq, D], lse [T, Hq]) in float64. For draft t and query head
    h of KV head g the key set is every valid token of the blocks in selected[g]
    followed by the drafts t sees (0..t for the chain, t and its ancestors in a
    tree); logits are scale * q.k; out is the softmax-weighted sum of values and lse
    the natural log of the softmax denominator.
    """
    qq = _f64(q)
    t_count, hq, d = qq.shape
    hkv = k_draft.shape[1]
    group = hq // hkv
    ctx = k_ctx.shape[0]
    vis = draft_visibility(parents, t_count)
    out = np.zeros((t_count, hq, d))
    lse = np.zeros((t_count, hq))
    for g in range(hkv):
        toks = [np.arange(j * block_size, min(ctx, (j + 1) * block_size))
                for j in selected[g]]
        toks = np.concatenate(toks) if toks else np.zeros(0, dtype=np.int64)
        kc = _f64(k_ctx[toks, g, :]).reshape(-1, d)
        vc = _f64(v_ctx[toks, g, :]).reshape(-1, d)
        for t in range(t_count):
            keys = np.concatenate([kc, _f64(k_draft[vis[t], g, :])], axis=0)
            vals = np.concatenate([vc, _f64(v_draft[vis[t], g, :])], axis=0)
            for h in range(g * group, (g + 1) * group):
                z = scale * (keys @ qq[t, h])
                m = z.max()
                e = np.exp(z - m)
                denom = e.sum()
                out[t, h] = (e @ vals) / denom
                lse[t, h] = m + np.log(denom)
    return out, lse


def merge_partials(outs, lses):
    """Combine attention results over disjoint key subsets (exact softmax identity).

    outs: [S, ..., D] normalised partial outputs; lses: [S, ...] their natural-log
    denominators. Returns (out, lse) equal to attention over the union of subsets.
    """
    o = _f64(outs)
    l = _f64(lses)
    top = l.max(axis=0)
    w = np.exp(l - top)
    total = w.sum(axis=0)
    out = (w[..., None] * o).sum(axis=0) / total[..., None]
    return out, top + np.log(total)


def verify_layer(q, k_ctx, v_ctx, k_draft, v_draft, ctx_lens, block_size: int,
                 scale: float, budget, prev_selection=None, parents=None):
    """One layer of the verification pass for a batch ([TUT-T1], [SS-F1]).

    q [B, T, Hq, D]; k_ctx/v_ctx [B, >=max ctx, Hkv, D]; k_draft/v_draft [B, T, Hkv, D];
    ctx_lens [B]; budget = (dense_ctx_tokens, min_blocks, frac_per_mille,
    keep_first, keep_last). If prev_selection is given (a reuse layer, reading R11)
    it is used unchanged and no scoring happens. parents: None (chain drafts) or
    [B][T] draft trees (reading R17).
    Returns dict(out [B,T,Hq,D], lse [B,T,Hq], selection [B][Hkv] arrays,
    scores [B] arrays [Hkv, nb] or None).
    """
    dense, min_blocks, frac, keep_first, keep_last = budget
    bsz, _, hq, d = q.shape
    hkv = k_draft.shape[2]
    group = hq // hkv
    out = np.zeros(q.shape)
    lse = np.zeros(q.shape[:3])
    selection, scores = [], []
    for b in range(bsz):
        ctx = int(ctx_lens[b])
        kc = k_ctx[b, :ctx]
        vc = v_ctx[b, :ctx]
        if prev_selection is not None:
            sel = [np.asarray(x, dtype=np.int64) for x in prev_selection[b]]
            sc = None
        else:
            reps = block_representatives(kc, block_size)
            sc = block_scores(q[b, 0], reps, group)
            kb = budget_blocks(ctx, block_size, dense, min_blocks, frac)
            sel = [select_blocks(sc[g], kb, keep_first, keep_last) for g in range(hkv)]
        out[b], lse[b] = verify_attention(q[b], kc, vc, k_draft[b], v_draft[b], sel,
                                          block_size, scale,
                                          None if parents is None else parents[b])
        selection.append(sel)
        scores.append(sc)
    return dict(out=out, lse=lse, selection=selection, scores=scores)
