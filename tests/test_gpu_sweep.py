"""GPU: a seeded sweep over the supported envelope, every unit against the oracle.

Each case draws one combination of the sizes and options the named workloads hold
fixed: dtype, head dim, block size, KV heads (1-4), GQA group (1-8, not only powers
of two), draft count (so rows T*G are padded to the next MFMA tile), 1-3 sequences
with empty, sub-block, whole-block and ragged contexts, a budget (dense threshold,
minimum, fraction, forced first/last blocks), k_max at, above or below the budget
(below: the capped selection), split count, separate or fused calls, chain / random
tree / star drafts, paged or contiguous tables, and a second layer that selects
again or reuses the first layer's blocks. The case parameters are printed before
each case runs.
"""

import gc

import numpy as np
import pytest
import torch

from block_sparse_speculative_amd import synth
from block_sparse_speculative_amd.workload import Instance
from oracle import sparse_verify as O

import parity as PT
from test_gpu_parity import run_and_check

NUM_CASES = 256


def sweep_case(i: int):
    """(workload, instance keyword arguments, description) of sweep case i."""
    r = np.random.default_rng(7919 * i + 17)
    dtype = "bf16" if r.random() < 0.7 else "fp32"
    d = int(r.choice([64, 128]))
    bs = int(r.choice([32, 64, 128]))
    hkv = int(r.integers(1, 5))
    g = int(r.integers(1, 9))
    t = int(r.integers(1, min(16, 128 // g) + 1))
    nseq = int(r.integers(1, 4))
    ctx = []
    for _ in range(nseq):
        kind = int(r.integers(0, 5))
        if kind == 0:
            c = int(r.integers(0, bs))                  # empty, or inside the first block
        elif kind == 1:
            c = int(r.integers(1, 40)) * bs             # whole blocks
        else:
            c = int(r.integers(bs, 9000))               # ragged
        ctx.append(c)
    ctx[0] = max(ctx[0], 3 * bs)
    if i % 16 == 5:
        # every 16th draw from 5 on: a row of more than 1024 blocks (the separate top-k
        # kernel, also behind the fused call)
        bs = 32
        ctx[0] = int(np.random.default_rng(1_000_003 + i).integers(33_000, 45_000))
    kf, kl = int(r.integers(0, 2)), int(r.integers(0, 2))
    forced = kf + kl
    budget = (int(r.choice([0, 2048, 6000])), int(r.integers(max(forced, 1), 25)),
              int(r.choice([0, 30, 100, 400])), kf, kl)
    need = max(O.budget_blocks(c, bs, *budget[:3]) for c in ctx)
    max_nb = max(-(-c // bs) for c in ctx)
    mode = int(r.integers(0, 3))
    if mode == 0:
        k_max, cap = None, False
    elif mode == 1:
        k_max, cap = min(max_nb, need + int(r.integers(1, 11))), False
    else:
        k_max, cap = int(r.integers(max(forced, 1), max(need, max(forced, 1)) + 1)), True
    splits = int(r.choice([0, 0, 1, 2, 3, 7, 20]))
    if i % 16 == 9:
        splits = 40   # every 16th draw from 9 on: the merge kernel when k_max allows it
    fused = bool(r.integers(0, 2))
    tree = str(r.choice(["chain", "random", "star"]))
    paged = bool(r.integers(0, 2))
    reuse = bool(r.integers(0, 2))
    w = synth.WORKLOADS["tiny"].with_(
        name=f"sweep{i}", num_seqs=nseq, num_q_heads=hkv * g, num_kv_heads=hkv,
        head_dim=d, dtype=dtype, block_size=bs, num_draft=t, num_layers=2,
        ctx=tuple(ctx), ctx_range=None, budget=budget,
        plant_count=int(r.integers(0, 6)), plant_percent=None,
        draft_rho=0.8 if r.random() < 0.5 else None, paged=paged,
        reuse_odd_layers=reuse, draft_tree=tree)
    kw = dict(num_splits=splits, fused=fused, k_max=k_max, cap_selection=cap)
    desc = (f"{dtype} D{d} bs{bs} Hkv{hkv} G{g} T{t} ctx{ctx} budget{budget} "
            f"k_max={k_max}{' (cap)' if cap else ''} splits={splits} "
            f"{'fused' if fused else 'separate'} {tree} {'paged' if paged else 'contiguous'} "
            f"{'reuse' if reuse else 'select'}")
    return w, kw, desc


def test_sweep_cases_are_distinct_and_inside_the_envelope():
    seen = set()
    for i in range(NUM_CASES):
        w, kw, desc = sweep_case(i)
        assert w.num_draft * w.group <= 128 and w.head_dim in (64, 128)
        assert kw["k_max"] is None or kw["k_max"] >= w.budget[3] + w.budget[4]
        seen.add(desc)
    assert len(seen) == NUM_CASES


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(NUM_CASES))
def test_sweep_case_all_units(i):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w, kw, desc = sweep_case(i)
    PT.log(f"[sweep {i}] {desc}")
    inst = Instance(w, seed=100 + i, nan_pool=True, **kw)
    PT.log(f"  resolved splits={inst.num_splits} k_max={inst.k_max} plan={inst.plan}")
    run_and_check(inst, case=f"sweep {i}")
    del inst
    gc.collect()
    torch.cuda.empty_cache()
