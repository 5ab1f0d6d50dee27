"""GPU: sv_select_and_attend_static, the allocation-free variant of sv_select_and_attend
(its workspace is the library's static per-device scratch), called through the C ABI,
must give exactly what sv_select_and_attend gives with a caller-owned workspace, on
consecutive calls of different sizes sharing that scratch."""

import pytest
import torch

from block_sparse_speculative_amd import _lib as L
from block_sparse_speculative_amd import synth
from block_sparse_speculative_amd.workload import Instance

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _call(inst, splits, static):
    ly = inst.layers[0]
    idx, cnt = torch.full_like(ly.idx, -9), torch.full_like(ly.cnt, -9)
    out, lse = torch.full_like(ly.out, float("nan")), torch.full_like(ly.lse, float("nan"))
    args = (inst.shape, inst.budget, ly.q, ly.pool.reps, ly.k_draft, ly.v_draft, ly.pool.k,
            ly.pool.v, inst.table, inst.ctx, inst.k_max, inst.scale, idx, cnt, out)
    if static:
        L.select_and_attend_static(*args, lse=lse, num_splits=splits,
                                   draft_mask=inst.draft_mask)
    else:
        ws = torch.zeros(L.select_and_attend_workspace_bytes(inst.shape, inst.k_max, splits),
                         dtype=torch.uint8, device=inst.device)
        L.select_and_attend(*args, lse=lse, ws=ws, num_splits=splits, draft_mask=inst.draft_mask)
    return idx, cnt, out, lse


def test_static_scratch_entry_matches_the_workspace_entry():
    _gpu()
    # 32 units (the stack64k head layout at 8K context), then 2 units at a smaller
    # context (fewer units, fewer blocks), then the first shape again at another split
    # count: the scratch keeps the last call's contents in between.
    big = Instance(W["stack64k"].with_(num_layers=1, ctx=(8192,) * 4), seed=51, fused=True)
    small = Instance(W["llama32k"].with_(num_seqs=1, num_q_heads=8, num_kv_heads=2, ctx=(5000,),
                                         draft_tree="random"), seed=52, fused=True)
    for inst, splits in ((big, 0), (small, 0), (big, 5)):
        print(f"[no-alloc] units={inst.w.num_seqs * inst.w.num_kv_heads} splits={splits} "
              f"plan={L.attn_plan(inst.shape, inst.k_max, splits)}", flush=True)
        got = _call(inst, splits, static=True)
        torch.cuda.synchronize()
        want = _call(inst, splits, static=False)
        torch.cuda.synchronize()
        assert torch.isfinite(got[2].float()).all()
        for x, y in zip(got, want):
            assert torch.equal(x, y)
