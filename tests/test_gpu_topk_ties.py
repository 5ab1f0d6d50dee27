"""GPU top-k on exact score ties, through sv_select_blocks and sv_select_and_attend.

Keys are constant per block with small integer values and the first query is all
ones, so every block score is the exact integer 2 * D * v_j in float32 and in fp64:
many blocks tie exactly, including +0 against -0. The oracle's selection (lowest
index wins a tie) must then match bit for bit, with no near-tie allowance; the
cases hit both ways the threshold search can end (more tied blocks than places
left, and exactly as many).
"""

import numpy as np
import pytest
import torch

from block_sparse_speculative_amd import _lib as L
from block_sparse_speculative_amd import pipeline as PL

import oracle as O
import parity as PT

pytestmark = pytest.mark.gpu

D, BS, T, HQ, HKV = 64, 32, 2, 2, 1


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _block_values(nb, case, rng):
    v = rng.integers(-3, 0, size=nb).astype(np.float32)       # negatives by default
    if case == "ties_exceed":      # 20 tied top blocks for 14 free places
        top = rng.choice(np.arange(1, nb - 1), size=20, replace=False)
        v[top] = 3.0
    elif case == "ties_exact":     # exactly 14 tied top blocks
        top = rng.choice(np.arange(1, nb - 1), size=14, replace=False)
        v[top] = 3.0
    elif case == "signed_zero":    # 10 top blocks, then +0 / -0 blocks share the cut
        rest = rng.permutation(np.arange(1, nb - 1))
        v[rest[:10]] = 2.0
        v[rest[10:22]] = 0.0
        v[rest[22:34]] = -0.0
    return v


@pytest.mark.parametrize("nb", [100, 1100])
@pytest.mark.parametrize("case", ["ties_exceed", "ties_exact", "signed_zero"])
@pytest.mark.parametrize("fused", [False, True])
def test_exact_ties_lowest_index(nb, case, fused):
    _gpu()
    PT.log(f"[ties] nb={nb} case={case} fused={fused}")
    dev = torch.device("cuda")
    rng = np.random.default_rng(1000 + nb)
    ctx = nb * BS
    vals = _block_values(nb, case, rng)
    k_ctx = torch.from_numpy(np.repeat(vals, BS)[None, :, None, None] *
                             np.ones((1, 1, HKV, D), np.float32)).to(dev)
    k_ctx = k_ctx.to(torch.bfloat16)
    gen = torch.Generator(device=dev).manual_seed(nb)
    v_ctx = torch.randn((1, ctx, HKV, D), generator=gen, device=dev).to(torch.bfloat16)
    q = torch.randn((1, T, HQ, D), generator=gen, device=dev)
    q[:, 0] = 1.0
    q = q.to(torch.bfloat16)
    k_draft = torch.randn((1, T, HKV, D), generator=gen, device=dev).to(torch.bfloat16)
    v_draft = torch.randn((1, T, HKV, D), generator=gen, device=dev).to(torch.bfloat16)
    table = torch.arange(nb, dtype=torch.int32, device=dev)[None]
    ctx_t = torch.tensor([ctx], dtype=torch.int32, device=dev)
    shape = L.make_shape(1, HQ, HKV, D, BS, nb, nb, T, torch.bfloat16)
    budget = L.make_budget(0, 16, 0, 1, 1)
    k_max = 16
    pool = PL.alloc_pool(shape, dev, fill_nan=True)
    PL.fill_pool(shape, pool, k_ctx, v_ctx, [ctx], table)
    ws = PL.Workspaces(shape, k_max, 0, dev)
    idx = torch.full((1, HKV, k_max), -7, dtype=torch.int32, device=dev)
    cnt = torch.full((1, HKV), -7, dtype=torch.int32, device=dev)
    out = torch.empty((1, T, HQ, D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((1, T, HQ), dtype=torch.float32, device=dev)
    scale = D ** -0.5
    if fused:
        PL.select_and_attend(shape, budget, q, k_draft, v_draft, pool, table, ctx_t, k_max, scale,
                             idx, cnt, out, ws, lse=lse)
    else:
        PL.select(shape, budget, q, pool, table, ctx_t, k_max, idx, cnt, ws)
        PL.attend(shape, q, k_draft, v_draft, pool, table, ctx_t, idx, cnt, k_max, scale, out, ws,
                  lse=lse)
    torch.cuda.synchronize()

    logical = {"q": q, "k_ctx": k_ctx, "v_ctx": v_ctx, "k_draft": k_draft, "v_draft": v_draft,
               "ctx_lens": [ctx]}
    u = PT.unit_inputs(logical, 0, 0, HQ // HKV)
    reps = O.block_representatives(u.k_ctx, BS)
    scores = O.block_scores(u.q[0], reps, HQ // HKV)[0]
    assert np.array_equal(scores, 2 * D * vals.astype(np.float64))
    osel = O.select_blocks(scores, 16, True, True)
    gsel = PT.gpu_unit_selection(idx.cpu(), cnt.cpu(), 0, 0)
    assert gsel == [int(x) for x in osel]
    PT.check_output(PT.np64(out)[0], PT.np64(lse)[0], u, np.array(gsel), BS, scale, "bf16")
