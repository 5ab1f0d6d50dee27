"""GPU: the verification pass inside a decode loop, against the fp64 oracle at every
intermediate context.

Each step drafts T tokens (fresh queries and draft K/V), runs the verification pass
(selection + sparse multi-draft attention; alternately through sv_select_and_attend
and through the separate calls), accepts 1..T of the drafts per sequence and appends
their K/V with sv_block_repr, which also refreshes the representatives of the blocks
the new tokens land in (sciencestack page, Figure 1 caption: KV blocks of prefix
tokens). The contexts start just below the 4096-token dense threshold, so the loop
crosses from dense to sparse verification and over many block boundaries, with
partly filled tail blocks along the way.

With periodic full verification (SpecPV page, highlights and introduction: a full
verification every few steps keeps errors from accumulating), every `full_every`-th
step verifies against every block, through the same entry points, and is followed by
a refresh: the cached K/V of the tokens accepted since the previous full verification
(all but the newest step's) are rewritten in place with sv_block_repr (ctx_after =
the current context), standing in for recomputed states, and the representatives of
the blocks they touch are re-derived. The following steps must match the oracle on
the refreshed cache.
"""

import numpy as np
import pytest
import torch

from block_sparse_speculative_amd import _lib as L
from block_sparse_speculative_amd import pipeline as PL
from block_sparse_speculative_amd import synth

import parity as PT

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
DENSE_ALL = 1 << 30       # dense_ctx_tokens of a full verification


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def run_loop(bs: int, steps: int, full_every: int = 0, seed: int = 0, head_dim: int = 128):
    _gpu()
    dev = torch.device("cuda")
    B, Hq, Hkv, T, D = 2, 8, 2, 8, head_dim
    G = Hq // Hkv
    start = [4096 - 150, 4096 - 37]
    sparse_budget = (4096, 16, 50, 1, 1)
    cap = max(start) + steps * T + bs
    NB = -(-cap // bs)
    w = W["llama32k"].with_(num_seqs=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                            block_size=bs, num_draft=T, ctx=(cap,) * B, budget=sparse_budget)
    # Logical K/V of the whole capacity (planted heavy blocks included) and the base query.
    x = synth.make_layer(w, seed, 0, dev)
    logical_k = _np(x["k_ctx"])            # [B, cap, Hkv, D], bf16 values in float64
    logical_v = _np(x["v_ctx"])
    q_base = x["q"].float()
    P = B * NB
    gen = torch.Generator().manual_seed(1000 + seed)
    table = torch.randperm(P, generator=gen).to(torch.int32).reshape(B, NB).to(dev)
    table_host = table.cpu()
    shape = L.make_shape(B, Hq, Hkv, D, bs, NB, P, T, torch.bfloat16)
    pool = PL.alloc_pool(shape, dev, fill_nan=True)
    ctx = list(start)
    PL.append(shape, pool, x["k_ctx"][:, :max(start)].contiguous(),
              x["v_ctx"][:, :max(start)].contiguous(),
              torch.tensor(ctx, dtype=torch.int32, device=dev),
              torch.zeros(B, dtype=torch.int32, device=dev), table)
    del x
    scale = 1.0 / np.sqrt(D)
    g_dev = torch.Generator(device=dev).manual_seed(2000 + seed)
    last_full = list(start)
    stats = dict(steps=0, sparse_steps=0, dense_steps=0, full_steps=0, refreshes=0,
                 max_abs=0.0, bound=0.0, lse=0.0, near_tie=0, tail_partial=0)
    crossed = [False] * B
    for step in range(steps):
        full = full_every > 0 and step % full_every == full_every - 1
        budget = L.make_budget(DENSE_ALL if full else 4096, 16, 50)
        budget_t = (DENSE_ALL if full else 4096, 16, 50, 1, 1)
        ks = [L.budget_blocks(budget, c, bs) for c in ctx]
        k_max = max(ks)
        q = (q_base + 0.3 * torch.randn(q_base.shape, generator=g_dev, device=dev)).to(torch.bfloat16)
        kd = torch.randn((B, T, Hkv, D), generator=g_dev, device=dev).to(torch.bfloat16)
        vd = torch.randn((B, T, Hkv, D), generator=g_dev, device=dev).to(torch.bfloat16)
        ctx_t = torch.tensor(ctx, dtype=torch.int32, device=dev)
        idx = torch.full((B, Hkv, k_max), -7, dtype=torch.int32, device=dev)
        cnt = torch.full((B, Hkv), -7, dtype=torch.int32, device=dev)
        out = torch.full((B, T, Hq, D), float("nan"), dtype=torch.bfloat16, device=dev)
        lse = torch.full((B, T, Hq), float("nan"), dtype=torch.float32, device=dev)
        if step % 2 == 0:
            ws = torch.zeros(L.select_and_attend_workspace_bytes(shape, k_max), dtype=torch.uint8,
                             device=dev)
            L.select_and_attend(shape, budget, q, pool.reps, kd, vd, pool.k, pool.v, table, ctx_t,
                                k_max, scale, idx, cnt, out, lse=lse, ws=ws)
        else:
            wsel = torch.empty(L.select_workspace_bytes(shape, k_max), dtype=torch.uint8,
                               device=dev)
            L.select_blocks(shape, budget, q, pool.reps, table, ctx_t, k_max, idx, cnt, ws=wsel)
            n = L.attn_workspace_bytes(shape, k_max)
            wa = torch.zeros(max(n, 1), dtype=torch.uint8, device=dev)
            L.sparse_verify_attn(shape, q, kd, vd, pool.k, pool.v, table, ctx_t, idx, cnt, k_max,
                                 scale, out, lse=lse, ws=wa if n else None)
        torch.cuda.synchronize()
        # ---- the verification pass against the oracle at this context
        qh, kdh, vdh = _np(q), _np(kd), _np(vd)
        idx_h, cnt_h = idx.cpu(), cnt.cpu()
        out_h, lse_h = _np(out), _np(lse)
        reps_h = _np(pool.reps)
        for b in range(B):
            nb = -(-ctx[b] // bs)
            if ctx[b] % bs:
                stats["tail_partial"] += 1
            for g in range(Hkv):
                sl = slice(g, g + 1)
                u = PT.UnitInputs(q=qh[b, :, g * G:(g + 1) * G], k_ctx=logical_k[b, :ctx[b], sl],
                                  v_ctx=logical_v[b, :ctx[b], sl], k_draft=kdh[b, :, sl],
                                  v_draft=vdh[b, :, sl], ctx=ctx[b])
                reps, scores, k, osel = PT.oracle_select(u, bs, budget_t, G)
                assert int(cnt_h[b, g]) == min(k, nb)
                gsel = PT.gpu_unit_selection(idx_h, cnt_h, b, g)
                kind = PT.check_selection(gsel, osel, scores, k, nb, 1, 1)
                stats["near_tie"] += kind == "near-tie"
                if k >= nb:
                    stats["dense_steps"] += 1
                else:
                    stats["sparse_steps"] += 1
                phys = table_host[b, :nb].numpy()
                PT.check_reps(reps_h[phys, g], u, bs, reps)
                e = PT.check_output(out_h[b, :, g * G:(g + 1) * G], lse_h[b, :, g * G:(g + 1) * G],
                                    u, np.array(gsel), bs, scale, "bf16")
                for key in ("max_abs", "bound", "lse"):
                    stats[key] = max(stats[key], e.get(key, 0.0))
            if ctx[b] > 4096 and not full:
                crossed[b] = True
        stats["steps"] += 1
        stats["full_steps"] += int(full)
        # ---- accept 1..T drafts per sequence and append their K/V
        acc = [int(torch.randint(1, T + 1, (1,), generator=gen)) for _ in range(B)]
        acc = [min(a, cap - c) for a, c in zip(acc, ctx)]
        PL.append(shape, pool, kd, vd, torch.tensor(acc, dtype=torch.int32, device=dev),
                  ctx_t, table)
        for b in range(B):
            logical_k[b, ctx[b]:ctx[b] + acc[b]] = kdh[b, :acc[b]]
            logical_v[b, ctx[b]:ctx[b] + acc[b]] = vdh[b, :acc[b]]
        ctx = [c + a for c, a in zip(ctx, acc)]
        # ---- refresh after a full verification: rewrite the tokens accepted since the
        # previous one (all but the newest step's) in place
        if full:
            lo = list(last_full)
            hi = [c - a for c, a in zip(ctx, acc)]
            n = [max(0, h - l_) for l_, h in zip(lo, hi)]
            if max(n) > 0:
                kn = torch.randn((B, max(n), Hkv, D), generator=g_dev, device=dev).to(torch.bfloat16)
                vn = torch.randn((B, max(n), Hkv, D), generator=g_dev, device=dev).to(torch.bfloat16)
                PL.append(shape, pool, kn, vn, torch.tensor(n, dtype=torch.int32, device=dev),
                          torch.tensor(lo, dtype=torch.int32, device=dev), table,
                          ctx_after=torch.tensor(ctx, dtype=torch.int32, device=dev))
                knh, vnh = _np(kn), _np(vn)
                for b in range(B):
                    logical_k[b, lo[b]:lo[b] + n[b]] = knh[b, :n[b]]
                    logical_v[b, lo[b]:lo[b] + n[b]] = vnh[b, :n[b]]
                stats["refreshes"] += 1
            last_full = list(ctx)
    # the loop covered what it is meant to cover
    assert all(crossed), "a sequence never crossed the dense threshold"
    assert stats["dense_steps"] > 0 and stats["sparse_steps"] > 0 and stats["tail_partial"] > 0
    assert all(c // bs > s // bs + 1 for c, s in zip(ctx, start)), "fewer than two block boundaries"
    if full_every:
        assert stats["full_steps"] >= 2 and stats["refreshes"] >= 2
    PT.log(f"  {stats}")
    return stats


@pytest.mark.parametrize("bs", [32, 64])
def test_decode_loop_verify_accept_append(bs):
    st = run_loop(bs, steps=2 * bs, seed=bs)
    PT.record(f"decode loop bs{bs} ({st['steps']} steps)", units=st["steps"] * 4,
              max_abs=st["max_abs"], bound=st["bound"], lse=st["lse"])


@pytest.mark.parametrize("bs", [32, 128])
def test_periodic_full_verification_with_refresh(bs):
    st = run_loop(bs, steps=2 * 32, full_every=4, seed=7 + bs, head_dim=64 if bs == 128 else 128)
    PT.record(f"full every 4 + refresh bs{bs}", units=st["steps"] * 4, max_abs=st["max_abs"],
              bound=st["bound"], lse=st["lse"])
