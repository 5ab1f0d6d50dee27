"""GPU: seeded sequences of KV appends and rewrites through sv_block_repr, against a
logical model of the cache and the oracle's block representatives.

Each case draws a shape (dtype, head dim, block size, 1-4 KV heads, 1-3 sequences, a
paged table with spare physical blocks) and runs six calls on a pool that starts as
NaN. A call is either an append at each sequence's end (0 to 3 blocks' worth of
tokens, across block boundaries) or a rewrite with ctx_after: per sequence a range
starting anywhere in the cached tokens, which may run past the old end and so extend
the sequence (the refresh after a periodic full verification). After every call:
  - every valid token of every sequence sits in the pool bit for bit where the table
    maps it, and no physical block outside the table was written;
  - the representative of every valid block is within the fp32 summation bound of the
    oracle's mean over the block's valid keys.
At the end, the representatives equal bit for bit those of one bulk append of the
final cache: a block's mean does not depend on how its tokens arrived.
"""

import numpy as np
import pytest
import torch

from block_sparse_speculative_amd import _lib as L
from block_sparse_speculative_amd import pipeline as PL
from oracle import sparse_verify as O

import parity as PT

pytestmark = pytest.mark.gpu

NUM_CASES = 24
CALLS = 6


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _case(i: int):
    r = np.random.default_rng(15485863 * i + 11)
    return dict(rng=r, dtype=torch.bfloat16 if r.random() < 0.6 else torch.float32,
                d=int(r.choice([64, 128])), bs=int(r.choice([32, 64, 128])),
                hkv=int(r.integers(1, 5)), nseq=int(r.integers(1, 4)),
                nb=int(r.integers(3, 21)), spare=int(r.integers(0, 6)))


def _same_bits(a, b):
    view = {torch.float32: torch.int32, torch.bfloat16: torch.int16}[a.dtype]
    return torch.equal(a.view(view), b.view(view))


@pytest.mark.parametrize("i", range(NUM_CASES))
def test_append_and_rewrite_sequence_against_the_oracle(i):
    _gpu()
    c = _case(i)
    r, dt, D, bs, Hkv, B, NB = c["rng"], c["dtype"], c["d"], c["bs"], c["hkv"], c["nseq"], c["nb"]
    P = B * NB + c["spare"]
    PT.log(f"[append sweep {i}] {dt} D{D} bs{bs} Hkv{Hkv} B{B} NB{NB} P{P}")
    dev = torch.device("cuda")
    g = torch.Generator(device="cpu").manual_seed(1000 + i)
    perm = torch.randperm(P, generator=g)[: B * NB].to(torch.int32).reshape(B, NB)
    table = perm.to(dev)
    shape = L.make_shape(B, Hkv, Hkv, D, bs, NB, P, 1, dt)
    pool = PL.alloc_pool(shape, dev, fill_nan=True)
    cap = NB * bs
    k_log = torch.zeros((B, cap, Hkv, D), dtype=dt)
    v_log = torch.zeros((B, cap, Hkv, D), dtype=dt)
    lens = [0] * B
    to = lambda x: torch.tensor(x, dtype=torch.int32, device=dev)
    unmapped = sorted(set(range(P)) - set(perm.reshape(-1).tolist()))

    for call in range(CALLS):
        rewrite = call > 0 and r.random() < 0.5
        starts, ns, after = [], [], []
        for b in range(B):
            if rewrite:
                s = int(r.integers(0, lens[b] + 1))
            else:
                s = lens[b]
            n = int(r.integers(0, min(3 * bs, cap - s) + 1))
            starts.append(s)
            ns.append(n)
            after.append(max(lens[b], s + n))
        n_max = max(max(ns), 1)
        k_new = torch.randn((B, n_max, Hkv, D), generator=g).to(dt)
        v_new = torch.randn((B, n_max, Hkv, D), generator=g).to(dt)
        for b in range(B):
            k_log[b, starts[b]:starts[b] + ns[b]] = k_new[b, :ns[b]]
            v_log[b, starts[b]:starts[b] + ns[b]] = v_new[b, :ns[b]]
        PT.log(f"  call {call}: {'rewrite' if rewrite else 'append'} start {starts} n {ns} "
               f"-> {after}")
        PL.append(shape, pool, k_new.to(dev), v_new.to(dev), to(ns), to(starts), table,
                  ctx_after=to(after) if rewrite else None)
        torch.cuda.synchronize()
        lens = after

        kp, vp, reps = pool.k.cpu(), pool.v.cpu(), pool.reps.cpu()
        for b in range(B):
            n_tok = lens[b]
            if n_tok == 0:
                continue
            pos = torch.arange(n_tok)
            phys = perm[b, pos // bs].long()
            slot = pos % bs
            got_k = kp[phys, :, slot]          # [n_tok, Hkv, D]
            got_v = vp[phys, :, slot]
            assert _same_bits(got_k, k_log[b, :n_tok]), f"K of sequence {b}"
            assert _same_bits(got_v, v_log[b, :n_tok]), f"V of sequence {b}"
            nbv = O.num_blocks(n_tok, bs)
            kk = k_log[b, :n_tok].double().numpy()
            for h in range(Hkv):
                u = PT.UnitInputs(q=None, k_ctx=kk[:, h:h + 1], v_ctx=None, k_draft=None,
                                  v_draft=None, ctx=n_tok)
                want = O.block_representatives(kk[:, h:h + 1], bs)[:, 0]
                PT.check_reps(reps[perm[b, :nbv].long(), h].double().numpy(), u, bs, want)
        if unmapped:
            idle = torch.tensor(unmapped)
            assert torch.isnan(kp[idle].float()).all() and torch.isnan(vp[idle].float()).all()
            assert torch.isnan(reps[idle]).all()

    # representatives do not depend on how the tokens arrived
    bulk = PL.alloc_pool(shape, dev, fill_nan=True)
    n_max = max(max(lens), 1)
    PL.append(shape, bulk, k_log[:, :n_max].contiguous().to(dev),
              v_log[:, :n_max].contiguous().to(dev), to(lens), to([0] * B), table)
    torch.cuda.synchronize()
    for b in range(B):
        nbv = O.num_blocks(lens[b], bs)
        rows = perm[b, :nbv].long().to(dev)
        assert _same_bits(pool.reps[rows], bulk.reps[rows]), f"reps of sequence {b} vs bulk"
