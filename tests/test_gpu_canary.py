"""GPU: canary-guarded outputs. Every buffer an entry point writes (outputs, workspace,
the K/V pool and representatives of an append) is a slice of a larger device buffer
whose guard zones before and after hold a byte pattern; after the call (twice, with a
synchronisation between) the guards must be unchanged, so a kernel that writes past
either end of a buffer it was given fails here. An append must also leave every pool
slot it does not own bit-identical.
"""

import pytest
import torch

from block_sparse_speculative_amd import _lib as L
from block_sparse_speculative_amd import pipeline as PL
from block_sparse_speculative_amd import synth
from block_sparse_speculative_amd.workload import Instance

import parity as PT

pytestmark = pytest.mark.gpu

GUARD = 64 * 1024          # bytes of guard on each side
CANARY = 0xA5


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


class Guarded:
    """A device tensor of the given shape and dtype inside guard zones."""

    def __init__(self, shape, dtype, fill=None):
        n = 1
        for s in shape:
            n *= s
        nbytes = n * torch.empty((), dtype=dtype).element_size()
        self.nbytes = nbytes
        self.buf = torch.full((GUARD + nbytes + GUARD,), CANARY, dtype=torch.uint8, device="cuda")
        self.t = self.buf[GUARD:GUARD + nbytes].view(dtype).view(*shape)
        if fill is not None:
            self.t.copy_(fill) if isinstance(fill, torch.Tensor) else self.t.fill_(fill)

    def check(self, name):
        torch.cuda.synchronize()
        lo = self.buf[:GUARD]
        hi = self.buf[GUARD + self.nbytes:]
        bad_lo = int((lo != CANARY).sum())
        bad_hi = int((hi != CANARY).sum())
        assert bad_lo == 0 and bad_hi == 0, (
            f"{name}: {bad_lo} guard bytes overwritten before the buffer, {bad_hi} after")


def _layer_inputs(w, seed=11):
    inst = Instance(w, seed=seed, num_layers=1)
    return inst, inst.layers[0]


CASES = {
    "llama_small": synth.WORKLOADS["llama32k"].with_(num_seqs=2, num_q_heads=8, num_kv_heads=2,
                                                     ctx=(8192, 6000)),
    "ragged_tail": synth.WORKLOADS["llama32k"].with_(num_seqs=3, num_q_heads=8, num_kv_heads=2,
                                                     ctx=(4097, 5001, 130)),
    "fp32_rows128": synth.WORKLOADS["tiny"].with_(num_q_heads=16, num_kv_heads=2, num_draft=16,
                                                  head_dim=128, block_size=64, ctx=(3000,),
                                                  budget=(0, 12, 0, 1, 1)),
}


@pytest.mark.parametrize("name", list(CASES))
def test_select_and_attend_writes_stay_inside_their_buffers(name):
    _gpu()
    inst, ly = _layer_inputs(CASES[name])
    s, B, Hkv, T, Hq, D = (inst.shape, inst.w.num_seqs, inst.w.num_kv_heads, inst.w.num_draft,
                           inst.w.num_q_heads, inst.w.head_dim)
    km = inst.k_max
    idx = Guarded((B, Hkv, km), torch.int32, -7)
    cnt = Guarded((B, Hkv), torch.int32, -7)
    out = Guarded((B, T, Hq, D), inst.w.torch_dtype, 0)
    lse = Guarded((B, T, Hq), torch.float32, 0)
    ws = Guarded((L.select_and_attend_workspace_bytes(s, km),), torch.uint8, 0)
    for _ in range(2):
        L.select_and_attend(s, inst.budget, ly.q, ly.pool.reps, ly.k_draft, ly.v_draft, ly.pool.k,
                            ly.pool.v, inst.table, inst.ctx, km, inst.scale, idx.t, cnt.t, out.t,
                            lse=lse.t, ws=ws.t, draft_mask=inst.draft_mask)
        for g, nm in ((idx, "idx"), (cnt, "cnt"), (out, "out"), (lse, "lse"), (ws, "ws")):
            g.check(f"{name} fused {nm}")
    assert torch.isfinite(out.t.float()).all() and torch.isfinite(lse.t).all()
    # the separate calls, each with its own guarded workspace
    idx2 = Guarded((B, Hkv, km), torch.int32, -7)
    cnt2 = Guarded((B, Hkv), torch.int32, -7)
    scores = Guarded((B, Hkv, s.max_blocks_per_seq), torch.float32, 0)
    wsel = Guarded((L.select_workspace_bytes(s, km),), torch.uint8, 0)
    na = L.attn_workspace_bytes(s, km)
    wat = Guarded((max(na, 1),), torch.uint8, 0)
    out2 = Guarded((B, T, Hq, D), inst.w.torch_dtype, 0)
    lse2 = Guarded((B, T, Hq), torch.float32, 0)
    for _ in range(2):
        L.select_blocks(s, inst.budget, ly.q, ly.pool.reps, inst.table, inst.ctx, km, idx2.t,
                        cnt2.t, scores=scores.t, ws=wsel.t)
        L.sparse_verify_attn(s, ly.q, ly.k_draft, ly.v_draft, ly.pool.k, ly.pool.v, inst.table,
                             inst.ctx, idx2.t, cnt2.t, km, inst.scale, out2.t, lse=lse2.t,
                             ws=wat.t if na else None, draft_mask=inst.draft_mask)
        for g, nm in ((idx2, "idx"), (cnt2, "cnt"), (scores, "scores"), (wsel, "select ws"),
                      (wat, "attn ws"), (out2, "out"), (lse2, "lse")):
            g.check(f"{name} separate {nm}")
    # both paths agree (same selection, same kernels' arithmetic up to the split merge)
    assert torch.equal(cnt.t, cnt2.t)
    PT.log(f"  canary {name}: guards intact on {B * Hkv} units")


def test_static_entry_point_and_reuse_stay_inside_their_buffers():
    _gpu()
    inst, ly = _layer_inputs(CASES["llama_small"])
    s, B, Hkv, T, Hq, D = (inst.shape, inst.w.num_seqs, inst.w.num_kv_heads, inst.w.num_draft,
                           inst.w.num_q_heads, inst.w.head_dim)
    km = inst.k_max
    idx = Guarded((B, Hkv, km), torch.int32, -7)
    cnt = Guarded((B, Hkv), torch.int32, -7)
    out = Guarded((B, T, Hq, D), inst.w.torch_dtype, 0)
    lse = Guarded((B, T, Hq), torch.float32, 0)
    L.select_and_attend_static(s, inst.budget, ly.q, ly.pool.reps, ly.k_draft, ly.v_draft,
                               ly.pool.k, ly.pool.v, inst.table, inst.ctx, km, inst.scale, idx.t,
                               cnt.t, out.t, lse=lse.t)
    for g, nm in ((idx, "idx"), (cnt, "cnt"), (out, "out"), (lse, "lse")):
        g.check(f"static {nm}")
    idx2 = Guarded((B, Hkv, km), torch.int32, -7)
    cnt2 = Guarded((B, Hkv), torch.int32, -7)
    L.reuse_indices(s, km, idx.t, cnt.t, idx2.t, cnt2.t)
    idx2.check("reuse idx")
    cnt2.check("reuse cnt")
    assert torch.equal(idx.t, idx2.t) and torch.equal(cnt.t, cnt2.t)


@pytest.mark.parametrize("bs", [32, 64, 128])
def test_append_writes_only_its_slots(bs):
    _gpu()
    dev = torch.device("cuda")
    B, Hkv, D, T = 3, 2, 128, 8
    start = [100, bs * 5 - 3, 0]        # a partial tail, a block-crossing append, an empty seq
    cap = max(start) + 3 * bs
    NB = -(-cap // bs)
    P = B * NB + 2                        # two physical blocks no sequence maps
    shape = L.make_shape(B, 8, Hkv, D, bs, NB, P, T, torch.bfloat16)
    g = torch.Generator(device=dev).manual_seed(bs)
    table = torch.randperm(B * NB, generator=torch.Generator().manual_seed(bs)).to(torch.int32)
    table = table.reshape(B, NB).to(dev)
    k = Guarded((P, Hkv, bs, D), torch.bfloat16,
                torch.randn((P, Hkv, bs, D), generator=g, device=dev).to(torch.bfloat16))
    v = Guarded((P, Hkv, bs, D), torch.bfloat16,
                torch.randn((P, Hkv, bs, D), generator=g, device=dev).to(torch.bfloat16))
    reps = Guarded((P, Hkv, D), torch.float32,
                   torch.randn((P, Hkv, D), generator=g, device=dev))
    k0, v0, r0 = k.t.clone(), v.t.clone(), reps.t.clone()
    n = [T, bs + 5, 0]                    # the last sequence appends nothing
    nmax = max(n)
    kn = torch.randn((B, nmax, Hkv, D), generator=g, device=dev).to(torch.bfloat16)
    vn = torch.randn((B, nmax, Hkv, D), generator=g, device=dev).to(torch.bfloat16)
    L.block_repr(shape, kn, vn, torch.tensor(n, dtype=torch.int32, device=dev),
                 torch.tensor(start, dtype=torch.int32, device=dev), table, k.t, v.t, reps.t)
    for gd, nm in ((k, "k_pool"), (v, "v_pool"), (reps, "repr_pool")):
        gd.check(f"append bs{bs} {nm}")
    # slots written: token positions start .. start + n - 1 of each sequence; reps: the
    # blocks those tokens land in
    tab = table.cpu()
    own = torch.zeros((P, bs), dtype=torch.bool)
    blk = torch.zeros(P, dtype=torch.bool)
    for b in range(B):
        for pos in range(start[b], start[b] + n[b]):
            p = int(tab[b, pos // bs])
            own[p, pos % bs] = True
            blk[p] = True
    own_d = own.to(dev)[:, None, :, None].expand(P, Hkv, bs, D)
    assert torch.equal(k.t[~own_d], k0[~own_d]) and torch.equal(v.t[~own_d], v0[~own_d])
    blk_d = blk.to(dev)
    assert torch.equal(reps.t[~blk_d], r0[~blk_d])
    # the written slots hold the new tokens
    for b in range(B):
        for j in range(n[b]):
            pos = start[b] + j
            p = int(tab[b, pos // bs])
            assert torch.equal(k.t[p, :, pos % bs], kn[b, j]) and torch.equal(v.t[p, :, pos % bs],
                                                                              vn[b, j])


def test_sparse_ffn_writes_stay_inside_their_buffers():
    _gpu()
    w = synth.FFN_WORKLOADS["ffn_llama8b"].__class__("canary", 5, 1024, 1000, 0.9, 0.3)
    inp = synth.make_ffn(w, 3, torch.device("cuda"))
    shape = L.make_ffn_shape(w.num_tokens, w.d_model, w.d_ffn)
    y = Guarded((w.num_tokens, w.d_model), torch.bfloat16, 0)
    keep = Guarded((w.d_ffn,), torch.int32, -1)
    ws = Guarded((L.sparse_ffn_workspace_bytes(shape),), torch.uint8, 0)
    for _ in range(2):
        L.sparse_ffn(shape, inp["x"], inp["w_gate"], inp["w_up"], inp["w_down_t"], w.tau, y.t,
                     keep_bits=keep.t, ws=ws.t)
        for g, nm in ((y, "y"), (keep, "keep_bits"), (ws, "ws")):
            g.check(f"ffn {nm}")
    assert torch.isfinite(y.t.float()).all()
    assert int((keep.t.cpu().to(torch.int64) & 0xFFFFFFFF).max()) < (1 << w.num_tokens)
