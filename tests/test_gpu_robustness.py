"""GPU: device-side values out of range. The C ABI documents block tables, indices,
counts and positions held in device memory as unchecked preconditions, but every kernel
bounds the values it turns into addresses: an index outside [0, nb) or a table entry
outside [0, P) is an empty block, a count is clamped to [0, k_max], an append is cut at
the table's capacity and skips bad blocks. These tests pass such values through the entry
points and check that the result is exactly what those bounds imply: attention over the
valid selected blocks only (against the oracle), and appends that write only the valid
slots (every other pool byte unchanged)."""

import numpy as np
import pytest
import torch

from block_sparse_speculative_amd import _lib as L
from block_sparse_speculative_amd import pipeline as PL
from block_sparse_speculative_amd import synth
from block_sparse_speculative_amd.workload import Instance

import parity as PT

pytestmark = pytest.mark.gpu


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_attention_skips_out_of_range_indices_table_entries_and_counts():
    _gpu()
    w = synth.WORKLOADS["ragged"].with_(num_seqs=3, num_q_heads=8, num_kv_heads=2,
                                        ctx=(4096, 5000, 9000), ctx_range=None)
    inst = Instance(w, seed=21, num_layers=1)
    ly = inst.layers[0]
    s, km, bs, P = inst.shape, inst.k_max, w.block_size, inst.shape.num_phys_blocks
    PL.select(s, inst.budget, ly.q, ly.pool, inst.table, inst.ctx, km, ly.idx, ly.cnt, inst.ws)
    torch.cuda.synchronize()
    idx, cnt, table = ly.idx.cpu().clone(), ly.cnt.cpu().clone(), inst.table_host.clone()
    nbs = [synth.num_blocks(c, bs) for c in inst.ctx_lens]
    assert int(cnt[0, 0]) > 3 and int(cnt[0, 1]) > 5 and int(cnt[1, 0]) > 2 and int(cnt[1, 1]) > 4
    idx[0, 0, 3] = nbs[0] + 5                 # index past the sequence's blocks
    idx[0, 1, 5] = -9                         # negative index
    cnt[0, 1] = km + 50                       # count above k_max: the -1 padding is skipped
    table[1, int(idx[1, 0, 2])] = P + 100     # table entries outside the pool
    table[1, int(idx[1, 1, 4])] = -3
    cnt[2, 0] = -4                            # negative count: the drafts alone
    dev = torch.device("cuda")
    idx_d, cnt_d, table_d = idx.to(dev), cnt.to(dev), table.to(dev)
    B, T, Hq, D, G = w.num_seqs, w.num_draft, w.num_q_heads, w.head_dim, w.group
    out = torch.full((B, T, Hq, D), float("nan"), dtype=w.torch_dtype, device=dev)
    lse = torch.full((B, T, Hq), float("nan"), dtype=torch.float32, device=dev)
    n = L.attn_workspace_bytes(s, km)
    ws = torch.zeros(max(n, 1), dtype=torch.uint8, device=dev)
    L.sparse_verify_attn(s, ly.q, ly.k_draft, ly.v_draft, ly.pool.k, ly.pool.v, table_d,
                         inst.ctx, idx_d, cnt_d, km, inst.scale, out, lse=lse,
                         ws=ws if n else None)
    torch.cuda.synchronize()
    logical = inst.logical(0)
    out_h, lse_h = PT.np64(out), PT.np64(lse)
    for b in range(B):
        for g in range(w.num_kv_heads):
            c = min(max(int(cnt[b, g]), 0), km)
            sel = [int(j) for j in idx[b, g, :c].tolist()
                   if 0 <= j < nbs[b] and 0 <= int(table[b, j]) < P]
            u = PT.unit_inputs(logical, b, g, G)
            e = PT.check_output(out_h[b, :, g * G:(g + 1) * G], lse_h[b, :, g * G:(g + 1) * G],
                                u, np.array(sel, dtype=np.int64), bs, inst.scale, "bf16")
            PT.log(f"  unit ({b},{g}): {len(sel)} valid of {c} listed, {e}")


@pytest.mark.parametrize("bs", [64, 128])
def test_append_writes_only_valid_slots(bs):
    _gpu()
    dev = torch.device("cuda")
    B, Hkv, D, nmax = 4, 2, 128, 8
    NB = 6
    cap = NB * bs
    P = B * NB
    shape = L.make_shape(B, 8, Hkv, D, bs, NB, P, 8, torch.bfloat16)
    g = torch.Generator(device=dev).manual_seed(bs + 1)
    table = torch.arange(P, dtype=torch.int32).reshape(B, NB)
    start = [bs + 10, cap - 3, 2 * bs, -5]   # seq 1 runs past the capacity; seq 3 negative
    n_new = [6, 8, nmax + 5, 4]               # seq 2 asks for more than n_new_max
    table[0, start[0] // bs] = P + 7          # seq 0's target block: a bad table entry
    k = torch.randn((P, Hkv, bs, D), generator=g, device=dev).to(torch.bfloat16)
    v = torch.randn((P, Hkv, bs, D), generator=g, device=dev).to(torch.bfloat16)
    reps = torch.randn((P, Hkv, D), generator=g, device=dev)
    k0, v0, r0 = k.clone(), v.clone(), reps.clone()
    kn = torch.randn((B, nmax, Hkv, D), generator=g, device=dev).to(torch.bfloat16)
    vn = torch.randn((B, nmax, Hkv, D), generator=g, device=dev).to(torch.bfloat16)
    L.block_repr(shape, kn, vn, torch.tensor(n_new, dtype=torch.int32, device=dev),
                 torch.tensor(start, dtype=torch.int32, device=dev), table.to(dev), k, v, reps)
    torch.cuda.synchronize()
    # the slots the bounds allow: seq 1's last 3 positions, seq 2's first n_new_max tokens
    exp_k, exp_v = k0.clone(), v0.clone()
    valid = {}   # touched physical block -> its valid slots after the append
    for b, (c0, nn) in enumerate(zip(start, n_new)):
        if b in (0, 3):
            continue
        end = min(c0 + min(nn, nmax), cap)
        for pos in range(c0, end):
            p = int(table[b, pos // bs])
            exp_k[p, :, pos % bs] = kn[b, pos - c0]
            exp_v[p, :, pos % bs] = vn[b, pos - c0]
            valid[p] = min(end, (pos // bs + 1) * bs) - (pos // bs) * bs
    assert sorted(valid.values()) == sorted([bs, min(n_new[2], nmax)])
    assert torch.equal(k, exp_k) and torch.equal(v, exp_v)
    for p in range(P):
        if p not in valid:
            assert torch.equal(reps[p], r0[p]), f"representative of block {p} changed"
        else:   # the mean of the block's valid keys
            want = exp_k[p, :, :valid[p]].float().mean(dim=1)
            assert torch.allclose(reps[p], want, rtol=1e-5, atol=1e-6), f"block {p}"
