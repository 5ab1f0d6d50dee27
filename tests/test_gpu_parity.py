"""GPU parity: the HIP path, called through the C ABI, against the fp64 oracle.

Small workloads are checked on every (sequence, KV head) unit; the full-size
workloads are checked on sampled units, in the launch configuration the bench times
(library-chosen split count). Selected indices must be exact except inside the
near-tie band; outputs must meet the fp32 / bf16 tolerances (tests/parity.py).
"""

import gc

import numpy as np
import pytest
import torch

from block_sparse_speculative_amd import synth
from block_sparse_speculative_amd.workload import Instance

import cases as C
import parity as PT

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
SMALL, EDGE, TREES = C.SMALL, C.EDGE, C.TREES


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _free():
    gc.collect()
    torch.cuda.empty_cache()


def _all_units(inst):
    return [(b, g) for b in range(inst.w.num_seqs) for g in range(inst.w.num_kv_heads)]


def run_and_check(inst, units=None, layers=None, check_reps=True, scores=False, case=None):
    """Run one pass of `inst` and check the listed units of the listed layers; the
    observed errors are recorded under `case` (default: the workload's name)."""
    n = len(inst.layers)
    layers = list(range(n)) if layers is None else layers
    units = _all_units(inst) if units is None else units
    gscores = None
    for l in range(n):
        if inst.fused:
            inst.run_layer(l)
        elif scores and not inst.layers[l].reuse:
            gscores = torch.full((inst.w.num_seqs, inst.w.num_kv_heads, inst.shape.max_blocks_per_seq),
                                 float("nan"), dtype=torch.float32, device=inst.device)
            inst.select_or_reuse(l, scores=gscores)
        else:
            inst.select_or_reuse(l)
        if not inst.fused:
            inst.attend(l)
    torch.cuda.synchronize()
    prev, stats_all = None, []
    for l in layers:
        ly = inst.layers[l]
        p = prev if ly.reuse else None
        if ly.reuse and prev is None:
            # the selecting layer before a reuse layer must be checked first
            p, _ = PT.verify_instance_units(inst, l - 1, units, check_reps_too=False)
        sels, st = PT.verify_instance_units(inst, l, units, prev_sel=p,
                                            check_reps_too=check_reps and not ly.reuse,
                                            gpu_scores=gscores if (scores and not ly.reuse) else None)
        PT.log(f"  layer {l} ({'reuse' if ly.reuse else 'select'}): {st}")
        PT.record(f"{case or inst.w.name} L{l}", **st)
        prev = sels
        stats_all.append(st)
    return stats_all


# ------------------------------------------------------------------ small workloads
@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("splits", [0, 1, 2, 1000])
def test_small_workload_all_units(name, splits):
    _gpu()
    PT.log(f"[small] {name} splits={splits}")
    inst = Instance(SMALL[name], seed=11, num_splits=splits, nan_pool=True)
    PT.log(f"  resolved splits={inst.num_splits} k_max={inst.k_max}")
    run_and_check(inst, scores=(splits == 0), case=f"small {name} s{splits}")
    del inst
    _free()


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_small_workload_fused_select_and_attend(name, splits):
    # sv_select_and_attend: oracle parity, and bit-identical to the separate calls
    _gpu()
    PT.log(f"[fused] {name} splits={splits}")
    w = SMALL[name].with_(num_layers=2, reuse_odd_layers=True)
    a = Instance(w, seed=12, num_splits=splits, nan_pool=True, fused=True)
    run_and_check(a, case=f"fused {name} s{splits}")
    b = Instance(w, seed=12, num_splits=splits, nan_pool=True, fused=False)
    b.step()
    torch.cuda.synchronize()
    for la, lb in zip(a.layers, b.layers):
        assert torch.equal(la.idx, lb.idx) and torch.equal(la.cnt, lb.cnt)
        assert torch.equal(la.out, lb.out) and torch.equal(la.lse, lb.lse)
    del a, b
    _free()


@pytest.mark.parametrize("case", C.matrix_cases(), ids=lambda c: c[0])
def test_build_matrix_all_units(case):
    # every attention build the library can launch (tests/cases.py), checked on every
    # unit against the oracle; the launch plan must be the build the case stands for
    _gpu()
    cid, w, splits, fused = case
    PT.log(f"[matrix] {cid}")
    inst = Instance(w, seed=41, num_splits=splits, nan_pool=True, fused=fused)
    plan = inst.plan
    PT.log(f"  plan {plan}")
    key = C.build_key(w, splits, fused)
    assert (plan["tile_tokens"], plan["padded_rows"], plan["ring_kb"]) == key[2:5]
    run_and_check(inst, case=cid)
    del inst
    _free()


def test_tiny_planted_blocks_selected():
    _gpu()
    inst = Instance(W["tiny"], seed=0)
    inst.step()
    torch.cuda.synchronize()
    heavy = synth.planted_sets(inst.w, inst.ctx_lens, 0, 0)
    idx, cnt = inst.layers[0].idx.cpu(), inst.layers[0].cnt.cpu()
    for g in range(inst.w.num_kv_heads):
        sel = PT.gpu_unit_selection(idx, cnt, 0, g)
        assert len(sel) == 16 and set(heavy[0][g]) <= set(sel)


# ------------------------------------------------------------------ edge cases

EDGE = W["llama32k"].with_(num_seqs=4, num_q_heads=8, num_kv_heads=2, ctx=(0, 17, 200, 1000),
                           budget=(0, 2, 0, 1, 1))


@pytest.mark.parametrize("splits", [0, 1, 3])
def test_edge_contexts_empty_partial_forced_only(splits):
    # ctx 0 (drafts only), one partial block, and sparse selections of forced blocks only
    _gpu()
    PT.log(f"[edge] contexts {EDGE.ctx} splits={splits}")
    inst = Instance(EDGE, seed=3, num_splits=splits, nan_pool=True)
    run_and_check(inst, case=f"edge ctx 0/17/200/1000 s{splits}")


def test_single_query_single_head_decode():
    # T = 1, G = 1: plain single-query decode
    _gpu()
    w = W["llama32k"].with_(num_seqs=2, num_q_heads=4, num_kv_heads=4, num_draft=1,
                            ctx=(3000, 9000), budget=(4096, 64, 50, 1, 1))
    inst = Instance(w, seed=5, nan_pool=True)
    run_and_check(inst, case="T=1 G=1 decode")


@pytest.mark.parametrize("flags", [(0, 0), (1, 0), (0, 1)])
def test_forced_block_flags(flags):
    _gpu()
    w = W["llama32k"].with_(num_seqs=1, num_q_heads=8, num_kv_heads=2, ctx=(6000,),
                            budget=(0, 5, 0) + flags)
    run_and_check(Instance(w, seed=9, nan_pool=True), case=f"forced flags {flags}")


def test_k_max_larger_than_budget_pads_with_minus_one():
    _gpu()
    w = W["llama32k"].with_(num_seqs=2, num_q_heads=8, num_kv_heads=2, ctx=(5000, 300),
                            budget=(0, 16, 0, 1, 1))
    inst = Instance(w, seed=2, k_max=40, nan_pool=True)
    run_and_check(inst, case="k_max 40 > budget")
    cnt = inst.layers[0].cnt.cpu()
    assert cnt[0].tolist() == [16, 16] and cnt[1].tolist() == [5, 5]


# k_max below the budget caps it: min(k, k_max) blocks, the forced ones and the best
# others by score, also for sequences whose budget keeps every block (their scores
# must then be computed). The oracle selects with the capped budget.
CAPS = {
    "sparse_budget": (SMALL["llama_small"], 20),
    "dense_budget": (SMALL["llama_small"].with_(budget=(16384, 64, 50, 1, 1)), 40),
    "forced_only": (SMALL["llama_small"], 2),
    "first_only": (SMALL["llama_small"].with_(budget=(0, 8, 0, 1, 0)), 1),
    "ragged_mixed": (SMALL["ragged_small"], 50),            # one dense, two sparse budgets
    "long_table": (SMALL["long_table"], 30),                # > 1024 blocks: LDS radix top-k
    "long_table_dense_budget": (SMALL["long_table"].with_(budget=(65536, 64, 50, 1, 1)), 200),
}


@pytest.mark.parametrize("name", list(CAPS))
def test_k_max_below_the_budget_caps_the_selection(name):
    _gpu()
    w, k_max = CAPS[name]
    PT.log(f"[cap] {name} k_max={k_max}")
    runs = []
    for fused in (False, True):
        inst = Instance(w, seed=23, k_max=k_max, cap_selection=True, nan_pool=True,
                        fused=fused)
        assert inst.k_max == k_max
        run_and_check(inst, case=f"cap {name} {'fused' if fused else 'separate'}")
        assert int(inst.layers[0].cnt.max()) <= k_max
        runs.append(inst)
    a, b = runs
    for la, lb in zip(a.layers, b.layers):
        assert torch.equal(la.idx, lb.idx) and torch.equal(la.cnt, lb.cnt)
        assert torch.equal(la.out, lb.out) and torch.equal(la.lse, lb.lse)
    del a, b, runs
    _free()


# ------------------------------------------------------------------ draft trees

TREES = {
    "llama_small": SMALL["llama_small"],
    "qwen_small": SMALL["qwen_small"],                  # T = 16: all 16 mask bits in use
    "fp32_rows32_bs128": SMALL["fp32_rows32_bs128"],
    "fp32_rows128_d128": SMALL["fp32_rows128_d128"],    # fp32, T = 16
    "edge": EDGE,                                       # ctx 0: the drafts alone
    "long_table": SMALL["long_table"],                  # > 1024 blocks: separate top-k
}


@pytest.mark.parametrize("tree", ["random", "star"])
@pytest.mark.parametrize("name", list(TREES))
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_draft_tree_all_units(name, tree, splits):
    # tree attention among the drafts: oracle parity on every unit, and the fused and
    # separate entry points bit-identical
    _gpu()
    PT.log(f"[tree] {name} {tree} splits={splits}")
    w = TREES[name].with_(draft_tree=tree, num_layers=2, reuse_odd_layers=True)
    a = Instance(w, seed=31, num_splits=splits, nan_pool=True, fused=True)
    assert a.draft_mask is not None
    run_and_check(a, case=f"tree {name} {tree} s{splits}")
    b = Instance(w, seed=31, num_splits=splits, nan_pool=True, fused=False)
    b.step()
    torch.cuda.synchronize()
    for la, lb in zip(a.layers, b.layers):
        assert torch.equal(la.out, lb.out) and torch.equal(la.lse, lb.lse)
    del a, b
    _free()


def test_chain_mask_self_bit_and_high_bits():
    # the chain's bits give exactly the mask-free result; a draft always sees itself;
    # bits at or above T are ignored
    _gpu()
    w = SMALL["llama_small"]
    T, B = w.num_draft, w.num_seqs
    ref = _outputs(Instance(w, seed=32))
    chain = [[t - 1 for t in range(T)]] * B
    full = synth.draft_mask(chain, T)
    variants = [full, full & ~torch.tensor([1 << t for t in range(T)], dtype=torch.int32),
                full | (1 << T) | (1 << 30)]
    for m in variants:
        inst = Instance(w, seed=32)
        inst.draft_mask = m.to(inst.device)
        for x, y in zip(_outputs(inst), ref):
            assert torch.equal(x, y)


def test_full_stack64k_tree_sampled_units():
    # the bench shape with a random draft tree, in the library's launch configuration
    _gpu()
    PT.log("[full] stack64k random tree")
    w = W["stack64k"].with_(num_layers=2, draft_tree="random")
    inst = Instance(w, seed=33, fused=True)
    run_and_check(inst, units=[(0, 0), (1, 3), (2, 6), (3, 7)], case="stack64k random tree")
    del inst
    _free()


# ------------------------------------------------------------------ full verification and
# the decode-loop append

def test_full_verification_dense_at_64k_sampled_units():
    # Periodic full verification runs through the same entry points with a budget that
    # keeps every block: 1024 blocks per unit at the stack64k shape, then a reuse layer.
    _gpu()
    PT.log("[full] stack64k dense verification")
    w = W["stack64k"].with_(num_layers=2, budget=(1 << 30, 64, 50, 1, 1))
    inst = Instance(w, seed=34, fused=True)
    assert inst.k_max == 1024
    run_and_check(inst, units=[(0, 0), (3, 7)], check_reps=False, case="stack64k dense budget")
    cnt = inst.layers[1].cnt.cpu()
    assert (cnt == 1024).all()
    del inst
    _free()


def test_decode_loop_append_matches_bulk_bit_identical():
    # Accepted tokens (1..T per sequence and step, different per sequence) appended
    # after each verification pass leave the pool and the representatives exactly as a
    # bulk append of the final contexts would.
    _gpu()
    from block_sparse_speculative_amd import pipeline as PL
    w = SMALL["ragged_small"]
    final = Instance(w, seed=35, num_layers=1)
    lens = final.ctx_lens
    x = final.logical(0)
    shape, table = final.shape, final.table
    B, T = w.num_seqs, w.num_draft
    pool = PL.alloc_pool(shape, final.device, fill_nan=True)
    start = [max(0, c - 300) for c in lens]
    PL.append(shape, pool, x["k_ctx"][:, :max(start)].contiguous(),
              x["v_ctx"][:, :max(start)].contiguous(),
              torch.tensor(start, dtype=torch.int32, device=final.device),
              torch.zeros(B, dtype=torch.int32, device=final.device), table)
    cur = list(start)
    g = torch.Generator().manual_seed(36)
    while any(c < l for c, l in zip(cur, lens)):
        acc = [min(int(torch.randint(1, T + 1, (1,), generator=g)), l - c) for c, l in zip(cur, lens)]
        n_max = max(max(acc), 1)
        kn = torch.zeros((B, n_max) + tuple(x["k_ctx"].shape[2:]), dtype=x["k_ctx"].dtype,
                         device=final.device)
        vn = torch.zeros_like(kn)
        for b in range(B):
            kn[b, :acc[b]] = x["k_ctx"][b, cur[b]:cur[b] + acc[b]]
            vn[b, :acc[b]] = x["v_ctx"][b, cur[b]:cur[b] + acc[b]]
        PL.append(shape, pool, kn, vn, torch.tensor(acc, dtype=torch.int32, device=final.device),
                  torch.tensor(cur, dtype=torch.int32, device=final.device), table)
        cur = [c + a for c, a in zip(cur, acc)]
    torch.cuda.synchronize()
    ref = final.layers[0].pool
    for b, c in enumerate(lens):
        nb = -(-c // w.block_size)
        phys = final.table_host[b, :nb].to(final.device).long()
        assert torch.equal(pool.reps[phys], ref.reps[phys])
        full = c // w.block_size
        assert torch.equal(pool.k[phys[:full]], ref.k[phys[:full]])
        assert torch.equal(pool.v[phys[:full]], ref.v[phys[:full]])
        tail = c - full * w.block_size
        if tail:
            last = phys[full]
            assert torch.equal(pool.k[last][:, :tail], ref.k[last][:, :tail])
            assert torch.equal(pool.v[last][:, :tail], ref.v[last][:, :tail])


# ------------------------------------------------------------------ invariances

def _outputs(inst):
    inst.step()
    torch.cuda.synchronize()
    ly = inst.layers[0]
    return ly.idx.cpu().clone(), ly.out.float().cpu().clone(), ly.lse.cpu().clone()


def test_run_to_run_bit_identical():
    _gpu()
    inst = Instance(SMALL["llama_small"], seed=21)
    a = _outputs(inst)
    b = _outputs(inst)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_merge_tags_on_a_shared_workspace():
    # The in-launch merge recognises a unit's workgroups by tags carrying the unit's
    # launch epoch. Launches with different split counts on one workspace (tags of other
    # split counts left in the slots), and a zero-fill of the whole workspace between
    # calls, must give exactly what the same call gives on a fresh workspace.
    _gpu()
    from block_sparse_speculative_amd import _lib as L
    inst = Instance(SMALL["llama_small"], seed=31)
    inst.step()
    torch.cuda.synchronize()
    ly = inst.layers[0]
    seq = [3, 7, 3, 11, 2, 7, 0, 3]
    nbytes = max(L.attn_workspace_bytes(inst.shape, inst.k_max, s) for s in seq)
    shared = torch.zeros(nbytes, dtype=torch.uint8, device=inst.device)

    def call(splits, ws):
        out, lse = torch.empty_like(ly.out), torch.empty_like(ly.lse)
        L.sparse_verify_attn(inst.shape, ly.q, ly.k_draft, ly.v_draft, ly.pool.k, ly.pool.v,
                             inst.table, inst.ctx, ly.idx, ly.cnt, inst.k_max, inst.scale, out,
                             lse=lse, ws=ws, num_splits=splits)
        return out, lse

    for i, splits in enumerate(seq):
        if i == 5:
            shared.zero_()
        a = call(splits, shared)
        fresh = torch.zeros(max(L.attn_workspace_bytes(inst.shape, inst.k_max, splits), 1),
                            dtype=torch.uint8, device=inst.device)
        b = call(splits, fresh)
        torch.cuda.synchronize()
        assert torch.isfinite(a[0].float()).all(), f"splits {splits}"
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]), f"splits {splits}"


def _copy_to_high_word(t: torch.Tensor) -> torch.Tensor:
    """A copy of t in device memory whose address has bit 31 set in its low 32 bits."""
    nbytes = t.numel() * t.element_size()
    buf = torch.empty(nbytes + 2 ** 31 + 512, dtype=torch.uint8, device=t.device)
    base = buf.data_ptr()
    off = 0 if (base & 0xFFFFFFFF) >= 0x80000000 else 0x80000000 - (base & 0xFFFFFFFF)
    off = (off + 255) // 256 * 256
    view = buf[off:off + nbytes].view(t.dtype).view(t.shape)
    view.copy_(t)
    assert (view.data_ptr() & 0xFFFFFFFF) >= 0x80000000
    return view


@pytest.mark.parametrize("name", ["llama_small", "tiny", "qwen_small"])
def test_buffers_whose_address_low_word_has_bit31_set(name):
    # Regression: the attention kernel forms its DMA base from two 32-bit halves; a low
    # half with bit 31 set must not spill into the high half. Pools, draft K/V and
    # queries at such addresses give exactly the results of ordinary allocations.
    _gpu()
    from block_sparse_speculative_amd import pipeline as PL
    inst = Instance(SMALL[name], seed=29)
    ref = _outputs(inst)
    for ly in inst.layers:
        ly.pool = PL.Pool(_copy_to_high_word(ly.pool.k), _copy_to_high_word(ly.pool.v),
                          _copy_to_high_word(ly.pool.reps))
        ly.k_draft = _copy_to_high_word(ly.k_draft)
        ly.v_draft = _copy_to_high_word(ly.v_draft)
        ly.q = _copy_to_high_word(ly.q)
    got = _outputs(inst)
    for x, y in zip(got, ref):
        assert torch.equal(x, y)
    del inst
    _free()


def test_paged_and_contiguous_tables_bit_identical():
    _gpu()
    w = SMALL["ragged_small"]
    a = _outputs(Instance(w, seed=4, paged=True))
    b = _outputs(Instance(w, seed=4, paged=False))
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_incremental_append_matches_bulk_bit_identical():
    # tokens appended in odd-sized chunks give the same pool and representatives
    _gpu()
    w = SMALL["llama_small"]
    bulk = Instance(w, seed=8)
    inc = Instance(w, seed=8, append_chunk=37)
    table = bulk.table_host
    for b, c in enumerate(bulk.ctx_lens):
        nb = -(-c // w.block_size)
        phys = table[b, :nb].to(bulk.device).long()
        pa, pb = bulk.layers[0].pool, inc.layers[0].pool
        assert torch.equal(pa.reps[phys], pb.reps[phys])
        full = c // w.block_size
        if full:
            assert torch.equal(pa.k[phys[:full]], pb.k[phys[:full]])
            assert torch.equal(pa.v[phys[:full]], pb.v[phys[:full]])


def test_split_counts_agree_within_tolerance():
    _gpu()
    w = SMALL["qwen_small"]
    outs = []
    for s in (1, 2, 7, 1000):
        _, o, _ = _outputs(Instance(w, seed=6, num_splits=s))
        outs.append(o)
    for o in outs[1:]:
        assert (o - outs[0]).abs().max().item() <= 1e-2


def test_last_arriver_merge_when_the_grid_exceeds_the_device():
    # 64 units x 17 workgroups > 512 resident workgroups: the last workgroup of each unit
    # to arrive merges the whole unit inside the launch
    _gpu()
    from block_sparse_speculative_amd import _lib as L
    w = W["llama32k"].with_(num_seqs=8, ctx=(8192,) * 8)
    inst = Instance(w, seed=23, num_splits=16, fused=True)
    assert inst.plan["workgroups"] == 17 * 64 > 512
    assert inst.plan["merge_mode"] == L.MERGE_IN_LAUNCH_LAST
    run_and_check(inst, units=[(0, 0), (3, 5), (7, 7), (5, 2)], case="merge last-arriver")


def test_merge_kernel_when_a_unit_has_more_than_32_workgroups():
    _gpu()
    from block_sparse_speculative_amd import _lib as L
    w = W["llama32k"].with_(num_seqs=1, num_q_heads=8, num_kv_heads=2, ctx=(8192,))
    inst = Instance(w, seed=25, num_splits=40, fused=True)
    assert inst.plan["merge_mode"] == L.MERGE_KERNEL
    run_and_check(inst, case="merge kernel")


def test_in_kernel_merge_at_full_residency():
    # 32 units x 16 workgroups = 512 workgroups, two per CU: every one resident
    _gpu()
    from block_sparse_speculative_amd import _lib as L
    w = W["stack64k"].with_(num_layers=2, ctx=(8192,) * 4)
    inst = Instance(w, seed=24, num_splits=15, fused=True)
    assert inst.plan["workgroups"] == 512 and inst.plan["ring_kb"] == 64
    assert inst.plan["merge_mode"] == L.MERGE_IN_LAUNCH_WAIT
    run_and_check(inst, units=[(0, 0), (1, 3), (3, 7)], case="merge wait, full residency")


def test_merge_with_other_kernels_holding_the_device():
    # The in-launch merge must not depend on the whole grid being resident: here long
    # independent matrix products run on a second stream (same priority) while the
    # attention runs, so some of a unit's workgroups may start only after others have
    # finished their stream. Each workgroup waits for its siblings at most a bounded
    # time, then hands its slice to the last one to arrive. Outputs must match the
    # oracle exactly as on an idle device, with no NaN.
    _gpu()
    from block_sparse_speculative_amd import _lib as L
    w = W["stack64k"].with_(num_layers=2, ctx=(8192,) * 4)
    inst = Instance(w, seed=26, fused=True)
    assert inst.plan["merge_mode"] == L.MERGE_IN_LAUNCH_WAIT
    inst.step()
    torch.cuda.synchronize()
    idle = [(ly.out.clone(), ly.lse.clone()) for ly in inst.layers]
    a = torch.randn(8192, 8192, device=inst.device, dtype=torch.bfloat16)
    bm = torch.randn(8192, 8192, device=inst.device, dtype=torch.bfloat16)
    side = torch.cuda.Stream()
    for rep in range(3):
        for ly in inst.layers:
            ly.out.fill_(float("nan"))
            ly.lse.fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            for _ in range(6):
                a = (a @ bm) * (1.0 / 128.0)
        inst.step()                     # on the current stream, concurrently
        torch.cuda.synchronize()
        for ly, (o, l_) in zip(inst.layers, idle):
            assert torch.isfinite(ly.out.float()).all() and torch.isfinite(ly.lse).all()
            assert torch.equal(ly.out, o) and torch.equal(ly.lse, l_), f"replay {rep}"
    run_and_check(inst, units=[(0, 0), (1, 3), (2, 5), (3, 7)], case="merge under load")


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("splits", [0, 1])
def test_largest_block_table_and_row_count(fused, splits):
    # The envelope's limits together: 16384 blocks per sequence (512K tokens in 32-token
    # blocks: the LDS radix top-k, the unstaged table, and with the library's split count
    # the merge kernel) and 128 rows per unit (16 drafts x a GQA group of 8).
    _gpu()
    w = W["llama32k"].with_(num_seqs=1, num_q_heads=8, num_kv_heads=1, head_dim=64,
                            block_size=32, num_draft=16, ctx=(16384 * 32,),
                            budget=(0, 64, 30, 1, 1))
    PT.log(f"[largest] fused={fused} splits={splits}")
    inst = Instance(w, seed=51, num_splits=splits, fused=fused, nan_pool=True)
    assert inst.shape.max_blocks_per_seq == 16384 and inst.k_max == 492
    PT.log(f"  plan {inst.plan}")
    run_and_check(inst, case=f"16384 blocks, 128 rows, {'fused' if fused else 'separate'} "
                             f"s{splits}")
    del inst
    _free()


def test_independent_passes_on_concurrent_streams():
    # Two instances with their own buffers and workspaces run their passes at the same
    # time on two streams (same priority): the library keeps no state between calls
    # beyond the caller's buffers, so each result is bit-identical to its pass run alone.
    _gpu()
    a = Instance(W["stack64k"].with_(num_layers=2, ctx=(8192,) * 4), seed=41, fused=True)
    b = Instance(SMALL["ragged_small"].with_(num_layers=2, reuse_odd_layers=True), seed=42)
    alone = []
    for x in (a, b):
        x.step()
        torch.cuda.synchronize()
        alone.append([(ly.out.clone(), ly.lse.clone(), ly.idx.clone(), ly.cnt.clone())
                      for ly in x.layers])
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(3):
        for x in (a, b):
            for ly in x.layers:
                ly.out.fill_(float("nan"))
                ly.lse.fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.stream(sa):
            a.step()
        with torch.cuda.stream(sb):
            b.step()
        torch.cuda.synchronize()
        for x, ref in zip((a, b), alone):
            for ly, (o, l_, i_, c_) in zip(x.layers, ref):
                assert torch.equal(ly.out, o) and torch.equal(ly.lse, l_), f"replay {rep}"
                assert torch.equal(ly.idx, i_) and torch.equal(ly.cnt, c_), f"replay {rep}"
    run_and_check(a, units=[(0, 0), (3, 7)], case="concurrent streams, stack64k shape")
    run_and_check(b, case="concurrent streams, ragged")


def test_workspace_grown_to_more_units_after_zero_fill():
    # A workspace used by calls of 2 units and then (after the documented zero-fill) of
    # 4 units, with a one-split call in between, gives exactly what fresh workspaces give.
    _gpu()
    from block_sparse_speculative_amd import _lib as L
    from block_sparse_speculative_amd import pipeline as PL
    small = W["llama32k"].with_(num_seqs=1, num_q_heads=8, num_kv_heads=2, ctx=(8192,))
    big = small.with_(num_seqs=2, ctx=(8192, 7000))
    insts = [Instance(small, seed=27, fused=True), Instance(big, seed=28, fused=True)]
    nbytes = max(L.select_and_attend_workspace_bytes(i.shape, i.k_max, s)
                 for i in insts for s in (0, 1, 3))
    shared = torch.zeros(nbytes, dtype=torch.uint8, device=insts[0].device)

    def call(inst, splits, ws):
        ly = inst.layers[0]
        idx, cnt = torch.empty_like(ly.idx), torch.empty_like(ly.cnt)
        out, lse = torch.empty_like(ly.out), torch.empty_like(ly.lse)
        L.select_and_attend(inst.shape, inst.budget, ly.q, ly.pool.reps, ly.k_draft, ly.v_draft,
                            ly.pool.k, ly.pool.v, inst.table, inst.ctx, inst.k_max, inst.scale,
                            idx, cnt, out, lse=lse, ws=ws, num_splits=splits)
        return idx, out, lse

    seq = [(0, 3), (0, 1), (0, 0), (1, 3), (1, 1), (1, 0), (1, 3)]
    for i, (which, splits) in enumerate(seq):
        inst = insts[which]
        if i == 3:
            shared.zero_()             # more units than before: zero-fill as documented
        got = call(inst, splits, shared)
        fresh = torch.zeros(L.select_and_attend_workspace_bytes(inst.shape, inst.k_max, splits),
                            dtype=torch.uint8, device=inst.device)
        want = call(inst, splits, fresh)
        torch.cuda.synchronize()
        for x, y in zip(got, want):
            assert torch.equal(x, y), f"call {i}"


def test_stack_with_reuse_small():
    _gpu()
    w = W["stack64k"].with_(num_seqs=2, num_q_heads=8, num_kv_heads=2, ctx=(8192, 7000))
    inst = Instance(w, seed=13, num_layers=4, nan_pool=True)
    run_and_check(inst, case="4-layer stack with reuse")


# ------------------------------------------------------------------ full sizes

def test_full_llama32k_all_units():
    _gpu()
    PT.log("[full] llama32k")
    inst = Instance(W["llama32k"], seed=1, fused=True)
    run_and_check(inst, case="full llama32k")
    del inst
    _free()


def test_full_ragged_all_units():
    # all 16 x 8 units of the ragged batch (contexts 4K-64K, paged), bench launch
    # configuration
    _gpu()
    PT.log("[full] ragged")
    inst = Instance(W["ragged"], seed=2, fused=True)
    PT.log(f"  ctx_lens={inst.ctx_lens} plan={inst.plan}")
    run_and_check(inst, case="full ragged")
    del inst
    _free()


def test_full_qwen128k_all_units():
    _gpu()
    PT.log("[full] qwen128k")
    inst = Instance(W["qwen128k"], seed=4, fused=True)
    PT.log(f"  plan={inst.plan}")
    run_and_check(inst, check_reps=False, case="full qwen128k")
    del inst
    _free()


@pytest.mark.parametrize("first,count", [(0, 4), (30, 2)])
def test_full_stack64k_layers_all_units(first, count):
    # all 4 x 8 units of stack64k layers 0-3 and 30-31 (select, reuse, select, reuse),
    # bench launch configuration (the layers' inputs are those of the 32-layer stack)
    _gpu()
    PT.log(f"[full] stack64k layers {first}..{first + count - 1}")
    inst = Instance(W["stack64k"], seed=3, fused=True, num_layers=count, layer_offset=first)
    PT.log(f"  plan={inst.plan}")
    run_and_check(inst, check_reps=False, case=f"full stack64k from L{first}")
    del inst
    _free()


def test_graph_replays_match_eager():
    # The bench replays a captured pass; every replay must equal the eager pass.
    _gpu()
    w = W["stack64k"].with_(num_seqs=2, num_q_heads=8, num_kv_heads=2, ctx=(8192, 7000))
    inst = Instance(w, seed=17, num_layers=4, fused=True)
    inst.step()
    torch.cuda.synchronize()
    eager = [(ly.idx.clone(), ly.cnt.clone(), ly.out.clone(), ly.lse.clone()) for ly in inst.layers]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        inst.step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        inst.step()
    for rep in range(4):
        for ly in inst.layers:           # clobber outputs so a stale value cannot pass
            ly.idx.fill_(-5)
            ly.out.fill_(float("nan"))
            ly.lse.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for ly, (i, c, o, s) in zip(inst.layers, eager):
            assert torch.equal(ly.idx, i) and torch.equal(ly.cnt, c)
            assert torch.equal(ly.out, o) and torch.equal(ly.lse, s)
        inst.step()                     # eager work between replays
        torch.cuda.synchronize()
