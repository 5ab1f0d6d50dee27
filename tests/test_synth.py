"""The seeded synthetic inputs (block_sparse_speculative_amd/synth.py) that stand in for
the pages' workloads: determinism, the counts and ranges each recipe states, the paged
block table, the reuse-layer heavy sets, the draft-query correlation and the FFN inputs.
CPU only; small shapes."""

import math

import pytest
import torch

from block_sparse_speculative_amd import synth

W = synth.WORKLOADS


def _corr(a, b):
    a = a.double().flatten() - a.double().mean()
    b = b.double().flatten() - b.double().mean()
    return float((a @ b) / (a.norm() * b.norm()))


def test_same_seed_gives_identical_inputs_and_seeds_and_layers_differ():
    w = W["tiny"]
    a, b = synth.make_layer(w, 3), synth.make_layer(w, 3)
    for key in ("q", "k_ctx", "v_ctx", "k_draft", "v_draft"):
        assert torch.equal(a[key], b[key]), key
    assert a["heavy"] == b["heavy"]
    assert not torch.equal(a["k_ctx"], synth.make_layer(w, 4)["k_ctx"])
    assert not torch.equal(a["q"], synth.make_layer(w, 3, layer=1)["q"])


@pytest.mark.parametrize("name,nb,n", [
    ("tiny", 64, 4),          # a fixed 4 planted blocks
    ("llama32k", 512, 15),    # round-half-up(3 % of 512)
    ("stack64k", 1024, 31),   # round-half-up(3 % of 1024)
    ("qwen128k", 1024, 20),   # round-half-up(2 % of 1024)
])
def test_planted_counts_follow_the_recipes(name, nb, n):
    w = W[name]
    assert synth.num_blocks(w.ctx[0], w.block_size) == nb
    assert synth.planted_count(w, nb) == n


def test_planted_blocks_are_distinct_non_forced_and_lifted_along_the_group_query():
    w = W["llama32k"].with_(num_seqs=2, num_q_heads=8, num_kv_heads=2, ctx=(8192, 5000))
    x = synth.make_layer(w, 5)
    bs, G = w.block_size, w.group
    for b, ctx in enumerate(x["ctx_lens"]):
        nb = synth.num_blocks(ctx, bs)
        for g in range(w.num_kv_heads):
            blocks = x["heavy"][b][g]
            assert blocks == sorted(set(blocks))
            assert len(blocks) == synth.planted_count(w, nb)
            assert all(1 <= j <= nb - 2 for j in blocks)        # never a forced block
            qg = x["q"][b, 0, g * G:(g + 1) * G].float().sum(0)
            qhat = qg / qg.norm()
            proj = (x["k_ctx"][b, :ctx, g].float() @ qhat).reshape(-1)
            tok = torch.zeros(ctx, dtype=torch.bool)
            for j in blocks:
                tok[j * bs:(j + 1) * bs] = True
            # planted keys gain plant_alpha along q-hat; the others are N(0, 1) along it
            assert abs(float(proj[tok].mean()) - w.plant_alpha) < 0.15
            assert abs(float(proj[~tok].mean())) < 0.1
    # tokens past a context are zero
    assert float(x["k_ctx"][1, 5000:].abs().max()) == 0.0


def test_ragged_contexts_are_multiples_of_64_in_range_and_seeded():
    w = W["ragged"]
    seen = set()
    for seed in range(6):
        lens = synth.context_lengths(w, seed)
        assert len(lens) == w.num_seqs
        assert all(c % 64 == 0 and 4096 <= c <= 65536 for c in lens)
        assert lens == synth.context_lengths(w, seed)
        seen.add(tuple(lens))
    assert len(seen) == 6


def test_paged_block_table_is_a_permutation_and_unpaged_is_the_identity():
    w = W["ragged"]
    lens = synth.context_lengths(w, 2)
    table, P = synth.block_table(w, lens, 2)
    nbs = [synth.num_blocks(c, w.block_size) for c in lens]
    assert P == sum(nbs) and table.shape == (w.num_seqs, max(nbs))
    used = torch.cat([table[b, :nbs[b]] for b in range(w.num_seqs)])
    assert torch.equal(used.sort().values, torch.arange(P, dtype=torch.int32))
    assert not torch.equal(used, torch.arange(P, dtype=torch.int32))   # actually scattered
    w2 = W["stack64k"]
    t2, P2 = synth.block_table(w2, list(w2.ctx), 0)
    assert P2 == w2.num_seqs * 1024
    for b in range(w2.num_seqs):
        assert torch.equal(t2[b], torch.arange(1024, dtype=torch.int32) + 1024 * b)


def test_stack_odd_layers_keep_four_fifths_of_the_even_layers_heavy_set():
    w = W["stack64k"]
    ctx = list(w.ctx)
    even = synth.planted_sets(w, ctx, 0, 2)
    odd = synth.planted_sets(w, ctx, 0, 3)
    nxt = synth.planted_sets(w, ctx, 0, 4)
    for b in range(w.num_seqs):
        for g in range(w.num_kv_heads):
            e, o = set(even[b][g]), set(odd[b][g])
            assert len(e) == len(o) == 31
            assert len(e & o) == 25 and len(o - e) == 6       # round(0.8 * 31) kept, 6 fresh
    assert even != nxt                                        # the next pair draws anew


def test_draft_queries_correlate_with_the_first_at_rho():
    w = W["llama32k"].with_(num_seqs=4, ctx=(512,) * 4)
    q = synth.make_layer(w, 1)["q"].float()
    for t in range(1, w.num_draft):
        assert abs(_corr(q[:, 0], q[:, t]) - w.draft_rho) < 0.03
    # the drafts' fresh parts are independent of each other: corr(q_1, q_2) = rho^2
    assert abs(_corr(q[:, 1], q[:, 2]) - w.draft_rho ** 2) < 0.03


def test_ffn_inputs_follow_the_recipe():
    w = synth.FfnWorkload("ffn_small", 8, 1024, 4096, 0.9, 0.3)
    d = synth.make_ffn(w, 0)
    e = synth.make_ffn(w, 0)
    for key in ("x", "w_gate", "w_up", "w_down_t"):
        assert torch.equal(d[key], e[key]) and d[key].dtype == torch.bfloat16
    x = d["x"].float()
    assert abs(_corr(x[0], x[1]) - w.rho ** 2) < 0.05          # shared component
    assert abs(float(d["w_gate"].float().std()) * math.sqrt(w.d_model) - 1.0) < 0.02
    assert abs(float(d["w_down_t"].float().std()) * math.sqrt(w.d_ffn) - 1.0) < 0.02
    # gate pre-activations ~N(0, |x|^2 / d_model): about N(0, 1), up to the norm of the one
    # drawn shared component
    g = x @ d["w_gate"].float().T
    pred = float(x.pow(2).sum(1).mean().sqrt() * d["w_gate"].float().std())
    assert abs(float(g.std()) / pred - 1.0) < 0.03
    assert 0.85 < pred < 1.15
