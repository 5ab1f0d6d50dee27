"""GPU: the attention entry point alone, on index sets it did not select.

sv_sparse_verify_attn is fed (a) the oracle's own selection of every unit and (b)
seeded random subsets of each unit's valid blocks (any count from none to every block
up to k_max, so first and last blocks may be absent and the blocks need not be the
best), through the library's split count and one split, with chain and tree drafts.
Every unit is checked against the oracle's attention over exactly that set, which
isolates the attention from the selection.
"""

import gc

import numpy as np
import pytest
import torch

from block_sparse_speculative_amd import pipeline as PL
from block_sparse_speculative_amd import synth
from block_sparse_speculative_amd.workload import Instance
from oracle import sparse_verify as O

import cases as C
import parity as PT

pytestmark = pytest.mark.gpu

CASES = {
    "llama_small": C.SMALL["llama_small"],
    "qwen_small_tree": C.SMALL["qwen_small"].with_(draft_tree="random"),
    "ragged_small": C.SMALL["ragged_small"],
    "fp32_d128": C.SMALL["fp32_d128"],
    "d64_bs32_star": C.SMALL["d64_bs32"].with_(draft_tree="star"),
    "long_table": C.SMALL["long_table"],
}


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("which", ["oracle", "random"])
@pytest.mark.parametrize("splits", [0, 1])
def test_attention_on_given_indices(name, which, splits):
    _gpu()
    w = CASES[name]
    PT.log(f"[given] {name} {which} splits={splits}")
    inst = Instance(w, seed=31, num_splits=splits, nan_pool=True)
    logical = inst.logical(0)
    G, bs, B, Hkv = w.group, w.block_size, w.num_seqs, w.num_kv_heads
    km = inst.k_max
    idx = torch.full((B, Hkv, km), -1, dtype=torch.int32)
    cnt = torch.zeros((B, Hkv), dtype=torch.int32)
    rng = np.random.default_rng(4099 + len(name) + (7 if which == "random" else 0) + splits)
    sets = {}
    for b in range(B):
        for g in range(Hkv):
            u = PT.unit_inputs(logical, b, g, G)
            nb = O.num_blocks(u.ctx, bs)
            if which == "oracle":
                sel = PT.oracle_select(u, bs, w.budget, G, km)[3]
            else:
                n = int(rng.integers(0, min(km, nb) + 1))
                sel = np.sort(rng.choice(nb, size=n, replace=False)) if n else np.zeros(0, int)
            sel = np.asarray(sel, dtype=np.int64)
            sets[(b, g)] = (u, sel)
            idx[b, g, :len(sel)] = torch.as_tensor(sel, dtype=torch.int32)
            cnt[b, g] = len(sel)
    ly = inst.layers[0]
    ly.out.fill_(float("nan"))
    ly.lse.fill_(float("nan"))
    PL.attend(inst.shape, ly.q, ly.k_draft, ly.v_draft, ly.pool, inst.table, inst.ctx,
              idx.to(inst.device), cnt.to(inst.device), km, inst.scale, ly.out, inst.ws,
              lse=ly.lse, draft_mask=inst.draft_mask)
    torch.cuda.synchronize()
    out, lse = PT.np64(ly.out), PT.np64(ly.lse)
    worst = {}
    for (b, g), (u, sel) in sets.items():
        par = None if inst.parents is None else inst.parents[b]
        e = PT.check_output(out[b, :, g * G:(g + 1) * G], lse[b, :, g * G:(g + 1) * G], u, sel,
                            bs, inst.scale, w.dtype, parents=par)
        for k, v in e.items():
            worst[k] = max(worst.get(k, 0.0), v)
    PT.record(f"given {name} {which} s{splits}", units=len(sets), **worst)
    del inst
    gc.collect()
    torch.cuda.empty_cache()
