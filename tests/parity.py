"""Helpers for the GPU parity tests: run the HIP path through the C ABI and compare
it, unit by unit, with the fp64 oracle on the same seeded inputs."""

from __future__ import annotations

import dataclasses
import sys

import numpy as np
import torch

import oracle as O

# Output tolerances: fp32 inputs 1e-4 max-abs; bf16 inputs (fp32 accumulation)
# 1e-2 max-abs and 5e-3 mean-abs. LSE is fp32 arithmetic on exactly representable
# inputs in both cases.
TOL = {"fp32": dict(max_abs=1e-4, mean_abs=1e-4), "bf16": dict(max_abs=1e-2, mean_abs=5e-3)}
LSE_TOL = 1e-4
NEAR_TIE_REL = 1e-5


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


@dataclasses.dataclass
class UnitInputs:
    q: np.ndarray        # [T, G, D]
    k_ctx: np.ndarray    # [ctx, 1, D]
    v_ctx: np.ndarray
    k_draft: np.ndarray  # [T, 1, D]
    v_draft: np.ndarray
    ctx: int


def unit_inputs(logical, b: int, g: int, group: int) -> UnitInputs:
    ctx = logical["ctx_lens"][b]
    sl = slice(g, g + 1)
    return UnitInputs(
        q=np64(logical["q"][b, :, g * group:(g + 1) * group]),
        k_ctx=np64(logical["k_ctx"][b, :ctx, sl]),
        v_ctx=np64(logical["v_ctx"][b, :ctx, sl]),
        k_draft=np64(logical["k_draft"][b, :, sl]),
        v_draft=np64(logical["v_draft"][b, :, sl]),
        ctx=ctx)


def oracle_select(u: UnitInputs, bs: int, budget, group: int):
    """Oracle scores and selection of one (sequence, KV head) unit."""
    dense, mn, frac, kf, kl = budget
    reps = O.block_representatives(u.k_ctx, bs)
    scores = O.block_scores(u.q[0], reps, group)[0]
    k = O.budget_blocks(u.ctx, bs, dense, mn, frac)
    sel = O.select_blocks(scores, k, bool(kf), bool(kl))
    return reps[:, 0], scores, k, sel


def check_selection(gpu_sel, oracle_sel, scores, k, nb, keep_first, keep_last):
    """Exact match, or the documented near-tie exception. Returns 'exact' or 'near-tie'."""
    gpu_sel = [int(x) for x in gpu_sel]
    oracle_sel = [int(x) for x in oracle_sel]
    assert gpu_sel == sorted(gpu_sel), "GPU selection not ascending"
    assert len(set(gpu_sel)) == len(gpu_sel), "GPU selection has duplicates"
    if gpu_sel == oracle_sel:
        return "exact"
    assert len(gpu_sel) == len(oracle_sel) == min(k, nb), (len(gpu_sel), len(oracle_sel), k)
    forced = set(([0] if keep_first else []) + ([nb - 1] if keep_last else []))
    assert forced <= set(gpu_sel), "forced blocks missing"
    cand = [j for j in range(nb) if j not in forced]
    cand.sort(key=lambda j: (-scores[j], j))
    kk = k - len(forced)
    assert kk >= 1, "selections differ although only forced blocks are kept"
    s_k, s_k1 = scores[cand[kk - 1]], scores[cand[kk]]
    band = NEAR_TIE_REL * abs(s_k)
    assert abs(s_k - s_k1) < band, (
        f"index mismatch outside the near-tie band: k-th {s_k!r}, (k+1)-th {s_k1!r}, "
        f"gpu-only {sorted(set(gpu_sel) - set(oracle_sel))}, "
        f"oracle-only {sorted(set(oracle_sel) - set(gpu_sel))}")
    diff = set(gpu_sel) ^ set(oracle_sel)
    assert all(abs(scores[j] - s_k) <= band for j in diff), "mismatch outside the tie band"
    return "near-tie"


def check_output(gpu_out, gpu_lse, u: UnitInputs, sel, bs: int, scale: float, dtype: str,
                 parents=None):
    """Compare one unit's GPU output [T, G, D] (and lse [T, G]) with the oracle run on
    the same selection (and draft tree). Returns (max_abs, mean_abs)."""
    ref, ref_lse = O.verify_attention(u.q, u.k_ctx, u.v_ctx, u.k_draft, u.v_draft, [sel], bs,
                                      scale, parents=parents)
    err = np.abs(gpu_out - ref)
    tol = TOL[dtype]
    assert np.isfinite(gpu_out).all(), "non-finite output"
    assert err.max() <= tol["max_abs"], f"max-abs {err.max():.3e} > {tol['max_abs']}"
    assert err.mean() <= tol["mean_abs"], f"mean-abs {err.mean():.3e} > {tol['mean_abs']}"
    if gpu_lse is not None:
        lerr = np.abs(gpu_lse - ref_lse).max()
        assert lerr <= LSE_TOL, f"lse error {lerr:.3e}"
    return float(err.max()), float(err.mean())


def check_reps(gpu_reps, u: UnitInputs, bs: int, oracle_reps):
    """Representatives within the fp32 recursive-summation bound
    |err| <= 2^-24 * (sum_i |k_i| + |mean|) per element (plus the division)."""
    nb = oracle_reps.shape[0]
    k = u.k_ctx[:, 0]
    bound = np.zeros_like(oracle_reps)
    for j in range(nb):
        blk = k[j * bs: min(u.ctx, (j + 1) * bs)]
        bound[j] = 2.0 ** -24 * (np.abs(blk).sum(axis=0) + np.abs(oracle_reps[j])) * 1.01 + 1e-30
    err = np.abs(gpu_reps - oracle_reps)
    assert (err <= bound).all(), f"representative error {err.max():.3e} above bound"


def gpu_unit_selection(idx, cnt, b, g):
    c = int(cnt[b, g])
    row = idx[b, g].tolist()
    assert all(x == -1 for x in row[c:]), "padding must be -1"
    return row[:c]


def verify_instance_units(inst, layer: int, units, logical=None, prev_sel=None, check_reps_too=False,
                          gpu_scores=None):
    """Run the parity checks for the listed (b, g) units of one layer of a workload
    instance (after its GPU pass). Returns {(b, g): selection used} and stats."""
    w = inst.w
    if logical is None:
        logical = inst.logical(layer)
    ly = inst.layers[layer]
    idx = ly.idx.cpu()
    cnt = ly.cnt.cpu()
    out = np64(ly.out)
    lse = None if ly.lse is None else np64(ly.lse)
    G, bs = w.group, w.block_size
    kf, kl = w.budget[3], w.budget[4]
    sels, stats = {}, {"exact": 0, "near-tie": 0, "max_abs": 0.0}
    for (b, g) in units:
        u = unit_inputs(logical, b, g, G)
        nb = O.num_blocks(u.ctx, bs)
        gsel = gpu_unit_selection(idx, cnt, b, g)
        if prev_sel is not None:
            assert gsel == [int(x) for x in prev_sel[(b, g)]], "reuse layer changed the selection"
            used = np.array(gsel, dtype=np.int64)
        else:
            reps, scores, k, osel = oracle_select(u, bs, w.budget, G)
            assert int(cnt[b, g]) == min(k, nb)
            kind = check_selection(gsel, osel, scores, k, nb, kf, kl)
            stats[kind] += 1
            used = np.array(gsel, dtype=np.int64)
            if gpu_scores is not None:
                gs = np64(gpu_scores[b, g, :nb])
                qs = np.abs(u.q[0]).sum(axis=0)
                bound = 1e-5 * (np.abs(reps) @ qs) + 1e-6
                assert (np.abs(gs - scores) <= bound).all(), "score error above bound"
            if check_reps_too:
                phys = inst.table_host[b, :nb].numpy()
                check_reps(np64(ly.pool.reps[torch.as_tensor(phys, device=ly.pool.reps.device), g]),
                           u, bs, reps)
        gout = out[b, :, g * G:(g + 1) * G]
        glse = None if lse is None else lse[b, :, g * G:(g + 1) * G]
        par = None if inst.parents is None else inst.parents[b]
        mx, _ = check_output(gout, glse, u, used, bs, inst.scale, w.dtype, parents=par)
        stats["max_abs"] = max(stats["max_abs"], mx)
        sels[(b, g)] = used
    return sels, stats
