"""Helpers for the GPU parity tests: run the HIP path through the C ABI and compare
it, unit by unit, with the fp64 oracle on the same seeded inputs."""

from __future__ import annotations

import dataclasses
import sys

import numpy as np
import torch

import oracle as O
from oracle import sparse_ffn as OF

# Output tolerances: fp32 inputs 1e-4 max-abs; bf16 inputs (fp32 accumulation)
# 1e-2 max-abs and 5e-3 mean-abs. LSE is fp32 arithmetic on exactly representable
# inputs in both cases.
TOL = {"fp32": dict(max_abs=1e-4, mean_abs=1e-4), "bf16": dict(max_abs=1e-2, mean_abs=5e-3)}
LSE_TOL = 1e-4
NEAR_TIE_REL = 1e-5

# Element-wise bound for bf16 outputs, derived from the two bf16 roundings the path
# makes (unit roundoff u = 2^-8 for bf16's 8-bit significand; everything else is fp32):
#  - each softmax weight p_i meets V as bf16(p_i) = p_i (1 + d_i), |d_i| <= u, while the
#    denominator sums the fp32 p_i, so the output moves by at most u * sum p_i |v_i| /
#    sum p_i = u * O_abs, where O_abs is attention with |V| in place of V;
#  - the output is rounded to bf16: at most u * |O|.
# Hence |O_gpu - O_ref| <= u (|O_ref| + O_abs), plus second-order and fp32 terms, covered
# by a factor (1 + 2^-6) and 1e-6 absolute.
BF16_U = 2.0 ** -8
BF16_BOUND_FACTOR = 1.0 + 2.0 ** -6
BF16_BOUND_ABS = 1e-6

# Observed errors of every checked case, printed at the end of the test run.
STATS = []


def record(case: str, **fields):
    STATS.append(dict(case=case, **fields))


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


def oracle_select(u: UnitInputs, bs: int, budget, group: int, k_max=None):
    """Oracle scores and selection of one (sequence, KV head) unit. A `k_max` below the
    budget caps it (the C ABI's documented cap: the oracle selects with min(k, k_max))."""
    dense, mn, frac, kf, kl = budget
    reps = O.block_representatives(u.k_ctx, bs)
    scores = O.block_scores(u.q[0], reps, group)[0]
    k = O.budget_blocks(u.ctx, bs, dense, mn, frac)
    if k_max is not None:
        k = min(k, k_max)
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
    the same selection (and draft tree). Returns a dict of the observed errors:
    max_abs, mean_abs, rel (max_abs / RMS of the reference output), lse, and for bf16
    bound (the largest error as a fraction of its element-wise bound)."""
    ref, ref_lse = O.verify_attention(u.q, u.k_ctx, u.v_ctx, u.k_draft, u.v_draft, [sel], bs,
                                      scale, parents=parents)
    err = np.abs(gpu_out - ref)
    tol = TOL[dtype]
    assert np.isfinite(gpu_out).all(), "non-finite output"
    assert err.max() <= tol["max_abs"], f"max-abs {err.max():.3e} > {tol['max_abs']}"
    assert err.mean() <= tol["mean_abs"], f"mean-abs {err.mean():.3e} > {tol['mean_abs']}"
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    out = dict(max_abs=float(err.max()) if err.size else 0.0,
               mean_abs=float(err.mean()) if err.size else 0.0,
               rel=float(err.max() / rms) if rms > 0 else 0.0)
    if dtype == "bf16" and err.size:
        ref_abs, _ = O.verify_attention(u.q, u.k_ctx, np.abs(u.v_ctx), u.k_draft,
                                        np.abs(u.v_draft), [sel], bs, scale, parents=parents)
        bound = BF16_U * BF16_BOUND_FACTOR * (np.abs(ref) + ref_abs) + BF16_BOUND_ABS
        frac = err / bound
        worst = np.unravel_index(int(np.argmax(frac)), frac.shape)
        assert frac.max() <= 1.0, (
            f"bf16 element bound exceeded at {worst}: error {err[worst]:.3e}, bound "
            f"{bound[worst]:.3e} (|O| {abs(ref[worst]):.3e}, O_abs {ref_abs[worst]:.3e})")
        out["bound"] = float(frac.max())
    if gpu_lse is not None:
        lerr = np.abs(gpu_lse - ref_lse).max() if ref_lse.size else 0.0
        assert lerr <= LSE_TOL, f"lse error {lerr:.3e}"
        out["lse"] = float(lerr)
    return out


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
    sels = {}
    stats = {"units": 0, "exact": 0, "near-tie": 0, "max_abs": 0.0, "mean_abs": 0.0, "rel": 0.0,
             "bound": 0.0, "lse": 0.0}
    mean_sum = 0.0
    for (b, g) in units:
        u = unit_inputs(logical, b, g, G)
        nb = O.num_blocks(u.ctx, bs)
        gsel = gpu_unit_selection(idx, cnt, b, g)
        if prev_sel is not None:
            assert gsel == [int(x) for x in prev_sel[(b, g)]], "reuse layer changed the selection"
            used = np.array(gsel, dtype=np.int64)
        else:
            reps, scores, k, osel = oracle_select(u, bs, w.budget, G, inst.k_max)
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
        e = check_output(gout, glse, u, used, bs, inst.scale, w.dtype, parents=par)
        for key in ("max_abs", "rel", "bound", "lse"):
            stats[key] = max(stats[key], e.get(key, 0.0))
        mean_sum += e["mean_abs"]
        stats["units"] += 1
        sels[(b, g)] = used
    stats["mean_abs"] = mean_sum / max(stats["units"], 1)
    return sels, stats


def check_ffn(name, x, wg, wu, wd, tau, bits, yg):
    """Check one sparse FFN call against the oracle (oracle/sparse_ffn.py): keep decisions
    exact outside the fp32 band around tau, y within the element bound derived in
    tests/test_gpu_ffn.py's header. x [N, Dm], the weights [F, Dm] and y [N, Dm] as
    float64 arrays of the bf16 values; bits [F] the keep bit masks. Returns the observed
    errors with the keep decisions and y."""
    n, dm = x.shape
    f = wg.shape[0]
    gpu_keep = ((bits[None, :] >> np.arange(n)[:, None]) & 1).astype(bool)
    assert (bits >> n == 0).all(), "keep bits set for tokens >= N"
    a = OF.gate_activation(x, wg)
    ref_keep = OF.kept_channels(a, tau)
    depth = (2 * dm / 256 + 8) + 256 + 61 + (f / 64 + 1) + 8
    gamma = depth * 2.0 ** -24
    g_abs = np.abs(x) @ np.abs(wg).T
    u_abs = np.abs(x) @ np.abs(wu).T
    eps = 1.1 * gamma * g_abs + 4 * 2.0 ** -24 * np.abs(a)
    diff = gpu_keep != ref_keep
    near = np.abs(np.abs(a) - tau) <= eps
    assert not (diff & ~near).any(), (
        f"keep decisions differ outside the fp32 band at {np.argwhere(diff & ~near)[:5].tolist()}")
    y_ref, _ = OF.sparse_ffn(x, wg, wu, wd, tau, keep=gpu_keep)
    u = x @ wu.T
    h = np.where(gpu_keep, a * u, 0.0)
    y_abs = np.abs(h) @ np.abs(wd)
    prop = (np.where(gpu_keep, np.abs(a) * u_abs + 1.1 * np.abs(u) * g_abs, 0.0)) @ np.abs(wd)
    bound = (2.0 ** -8 * np.abs(y_ref) + gamma * (y_abs + prop) + 4 * 2.0 ** -24 * y_abs) * 1.01 \
        + 1e-30
    assert np.isfinite(yg).all()
    err = np.abs(yg - y_ref)
    frac = err / bound
    worst = np.unravel_index(int(np.argmax(frac)), frac.shape)
    assert frac.max() <= 1.0, (f"y error {err[worst]:.3e} above its bound {bound[worst]:.3e} at "
                               f"{worst} (|y| {abs(y_ref[worst]):.3e})")
    rms = float(np.sqrt(np.mean(y_ref ** 2))) if y_ref.size else 0.0
    kept_any = gpu_keep.any(axis=0).mean()
    st = dict(units=n, max_abs=float(err.max()), mean_abs=float(err.mean()),
              rel=float(err.max() / rms) if rms > 0 else 0.0, bound=float(frac.max()),
              lse=0.0)
    log(f"  {name} tau={tau}: kept per token {gpu_keep.mean():.3f}, channels any token "
        f"keeps {kept_any:.3f}, near-threshold mismatches {int(diff.sum())}, {st}")
    record(f"ffn {name} N{n} Dm{dm} F{f} tau{tau}", **st)
    return dict(st, kept_any=float(kept_any), keep=gpu_keep, y=yg)
