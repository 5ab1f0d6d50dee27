"""Pins of the sparse-FFN oracle (oracle/sparse_ffn.py) to things other than itself: a
library SiLU and a dense gated FFN built from torch.nn layers, closed forms, a
brute-force loop on tiny inputs, the exact threshold boundary, and invariants chosen so
that a dropped absolute value, a strict/non-strict swap, a transposed weight or a
missing up-projection fails one of them."""

import math

import numpy as np
import pytest
import torch

from oracle import sparse_ffn as F


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def test_silu_matches_torch_and_its_closed_forms():
    z = np.linspace(-30, 30, 1201)
    ref = torch.nn.functional.silu(torch.tensor(z, dtype=torch.float64)).numpy()
    assert np.allclose(F.silu(z), ref, rtol=1e-15, atol=1e-300)
    assert F.silu(np.array([0.0]))[0] == 0.0
    assert F.silu(np.array([1.0]))[0] == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15)
    # the negative lobe's minimum: z = -1.27846..., SiLU = -0.27846...
    assert F.silu(np.linspace(-10, 0, 100001)).min() == pytest.approx(-0.2784645, abs=1e-6)


def test_tau_zero_is_the_dense_gated_ffn_of_torch_layers():
    n, dm, f = 5, 24, 40
    x = _rand((n, dm), 1)
    wg, wu, wd = _rand((f, dm), 2, 0.3), _rand((f, dm), 3, 0.3), _rand((f, dm), 4, 0.3)
    gate = torch.nn.Linear(dm, f, bias=False, dtype=torch.float64)
    up = torch.nn.Linear(dm, f, bias=False, dtype=torch.float64)
    down = torch.nn.Linear(f, dm, bias=False, dtype=torch.float64)
    with torch.no_grad():
        gate.weight.copy_(torch.tensor(wg))
        up.weight.copy_(torch.tensor(wu))
        down.weight.copy_(torch.tensor(wd).T)        # Linear weight is [out, in]
        xt = torch.tensor(x)
        ref = down(torch.nn.functional.silu(gate(xt)) * up(xt)).numpy()
    y, keep = F.sparse_ffn(x, wg, wu, wd, 0.0)
    assert keep.all()
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_loops_on_tiny_inputs(seed):
    n, dm, f = 3, 5, 7
    x = _rand((n, dm), 10 + seed)
    wg, wu, wd = _rand((f, dm), 20 + seed), _rand((f, dm), 30 + seed), _rand((f, dm), 40 + seed)
    tau = 0.35
    y, keep = F.sparse_ffn(x, wg, wu, wd, tau)
    for t in range(n):
        for d in range(dm):
            acc = 0.0
            for c in range(f):
                g = sum(x[t][k] * wg[c][k] for k in range(dm))
                a = g / (1.0 + math.exp(-g))
                if abs(a) < tau:
                    continue                          # pruned channel
                u = sum(x[t][k] * wu[c][k] for k in range(dm))
                acc += a * u * wd[c][d]
            assert y[t, d] == pytest.approx(acc, rel=1e-12, abs=1e-12)
    assert keep.any() and not keep.all()             # the threshold actually prunes here


def test_one_hot_activation_closed_form():
    # gate pre-activations: +8 for channel 2 of token 0, -40 elsewhere (|SiLU(-40)| ~ 2e-16)
    dm, f = 6, 5
    x = np.zeros((1, dm))
    x[0, 0] = 1.0
    wg = np.full((f, dm), 0.0)
    wg[:, 0] = -40.0
    wg[2, 0] = 8.0
    wu, wd = _rand((f, dm), 5), _rand((f, dm), 6)
    y, keep = F.sparse_ffn(x, wg, wu, wd, 0.5)
    assert keep[0].tolist() == [False, False, True, False, False]
    a = 8.0 / (1.0 + math.exp(-8.0))
    want = a * wu[2, 0] * wd[2]
    assert np.allclose(y[0], want, rtol=1e-14, atol=0)


def test_threshold_boundary_is_kept_and_pruning_is_on_the_magnitude():
    # g = 0 gives a = 0 exactly: kept at tau = 0, pruned at any tau > 0
    x = np.zeros((1, 4))
    w = np.ones((3, 4))
    _, keep0 = F.sparse_ffn(x, w, w, w, 0.0)
    _, keep1 = F.sparse_ffn(x, w, w, w, 1e-300)
    assert keep0.all() and not keep1.any()
    # negative activations: |SiLU(g)| <= 0.2785 for g < 0, so at tau = 0.2 some channels
    # with g in (-2.3, -0.6) are kept (a rule without the absolute value keeps none)
    rng = np.random.default_rng(7)
    xs = rng.standard_normal((8, 16))
    wg = rng.standard_normal((64, 16)) * 0.4
    g = xs @ wg.T
    _, keep = F.sparse_ffn(xs, wg, wg, wg, 0.2)
    assert (keep & (g < 0)).any()
    assert not (keep & (g < 0) & (np.abs(F.silu(g)) < 0.2)).any()
    _, keep3 = F.sparse_ffn(xs, wg, wg, wg, 0.28)
    assert not (keep3 & (g < 0)).any()


def test_tau_above_every_activation_gives_zero_and_keep_sets_nest():
    n, dm, f = 4, 12, 30
    x = _rand((n, dm), 8)
    wg, wu, wd = _rand((f, dm), 9, 0.5), _rand((f, dm), 11), _rand((f, dm), 12)
    a = F.gate_activation(x, wg)
    y, keep = F.sparse_ffn(x, wg, wu, wd, float(np.abs(a).max()) * 1.0001)
    assert not keep.any() and (y == 0.0).all()
    prev = None
    for tau in (0.0, 0.05, 0.1, 0.3, 0.6, 1.0):
        _, k = F.sparse_ffn(x, wg, wu, wd, tau)
        if prev is not None:
            assert not (k & ~prev).any()              # raising tau never un-prunes
        prev = k


def test_given_decisions_and_linearity_in_the_down_projection():
    n, dm, f = 3, 10, 20
    x = _rand((n, dm), 13)
    wg, wu, wd = _rand((f, dm), 14, 0.5), _rand((f, dm), 15), _rand((f, dm), 16)
    y, keep = F.sparse_ffn(x, wg, wu, wd, 0.25)
    y2, _ = F.sparse_ffn(x, wg, wu, wd, 123.0, keep=keep)   # decisions given: tau unused
    assert np.array_equal(y, y2)
    y3, _ = F.sparse_ffn(x, wg, wu, 2.5 * wd, 0.25)
    assert np.allclose(y3, 2.5 * y, rtol=1e-14, atol=1e-14)
    # the up projection matters: swapping gate and up weights changes the result
    y4, _ = F.sparse_ffn(x, wu, wg, wd, 0.0)
    y5, _ = F.sparse_ffn(x, wg, wu, wd, 0.0)
    assert not np.allclose(y4, y5)
