"""GPU parity of the threshold-pruned FFN (sv_sparse_ffn, through the C ABI) against the
fp64 oracle (oracle/sparse_ffn.py), every token and output element.

Keep decisions (|a| >= tau) must match the oracle's exactly, except for channels whose
oracle activation lies within the fp32 error of the kernel's activation from tau (the
decision is taken in the kernel's precision there); y is then compared with the oracle
run on the kernel's decisions. Element bound on y, derived from the arithmetic: the
output is rounded to bf16 (at most 2^-8 |y|), and every sum is fp32 with at most D
sequential additions, so each computed dot product is within gamma = D * 2^-24 of its
sum of absolute terms, with D = (2 Dm/256 + 8) + 256 + 61 + (F/64 + 1) + 8:
  - the gate and up products are chains of Dm/256 MFMA steps per wave
    (v_mfma_f32_16x16x32_bf16: 32 products and the running sum per step, each step
    measured on gfx950 to stay within 1.89 * 2^-24 of its own sum of absolute terms)
    followed by the sum of the 8 waves' partials;
  - the down projection takes h as two bf16 parts, h = hi + lo + r with
    |r| <= 2^-16 |h| (256 units);
  - it then runs at most 16 MFMA K steps of two MFMAs per channel range (ranges of at
    most 512 channels: 2 * 1.89 * 16 < 61);
  - the range partials (at most F/64 + 1 of them) are summed in order;
  - 8 more cover the rounding of h = a u and slack. Propagated
through a = SiLU(g) (|SiLU'| <= 1.1), h = a u and y = sum_c h_c w_c:
  |y_gpu - y_ref| <= 2^-8 |y_ref| + gamma * (Y_abs + sum_c |w_cd| (|a_c| U_abs_c
                      + 1.1 |u_c| G_abs_c)) + 4 * 2^-24 * Y_abs,
with G_abs = |x| |W_gate|^T, U_abs = |x| |W_up|^T, Y_abs = |h| |W_down|, times 1.01.
"""

import numpy as np
import pytest
import torch

from block_sparse_speculative_amd import _lib as L
from block_sparse_speculative_amd import synth

import parity as PT

pytestmark = pytest.mark.gpu


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def run_ffn(w, seed, tau=None):
    """Run the GPU FFN and check it against the oracle. Returns the stats."""
    tau = w.tau if tau is None else tau
    dev = torch.device("cuda")
    inp = synth.make_ffn(w, seed, dev)
    shape = L.make_ffn_shape(w.num_tokens, w.d_model, w.d_ffn)
    ws = torch.empty(L.sparse_ffn_workspace_bytes(shape), dtype=torch.uint8, device=dev)
    y = torch.full((w.num_tokens, w.d_model), float("nan"), dtype=torch.bfloat16, device=dev)
    keep_bits = torch.full((w.d_ffn,), -1, dtype=torch.int32, device=dev)
    L.sparse_ffn(shape, inp["x"], inp["w_gate"], inp["w_up"], inp["w_down_t"], tau, y,
                 keep_bits=keep_bits, ws=ws)
    torch.cuda.synchronize()
    x, wg, wu, wd = (_np(inp[k]) for k in ("x", "w_gate", "w_up", "w_down_t"))
    bits = keep_bits.cpu().numpy().astype(np.int64) & 0xFFFFFFFF
    return PT.check_ffn(w.name, x, wg, wu, wd, tau, bits, _np(y))


FFN = synth.FFN_WORKLOADS["ffn_llama8b"]
SMALL_FFN = {
    "n8_dm1024_f2048": FFN.__class__("n8_dm1024_f2048", 8, 1024, 2048, 0.9, 0.3),
    "n5_dm512_f1000": FFN.__class__("n5_dm512_f1000", 5, 512, 1000, 0.9, 0.3),     # ragged F, N
    "n1_dm512_f600": FFN.__class__("n1_dm512_f600", 1, 512, 600, 0.9, 0.3),        # one token
    "n16_dm2048_f3000": FFN.__class__("n16_dm2048_f3000", 16, 2048, 3000, 0.9, 0.25),
    "n16_dm4096_f1536": FFN.__class__("n16_dm4096_f1536", 16, 4096, 1536, 0.5, 0.3),  # 128 KB x
    "n12_dm8192_f700": FFN.__class__("n12_dm8192_f700", 8, 8192, 700, 0.9, 0.3),    # widest Dm
}


@pytest.mark.parametrize("name", list(SMALL_FFN))
def test_sparse_ffn_small_shapes_every_element(name):
    _gpu()
    run_ffn(SMALL_FFN[name], seed=3)


@pytest.mark.parametrize("tau", [0.0, 0.1, 0.3, 0.6])
def test_sparse_ffn_full_size_every_element(tau):
    # the Llama-3.1-8B FFN shape, 8 draft tokens
    _gpu()
    st = run_ffn(FFN, seed=5, tau=tau)
    if tau == 0.0:
        assert st["keep"].all()


def test_tau_above_every_activation_prunes_all_and_gives_zero():
    _gpu()
    st = run_ffn(SMALL_FFN["n8_dm1024_f2048"], seed=4, tau=1e9)
    assert not st["keep"].any() and (st["y"] == 0.0).all()


def test_sparse_ffn_bit_identical_run_to_run():
    _gpu()
    a = run_ffn(FFN, seed=6)
    b = run_ffn(FFN, seed=6)
    assert np.array_equal(a["y"], b["y"]) and np.array_equal(a["keep"], b["keep"])


def test_sparse_ffn_largest_shape_every_element():
    # Llama-3-70B's FFN shape (d_model 8192, d_ffn 28672; 470 MB per weight matrix):
    # the widest x stage, the longest gate/up slices and 512-channel down ranges
    _gpu()
    w = FFN.__class__("ffn_70b_shape", 8, 8192, 28672, 0.9, 0.3)
    st = run_ffn(w, seed=9)
    assert 0.2 < st["kept_any"] < 0.9


def test_sparse_ffn_sixteen_tokens_full_size_every_element():
    # 16 draft tokens (the most the entry point takes) through the Llama-3.1-8B shape
    _gpu()
    run_ffn(FFN.__class__("ffn_llama8b_n16", 16, 4096, 14336, 0.9, 0.3), seed=10)


# ---- seeded sweep over the envelope: token counts 1-16, model dims 512 x 1..8 (within
# the x-staging limit), channel counts at and around the 16-channel gate tiles and the
# 64-channel range granule as well as ragged ones, thresholds from dense to prune-all,
# and token correlations from none to strong.
NUM_FFN_CASES = 24


def ffn_sweep_case(i: int):
    r = np.random.default_rng(104729 * i + 3)
    n = int(r.integers(1, 17))
    dm_max = 8 if n <= 8 else 4
    dm = 512 * int(r.integers(1, dm_max + 1))
    if r.random() < 0.4:
        f = int(r.choice([1, 15, 16, 17, 63, 64, 65, 511, 512, 513]))
    else:
        f = int(r.integers(100, 6001))
    u = r.random()
    tau = 0.0 if u < 0.15 else (8.0 if u < 0.25 else float(r.uniform(0.05, 0.8)))
    rho = float(r.choice([0.0, 0.5, 0.9]))
    return FFN.__class__(f"sweep{i}_n{n}_dm{dm}_f{f}", n, dm, f, rho, tau)


def test_ffn_sweep_inside_the_envelope():
    names = set()
    for i in range(NUM_FFN_CASES):
        w = ffn_sweep_case(i)
        assert 1 <= w.num_tokens <= 16 and w.d_model % 512 == 0
        assert (8 if w.num_tokens <= 8 else 16) * w.d_model * 2 <= 128 * 1024
        names.add(w.name)
    assert len(names) == NUM_FFN_CASES


@pytest.mark.parametrize("i", range(NUM_FFN_CASES))
def test_sparse_ffn_sweep_every_element(i):
    _gpu()
    w = ffn_sweep_case(i)
    PT.log(f"[ffn sweep {i}] N {w.num_tokens} Dm {w.d_model} F {w.d_ffn} tau {w.tau:.3f} "
           f"rho {w.rho}")
    st = run_ffn(w, seed=200 + i)
    if w.tau == 0.0:
        assert st["keep"].all()
    if w.tau >= 8.0:
        assert not st["keep"].any() and (st["y"] == 0.0).all()
