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
from oracle import sparse_ffn as F

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
    n, dm, f = w.num_tokens, w.d_model, w.d_ffn
    bits = keep_bits.cpu().numpy().astype(np.int64) & 0xFFFFFFFF
    gpu_keep = ((bits[None, :] >> np.arange(n)[:, None]) & 1).astype(bool)
    assert (bits >> n == 0).all(), "keep bits set for tokens >= N"
    a = F.gate_activation(x, wg)
    ref_keep = F.kept_channels(a, tau)
    depth = (2 * dm / 256 + 8) + 256 + 61 + (f / 64 + 1) + 8
    gamma = depth * 2.0 ** -24
    g_abs = np.abs(x) @ np.abs(wg).T
    u_abs = np.abs(x) @ np.abs(wu).T
    eps = 1.1 * gamma * g_abs + 4 * 2.0 ** -24 * np.abs(a)
    diff = gpu_keep != ref_keep
    near = np.abs(np.abs(a) - tau) <= eps
    assert not (diff & ~near).any(), (
        f"keep decisions differ outside the fp32 band at {np.argwhere(diff & ~near)[:5].tolist()}")
    y_ref, _ = F.sparse_ffn(x, wg, wu, wd, tau, keep=gpu_keep)
    u = x @ wu.T
    h = np.where(gpu_keep, a * u, 0.0)
    y_abs = np.abs(h) @ np.abs(wd)
    prop = (np.where(gpu_keep, np.abs(a) * u_abs + 1.1 * np.abs(u) * g_abs, 0.0)) @ np.abs(wd)
    bound = (2.0 ** -8 * np.abs(y_ref) + gamma * (y_abs + prop) + 4 * 2.0 ** -24 * y_abs) * 1.01 \
        + 1e-30
    yg = _np(y)
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
    PT.log(f"  {w.name} tau={tau}: kept per token {gpu_keep.mean():.3f}, channels any token "
           f"keeps {kept_any:.3f}, near-threshold mismatches {int(diff.sum())}, {st}")
    PT.record(f"ffn {w.name} N{n} Dm{dm} F{f} tau{tau}", **st)
    return dict(st, kept_any=float(kept_any), keep=gpu_keep, y=yg)


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
