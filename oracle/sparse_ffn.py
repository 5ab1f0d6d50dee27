"""Plain fp64 reference for the threshold-pruned (sparse) FFN of the verification pass.

TEST INFRASTRUCTURE ONLY: used by ``tests/`` and ``bench.py``'s ``cpu_baseline`` leg;
never by the product path. It shares no code with the HIP library.

Sources:

* [TUT-T2]  Tutorial page "Accelerate Speculative Decoding with Sparse Computation in
  Verification", section "Core technique 2: plug-and-play sparse FFN": FFN activations
  are highly sparse; at inference time, channels whose intermediate activation is below
  a threshold tau are pruned dynamically, with no retraining, cutting matrix-product
  work.
* [SS-F1]   sciencestack page of arXiv 2512.21911, Figure 1 caption: in sparse FFN the
  pruned channels are determined by the output of the activation function and a given
  threshold.

Readings taken where the pages leave a step open:

* R21 the FFN is the gated (SwiGLU) FFN of the evaluated models (Llama-3.1-8B):
  y = W_down (SiLU(W_gate x) * (W_up x)); "the output of the activation function" is
  a = SiLU(W_gate x), per token and channel.
* R22 channel c of token t is pruned when |a[t, c]| < tau (strictly below); a pruned
  channel contributes nothing: its up-projection and down-projection terms are skipped.
  tau = 0 prunes nothing and gives the dense FFN.
* R23 every token decides for itself; the weights of a channel are needed if any token
  keeps it.

All arithmetic is float64; inputs may be bfloat16-valued arrays, widened exactly.
"""

from __future__ import annotations

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def silu(z):
    """SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z)), elementwise ([SS-F1]'s activation
    function of the gated FFN, reading R21)."""
    z = _f64(z)
    return z / (1.0 + np.exp(-z))


def gate_activation(x, w_gate):
    """a = SiLU(x W_gate^T) for every token and channel (reading R21).

    x: [N, Dm]; w_gate: [F, Dm] (row c = channel c's gate weights). Returns [N, F]."""
    return silu(_f64(x) @ _f64(w_gate).T)


def kept_channels(a, tau: float):
    """keep[t, c] = |a[t, c]| >= tau: the channels token t does not prune ([TUT-T2],
    [SS-F1], reading R22). Returns a bool array [N, F]."""
    return np.abs(_f64(a)) >= float(tau)


def sparse_ffn(x, w_gate, w_up, w_down_t, tau: float, keep=None):
    """The threshold-pruned gated FFN (readings R21-R23).

    x [N, Dm]; w_gate, w_up, w_down_t [F, Dm] (row c = channel c's weights; w_down_t is
    the down projection stored channel-major). keep: optional [N, F] bool decisions to
    use instead of the threshold (for checking a result against given decisions).
    Returns (y [N, Dm], keep [N, F]) with
      y[t] = sum over channels c kept by t of  a[t, c] * (x[t] . w_up[c]) * w_down_t[c].
    """
    xx = _f64(x)
    a = gate_activation(xx, w_gate)
    if keep is None:
        keep = kept_channels(a, tau)
    u = xx @ _f64(w_up).T
    h = np.where(keep, a * u, 0.0)
    return h @ _f64(w_down_t), np.asarray(keep, dtype=bool)
