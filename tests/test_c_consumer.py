"""The C ABI from plain C: tests/c/sv_consumer.c, a C99 program that links libsv.so and
the HIP runtime, with no Python and no C++ between it and the library.

CPU: the consumer compiles as C99 with -pedantic -Werror against include/sv.h, and its
host mode passes (ABI version, status names, the budget formula, workspace and plan
queries, rejections with their messages, a misaligned pointer named in the error).

GPU: its gpu mode runs one verification layer through every entry point on a small
paged problem (2 sequences of 1000 and 2500 tokens, 8 query and 2 KV heads, head dim
128, bf16, 4 chain drafts, 8 blocks selected of 16 and 40) and a small sparse FFN
(4 tokens, 512 x 600, tau 0.3), and writes its inputs and outputs. Here they are checked
against the oracle:
  - the pool holds every appended token bit for bit where the table maps it;
  - the representatives are within their fp32 summation bound;
  - the selection matches (exact, or the near-tie rule);
  - attention on the selection and the fused call both match within the bf16 bound;
  - the fused call selects exactly what the separate call does;
  - the allocation-free fused call equals the fused call bit for bit (compared in C);
  - reuse copies exactly;
  - the FFN keeps and output match within the bound derived for it.
"""

import os
import shutil
import subprocess
import sys

import numpy as np
import pytest

from block_sparse_speculative_amd import _lib as L

import parity as PT

sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), "c"))
import build_consumer as BC  # noqa: E402


def _can_build():
    try:
        BC.rocm()
    except RuntimeError:
        return False
    return os.path.exists(L.LIB_PATH) and bool(shutil.which("gcc") or shutil.which("cc"))


def test_c_consumer_compiles_as_c99_and_checks_the_host_abi(tmp_path):
    if not _can_build():
        pytest.skip("libsv.so, a C compiler or the ROCm headers are missing")
    exe = BC.build(str(tmp_path / "sv_consumer"))
    r = subprocess.run([exe, "host"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host ok" in r.stdout


def _bf16(u16):
    return (u16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _load(d, name, dtype, shape):
    a = np.fromfile(os.path.join(d, name), dtype=dtype)
    assert a.size == int(np.prod(shape)), f"{name}: {a.size} elements, expected {shape}"
    return a.reshape(shape)


@pytest.mark.gpu
def test_c_consumer_layer_matches_the_oracle(tmp_path):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(BC.OUT):
        pytest.skip("tests/c/sv_consumer is not built (__graft_entry__.build() builds it)")
    PT.log("  C consumer: one layer and a sparse FFN through the C ABI")
    r = subprocess.run([BC.OUT, "gpu", str(tmp_path)], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    meta = {}
    for line in open(tmp_path / "meta.txt"):
        k, v = line.split()
        meta[k] = float(v)
    m = {k: int(v) for k, v in meta.items() if k not in ("SCALE", "TAU")}
    B, HQ, HKV, D, BS, T = m["B"], m["HQ"], m["HKV"], m["D"], m["BS"], m["T"]
    NB, P, NMAX, KMAX = m["NB"], m["P"], m["NMAX"], m["KMAX"]
    G = HQ // HKV
    ctx = [m["CTX0"], m["CTX1"]]
    budget = (m["DENSE"], m["MIN"], m["FRAC"], m["KF"], m["KL"])
    scale = meta["SCALE"]
    d = str(tmp_path)
    k_new = _load(d, "k_new.bin", np.uint16, (B, NMAX, HKV, D))
    v_new = _load(d, "v_new.bin", np.uint16, (B, NMAX, HKV, D))
    q = _bf16(_load(d, "q.bin", np.uint16, (B, T, HQ, D)))
    kd = _bf16(_load(d, "k_draft.bin", np.uint16, (B, T, HKV, D)))
    vd = _bf16(_load(d, "v_draft.bin", np.uint16, (B, T, HKV, D)))
    table = _load(d, "table.bin", np.int32, (B, NB))
    k_pool = _load(d, "k_pool.bin", np.uint16, (P, HKV, BS, D))
    v_pool = _load(d, "v_pool.bin", np.uint16, (P, HKV, BS, D))
    reps = _load(d, "reps.bin", np.float32, (P, HKV, D)).astype(np.float64)
    idx, idx2, idx3 = (_load(d, f"{n}.bin", np.int32, (B, HKV, KMAX))
                       for n in ("idx", "idx2", "idx3"))
    cnt, cnt2, cnt3 = (_load(d, f"{n}.bin", np.int32, (B, HKV)) for n in ("cnt", "cnt2", "cnt3"))
    out, out2 = (_bf16(_load(d, f"{n}.bin", np.uint16, (B, T, HQ, D))) for n in ("out", "out2"))
    lse, lse2 = (_load(d, f"{n}.bin", np.float32, (B, T, HQ)).astype(np.float64)
                 for n in ("lse", "lse2"))

    # the append wrote every token where the table maps it
    for b in range(B):
        for j in range((ctx[b] + BS - 1) // BS):
            n = min(BS, ctx[b] - j * BS)
            p = int(table[b, j])
            want_k = k_new[b, j * BS:j * BS + n].transpose(1, 0, 2)
            want_v = v_new[b, j * BS:j * BS + n].transpose(1, 0, 2)
            assert np.array_equal(k_pool[p, :, :n], want_k), f"K of block ({b}, {j})"
            assert np.array_equal(v_pool[p, :, :n], want_v), f"V of block ({b}, {j})"
    assert np.array_equal(idx2, idx) and np.array_equal(cnt2, cnt), "fused and separate selections"
    assert np.array_equal(idx3, idx) and np.array_equal(cnt3, cnt), "reuse copy"

    worst = {}
    for b in range(B):
        nb = (ctx[b] + BS - 1) // BS
        k_ctx = _bf16(k_new[b, :ctx[b]])
        v_ctx = _bf16(v_new[b, :ctx[b]])
        for g in range(HKV):
            u = PT.UnitInputs(q=q[b, :, g * G:(g + 1) * G], k_ctx=k_ctx[:, g:g + 1],
                              v_ctx=v_ctx[:, g:g + 1], k_draft=kd[b, :, g:g + 1],
                              v_draft=vd[b, :, g:g + 1], ctx=ctx[b])
            o_reps, o_scores, k, o_sel = PT.oracle_select(u, BS, budget, G)
            PT.check_reps(reps[table[b, :nb], g], u, BS, o_reps)
            sel = PT.gpu_unit_selection(idx, cnt, b, g)
            assert len(sel) == min(k, KMAX)
            PT.check_selection(sel, o_sel, o_scores, k, nb, budget[3], budget[4])
            sel = np.array(sel, dtype=np.int64)
            for o_, l_ in ((out, lse), (out2, lse2)):
                e = PT.check_output(o_[b, :, g * G:(g + 1) * G], l_[b, :, g * G:(g + 1) * G], u,
                                    sel, BS, scale, "bf16")
                for key, val in e.items():
                    worst[key] = max(worst.get(key, 0.0), val)
    PT.record("c consumer layer (bf16, 2 seqs, paged)", units=B * HKV, **worst)

    n, dm, f = m["FN"], m["FDM"], m["FF"]
    x = _bf16(_load(d, "x.bin", np.uint16, (n, dm)))
    wg, wu, wd = (_bf16(_load(d, f"{nm}.bin", np.uint16, (f, dm)))
                  for nm in ("w_gate", "w_up", "w_down_t"))
    y = _bf16(_load(d, "y.bin", np.uint16, (n, dm)))
    bits = _load(d, "keep.bin", np.uint32, (f,)).astype(np.int64)
    PT.check_ffn("c_consumer", x, wg, wu, wd, meta["TAU"], bits, y)
