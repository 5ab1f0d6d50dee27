"""C-ABI library tests that need no GPU: the library loads, exports every symbol the
header declares, and rejects invalid host-visible arguments before launching.

Calls here that pass fake (non-null, never dereferenced) pointers always fail host
validation first, so nothing reaches the GPU.
"""

import ctypes
import os
import re

import pytest

import block_sparse_speculative_amd as sv
from block_sparse_speculative_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sv.h")

pytestmark = pytest.mark.skipif(not os.path.exists(L.LIB_PATH),
                                reason="libsv.so not built (run __graft_entry__.build())")

FAKE = ctypes.c_void_p(0x1000)


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sv_[a-z_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert header_functions() == sorted(sv.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = sv.lib()
    for name in header_functions():
        assert hasattr(lib, name), name
    assert sv.abi_version() == 3


def test_status_strings():
    lib = sv.lib()
    assert lib.sv_status_str(0) == b"SV_OK"
    assert lib.sv_status_str(4) == b"SV_ERR_WORKSPACE"
    assert lib.sv_status_str(99) == b"SV_ERR_UNKNOWN"


def _golden_budget_rows():
    rows = []
    with open(os.path.join(ROOT, "tests", "golden", "budget_table.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                rows.append(tuple(int(x) for x in line.split()))
    return rows


@pytest.mark.parametrize("row", _golden_budget_rows())
def test_host_budget_matches_hand_derived_table(row):
    ctx, bs, dense, mn, frac, expected = row
    assert sv.budget_blocks(sv.make_budget(dense, mn, frac), ctx, bs) == expected


def test_budget_rejects_invalid():
    assert sv.budget_blocks(sv.make_budget(0, 1, 0, 1, 1), 100, 64) == -1      # min < forced
    assert sv.budget_blocks(sv.make_budget(0, 4, 1001), 100, 64) == -1
    assert sv.budget_blocks(sv.make_budget(0, 4, 10), -1, 64) == -1
    assert sv.budget_blocks(sv.make_budget(0, 4, 10), 10, 0) == -1


def _shape(**kw):
    base = dict(num_seqs=2, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=64,
                max_blocks_per_seq=1024, num_phys_blocks=2048, num_draft=8, dtype=sv.SV_BF16)
    base.update(kw)
    return L.Shape(**base)


def _attn(shape, k_max=64, ws=None, ws_bytes=0, out=FAKE, scale=0.1, splits=0):
    lib = sv.lib()
    return lib.sv_sparse_verify_attn(ctypes.byref(shape), FAKE, FAKE, FAKE, None, FAKE, FAKE,
                                     FAKE, FAKE, FAKE, FAKE, k_max, scale, splits, out, None, ws,
                                     ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), 3), (dict(block_size=16), 3), (dict(num_q_heads=30), 2),
    (dict(num_draft=17), 3), (dict(num_draft=0), 2), (dict(dtype=7), 3),
    (dict(num_q_heads=64, num_kv_heads=4, num_draft=16), 3),   # T*G = 256 > 128
    (dict(max_blocks_per_seq=20000), 3), (dict(num_phys_blocks=0), 2), (dict(num_seqs=-1), 2),
])
def test_attention_rejects_shapes_before_launch(kw, status):
    assert _attn(_shape(**kw)) == status
    assert sv.lib().sv_last_error() != b""


def test_attention_rejects_workspace_null_args_and_kmax():
    shape = _shape()
    need = sv.attn_workspace_bytes(shape, 64)
    assert need > 0 and sv.attn_num_splits(shape, 64) > 1
    assert _attn(shape, ws=None, ws_bytes=0) == 4
    assert _attn(shape, ws=FAKE, ws_bytes=need - 1) == 4
    assert _attn(shape, out=None, ws=FAKE, ws_bytes=need) == 1
    assert _attn(shape, k_max=0) == 2
    assert _attn(shape, k_max=2000) == 2
    assert _attn(shape, scale=float("nan")) == 2
    assert _attn(shape, scale=0.0) == 2
    assert _attn(shape, scale=-0.5) == 2
    assert _attn(shape, splits=-3) == 2


def test_split_count_and_workspace_size():
    shape = _shape(num_seqs=1)
    assert sv.attn_num_splits(shape, 64, 1) == 1
    assert sv.attn_workspace_bytes(shape, 64, 1) == 0
    assert sv.attn_num_splits(shape, 64, 10_000) == 64          # clamped to the context tiles
    s4 = sv.attn_num_splits(shape, 64, 4)
    rows, d, units = 8 * 4, 128, 8
    assert s4 == 4
    assert sv.attn_workspace_bytes(shape, 64, 4) >= units * 4 * rows * (d + 2) * 4
    # bs 128 uses two 64-token tiles per block at up to 64 rows per unit, one
    # 128-token tile per block above that
    assert sv.attn_num_splits(_shape(num_seqs=1, block_size=128), 64, 10_000) == 128
    assert sv.attn_num_splits(_shape(num_seqs=1, block_size=128, num_draft=16,
                                     num_q_heads=64), 64, 10_000) == 64
    assert sv.attn_num_splits(_shape(num_seqs=1, block_size=128, num_draft=16,
                                     num_q_heads=64, dtype=sv.SV_F32), 64, 10_000) == 256


def test_select_rejects_bad_budget_and_workspace():
    lib = sv.lib()
    shape = _shape()

    def call(budget, ws=FAKE, ws_bytes=1 << 30, k_max=64, q=FAKE):
        return lib.sv_select_blocks(ctypes.byref(shape), budget, q, FAKE, FAKE, FAKE, k_max, FAKE,
                                    FAKE, None, ws, ws_bytes, None)

    good = ctypes.byref(sv.make_budget(4096, 64, 50))
    assert call(None) == 1
    assert call(ctypes.byref(sv.make_budget(4096, 1, 50, 1, 1))) == 2
    assert call(ctypes.byref(sv.make_budget(4096, 64, 2000))) == 2
    assert call(ctypes.byref(sv.make_budget(-1, 64, 50))) == 2
    assert call(good, ws=None, ws_bytes=0) == 4
    need = sv.select_workspace_bytes(shape, 64)
    assert need >= 2 * 8 * 1024 * 4
    assert call(good, ws_bytes=need - 1) == 4
    assert call(good, q=None) == 1
    assert call(good, k_max=0) == 2
    # k_max caps the budget but must hold the forced blocks
    assert call(good, k_max=1) == 2 and b"forced" in lib.sv_last_error()
    assert call(ctypes.byref(sv.make_budget(4096, 64, 50, 1, 0)), k_max=1, ws_bytes=0) == 4
    assert call(ctypes.byref(sv.make_budget(4096, 64, 50, 0, 0)), k_max=1, ws_bytes=0) == 4


def test_repr_and_reuse_reject_before_launch():
    lib = sv.lib()
    shape = _shape()
    assert lib.sv_block_repr(ctypes.byref(shape), None, FAKE, 4, FAKE, FAKE, None, FAKE, FAKE,
                             FAKE, FAKE, None) == 1
    assert lib.sv_block_repr(ctypes.byref(shape), FAKE, FAKE, -1, FAKE, FAKE, None, FAKE, FAKE,
                             FAKE, FAKE, None) == 2
    assert lib.sv_block_repr(ctypes.byref(_shape(head_dim=32)), FAKE, FAKE, 4, FAKE, FAKE, FAKE,
                             FAKE, FAKE, FAKE, FAKE, None) == 3
    assert lib.sv_reuse_indices(ctypes.byref(shape), 64, None, FAKE, FAKE, FAKE, None) == 1
    # overlapping source and destination
    assert lib.sv_reuse_indices(ctypes.byref(shape), 64, FAKE, ctypes.c_void_p(0x900000), FAKE,
                                ctypes.c_void_p(0xA00000), None) == 2


def test_binding_refuses_host_tensors():
    import torch
    shape = _shape(num_seqs=1)
    t = torch.zeros(1, 8, 8, 64, dtype=torch.int32)
    with pytest.raises(ValueError):
        sv.reuse_indices(shape, 64, t, t, t, t)


def test_select_and_attend_rejects_before_launch():
    lib = sv.lib()
    shape = _shape()
    good = ctypes.byref(sv.make_budget(4096, 64, 50))
    need = sv.select_and_attend_workspace_bytes(shape, 64)
    # the score scratch follows the attention workspace
    assert need >= sv.attn_workspace_bytes(shape, 64) + 2 * 8 * 1024 * 4

    def call(budget=good, ws=FAKE, ws_bytes=need, k_max=64, scale=0.1, q=FAKE, splits=0):
        return lib.sv_select_and_attend(ctypes.byref(shape), budget, q, FAKE, FAKE, FAKE, None,
                                        FAKE, FAKE, FAKE, FAKE, k_max, scale, splits, FAKE, FAKE,
                                        FAKE, None, ws, ws_bytes, None)

    assert call(budget=None) == 1
    assert call(budget=ctypes.byref(sv.make_budget(4096, 1, 50, 1, 1))) == 2
    assert call(ws=None, ws_bytes=0) == 4
    assert call(ws_bytes=need - 1) == 4
    assert call(q=None) == 1
    assert call(k_max=0) == 2
    assert call(k_max=1) == 2 and b"forced" in lib.sv_last_error()
    assert call(budget=ctypes.byref(sv.make_budget(4096, 64, 50, 1, 0)), k_max=1,
                ws_bytes=0) == 4
    assert call(scale=0.0) == 2
    assert call(splits=-1) == 2
    assert lib.sv_select_and_attend(ctypes.byref(_shape(head_dim=96)), good, FAKE, FAKE, FAKE,
                                    FAKE, None, FAKE, FAKE, FAKE, FAKE, 64, 0.1, 0, FAKE, FAKE,
                                    FAKE, None, FAKE, need, None) == 3


def test_split_ranges_balanced_over_k_max():
    # the tile slots of a unit are cut into balanced ranges: no split is left empty
    shape = _shape(num_seqs=1)
    for k_max in (64, 100, 1000):
        for s in (3, 7, 10, 15):
            assert sv.attn_num_splits(shape, k_max, s) == min(s, k_max)


# ------------------------------------------------------------------ launch plans

def test_plan_query_reports_the_launch():
    # stack64k shape: 4 x 8 units, 11 splits (short streams of 5-6 tiles: three
    # workgroups for every two CUs), 64-token tiles, 32 rows, two workgroups per CU
    # (64 KB ring), the bounded-wait merge in the launch
    p = sv.attn_plan(_shape(num_seqs=4), 64, 0)
    assert p == dict(num_splits=11, workgroups=12 * 32, tile_tokens=64, padded_rows=32,
                     ring_kb=64, merge_mode=L.MERGE_IN_LAUNCH_WAIT)
    # 128 units (the ragged batch): 2 splits would stream 32 tiles each, so 3 splits
    # and two workgroups per CU (512)
    r = sv.attn_plan(_shape(num_seqs=16), 64, 0)
    assert (r["num_splits"], r["workgroups"], r["ring_kb"]) == (3, 512, 64)
    # the threshold: 2 splits until each would stream 16 tiles (k_max 32 of 64-token
    # tiles at block size 64), then 3
    assert sv.attn_num_splits(_shape(num_seqs=16), 31, 0) == 2
    assert sv.attn_num_splits(_shape(num_seqs=16), 32, 0) == 3
    # 12 units with long streams: two per CU would be 41 splits, past the 32 workgroups
    # per unit the launch merges in place; capped at 31 instead
    t = sv.attn_plan(_shape(num_seqs=3, num_kv_heads=4, num_q_heads=16), 1024, 0)
    assert t["num_splits"] == 31 and t["merge_mode"] != L.MERGE_KERNEL
    # qwen128k shape: 2 x 4 units of 128 rows, 128-token tiles, one workgroup per CU
    q = sv.attn_plan(_shape(num_seqs=2, num_kv_heads=4, num_draft=16, block_size=128), 128, 0)
    assert (q["tile_tokens"], q["padded_rows"], q["ring_kb"]) == (128, 128, 128)
    assert q["workgroups"] == (q["num_splits"] + 1) * 8 <= 256
    assert q["merge_mode"] == L.MERGE_IN_LAUNCH_WAIT
    # one split: no merge; a grid beyond the device: the last arriver merges; more than
    # 32 workgroups per unit: the merge kernel
    assert sv.attn_plan(_shape(num_seqs=4), 64, 1)["merge_mode"] == L.MERGE_NONE
    big = sv.attn_plan(_shape(num_seqs=8), 64, 16)
    assert big["workgroups"] == 17 * 64 > 512 and big["merge_mode"] == L.MERGE_IN_LAUNCH_LAST
    assert sv.attn_plan(_shape(num_seqs=1), 64, 40)["merge_mode"] == L.MERGE_KERNEL


def test_plan_query_rejects_bad_arguments():
    lib = sv.lib()
    plan = L.AttnPlan()
    assert lib.sv_attn_plan_query(ctypes.byref(_shape()), 64, 0, None) == 1
    assert lib.sv_attn_plan_query(ctypes.byref(_shape()), 0, 0, ctypes.byref(plan)) == 2
    assert lib.sv_attn_plan_query(ctypes.byref(_shape(head_dim=96)), 64, 0,
                                  ctypes.byref(plan)) == 3
    assert lib.sv_attn_plan_query(ctypes.byref(_shape()), 64, -1, ctypes.byref(plan)) == 2


def _reachable_builds():
    """Every (dtype, D, tile tokens, padded rows, ring KB) the plan query can return,
    swept over the supported envelope."""
    out = set()
    rows_gt = [(1, 1), (2, 8), (4, 4), (4, 8), (8, 8), (8, 16), (3, 5), (6, 10)]
    for dtype, dname in ((sv.SV_F32, "fp32"), (sv.SV_BF16, "bf16")):
        for d in (64, 128):
            for bs in (32, 64, 128):
                for g, t in rows_gt:
                    for b, hkv in ((1, 1), (1, 8), (2, 8), (4, 8), (16, 8)):
                        for k_max in (1, 8, 64, 512):
                            shape = _shape(num_seqs=b, num_kv_heads=hkv, num_q_heads=hkv * g,
                                           num_draft=t, head_dim=d, block_size=bs, dtype=dtype,
                                           max_blocks_per_seq=1024)
                            for splits in (0, 1, 2, 7, 20, 31, 1000):
                                p = sv.attn_plan(shape, k_max, splits)
                                out.add((dname, d, p["tile_tokens"], p["padded_rows"],
                                         p["ring_kb"]))
    return out


def test_parity_matrix_launches_every_build():
    # The GPU parity matrix (tests/cases.py) must launch every attention build the
    # library can pick, through the separate calls and through the fused entry point.
    import cases as C
    universe = _reachable_builds()
    assert len(universe) >= 30
    covered = {C.build_key(w, splits, fused) for _, w, splits, fused in C.matrix_cases()}
    missing = [(b, f) for b in sorted(universe) for f in (False, True) if b + (f,) not in covered]
    assert not missing, f"builds no parity test launches: {missing}"


def test_static_entry_point_rejects_what_its_scratch_cannot_hold():
    # validated on the host before anything touches a device
    lib = sv.lib()
    good = ctypes.byref(sv.make_budget(4096, 64, 50))

    def call(shape, k_max=64, splits=0):
        return lib.sv_select_and_attend_static(ctypes.byref(shape), good, FAKE, FAKE, FAKE, FAKE,
                                               None, FAKE, FAKE, FAKE, FAKE, k_max, 0.1, splits,
                                               FAKE, FAKE, FAKE, None, None)

    assert call(_shape(num_seqs=257)) == 4                     # 2056 units > 2048
    assert b"units" in lib.sv_last_error()
    # 128 units x 32 workgroups x 128 rows x 128 dims of fp32 partials: 64 MiB > 32 MiB
    assert call(_shape(num_seqs=32, num_kv_heads=4, num_q_heads=32, num_draft=16),
                k_max=256, splits=31) == 4
    assert b"bytes" in lib.sv_last_error()
    assert call(_shape(head_dim=96)) == 3
    assert call(_shape(), k_max=0) == 2


def _ffn_shape(n=8, dm=4096, f=14336, dtype=None):
    s = L.make_ffn_shape(n, dm, f)
    if dtype is not None:
        s.dtype = dtype
    return s


@pytest.mark.parametrize("kw,status", [
    (dict(n=17), 3), (dict(n=-1), 2), (dict(dm=0), 2), (dict(f=0), 2), (dict(dm=1000), 3),
    (dict(n=16, dm=8192), 3),                 # 16 padded tokens x 8192 dims: 256 KB of x
    (dict(dtype=0), 3),                       # fp32 is not supported
    (dict(dm=8192, f=131072), 3),             # a 2 GiB weight matrix
])
def test_sparse_ffn_rejects_shapes_before_launch(kw, status):
    lib = sv.lib()
    shape = _ffn_shape(**kw)
    assert lib.sv_sparse_ffn_workspace_bytes(ctypes.byref(shape)) == 0
    st = lib.sv_sparse_ffn(ctypes.byref(shape), FAKE, FAKE, FAKE, FAKE, 0.3, FAKE, None, FAKE,
                           1 << 40, None)
    assert st == status
    assert lib.sv_last_error() != b""


def test_sparse_ffn_rejects_tau_null_args_and_workspace():
    lib = sv.lib()
    shape = _ffn_shape()
    need = lib.sv_sparse_ffn_workspace_bytes(ctypes.byref(shape))
    # mask [F] u32, h [F, 16] f32 and the range partials [32 ranges of 448, 8, Dm] f32
    assert need >= 14336 * 4 + 14336 * 16 * 4 + 32 * 8 * 4096 * 4
    call = lambda tau=0.3, x=FAKE, y=FAKE, ws=FAKE, nbytes=need: lib.sv_sparse_ffn(
        ctypes.byref(shape), x, FAKE, FAKE, FAKE, tau, y, None, ws, nbytes, None)
    for tau in (-1.0, float("nan"), float("inf")):
        assert call(tau=tau) == 2
    assert call(x=None) == 1 and call(y=None) == 1
    assert call(ws=None) == 4 and call(nbytes=need - 1) == 4
    # no tokens: nothing to do, nothing read (null pointers accepted)
    empty = _ffn_shape(n=0)
    assert lib.sv_sparse_ffn(ctypes.byref(empty), None, None, None, None, 0.3, None, None,
                             None, 0, None) == 0


# Pointer arguments of each entry point, in call order, with the alignment the kernels need
# (16: vector/LDS-DMA data arrays and workspaces, 4: int32 and scalar-float arrays), and a
# call builder taking those pointers by name. Every pointer is distinct and 16-byte aligned,
# so with one of them misaligned, alignment is the only check that can fail before the
# workspace size (given as large enough). Nothing is launched: every call below fails.
_A16, _A4 = 16, 4


def _ptrs(names):
    return {n: 0x10000000 * (i + 1) for i, n in enumerate(names)}


def _entry_calls():
    lib = sv.lib()
    shape = _shape()
    budget = ctypes.byref(sv.make_budget(4096, 64, 50))
    fshape = _ffn_shape()
    P = ctypes.c_void_p
    big = 1 << 40
    return {
        "sv_sparse_verify_attn": (
            dict(q=_A16, k_draft=_A16, v_draft=_A16, draft_mask=_A4, k_pool=_A16, v_pool=_A16,
                 block_table=_A4, ctx_lens=_A4, idx=_A4, cnt=_A4, out=_A16, lse=_A4, ws=_A16),
            lambda a: lib.sv_sparse_verify_attn(
                ctypes.byref(shape), P(a["q"]), P(a["k_draft"]), P(a["v_draft"]),
                P(a["draft_mask"]), P(a["k_pool"]), P(a["v_pool"]), P(a["block_table"]),
                P(a["ctx_lens"]), P(a["idx"]), P(a["cnt"]), 64, 0.1, 0, P(a["out"]), P(a["lse"]),
                P(a["ws"]), 1 << 30, None)),
        "sv_select_blocks": (
            dict(q=_A16, repr_pool=_A16, block_table=_A4, ctx_lens=_A4, idx=_A4, cnt=_A4,
                 scores=_A4, ws=_A16),
            lambda a: lib.sv_select_blocks(
                ctypes.byref(shape), budget, P(a["q"]), P(a["repr_pool"]), P(a["block_table"]),
                P(a["ctx_lens"]), 64, P(a["idx"]), P(a["cnt"]), P(a["scores"]), P(a["ws"]),
                1 << 30, None)),
        "sv_select_and_attend": (
            dict(q=_A16, repr_pool=_A16, k_draft=_A16, v_draft=_A16, draft_mask=_A4,
                 k_pool=_A16, v_pool=_A16, block_table=_A4, ctx_lens=_A4, idx=_A4, cnt=_A4,
                 out=_A16, lse=_A4, ws=_A16),
            lambda a: lib.sv_select_and_attend(
                ctypes.byref(shape), budget, P(a["q"]), P(a["repr_pool"]), P(a["k_draft"]),
                P(a["v_draft"]), P(a["draft_mask"]), P(a["k_pool"]), P(a["v_pool"]),
                P(a["block_table"]), P(a["ctx_lens"]), 64, 0.1, 0, P(a["idx"]), P(a["cnt"]),
                P(a["out"]), P(a["lse"]), P(a["ws"]), 1 << 30, None)),
        "sv_select_and_attend_static": (
            dict(q=_A16, repr_pool=_A16, k_draft=_A16, v_draft=_A16, draft_mask=_A4,
                 k_pool=_A16, v_pool=_A16, block_table=_A4, ctx_lens=_A4, idx=_A4, cnt=_A4,
                 out=_A16, lse=_A4),
            lambda a: lib.sv_select_and_attend_static(
                ctypes.byref(shape), budget, P(a["q"]), P(a["repr_pool"]), P(a["k_draft"]),
                P(a["v_draft"]), P(a["draft_mask"]), P(a["k_pool"]), P(a["v_pool"]),
                P(a["block_table"]), P(a["ctx_lens"]), 64, 0.1, 0, P(a["idx"]), P(a["cnt"]),
                P(a["out"]), P(a["lse"]), None)),
        "sv_block_repr": (
            dict(k_new=_A16, v_new=_A16, n_new=_A4, ctx_before=_A4, ctx_after=_A4,
                 block_table=_A4, k_pool=_A16, v_pool=_A16, repr_pool=_A16),
            lambda a: lib.sv_block_repr(
                ctypes.byref(shape), P(a["k_new"]), P(a["v_new"]), 8, P(a["n_new"]),
                P(a["ctx_before"]), P(a["ctx_after"]), P(a["block_table"]), P(a["k_pool"]),
                P(a["v_pool"]), P(a["repr_pool"]), None)),
        "sv_reuse_indices": (
            dict(prev_idx=_A4, prev_cnt=_A4, idx=_A4, cnt=_A4),
            lambda a: lib.sv_reuse_indices(ctypes.byref(shape), 64, P(a["prev_idx"]),
                                           P(a["prev_cnt"]), P(a["idx"]), P(a["cnt"]), None)),
        "sv_sparse_ffn": (
            dict(x=_A16, w_gate=_A16, w_up=_A16, w_down_t=_A16, y=_A16, keep_bits=_A4, ws=_A16),
            lambda a: lib.sv_sparse_ffn(
                ctypes.byref(fshape), P(a["x"]), P(a["w_gate"]), P(a["w_up"]), P(a["w_down_t"]),
                0.3, P(a["y"]), P(a["keep_bits"]), P(a["ws"]), big, None)),
    }


@pytest.mark.parametrize("entry", ["sv_sparse_verify_attn", "sv_select_blocks",
                                   "sv_select_and_attend", "sv_select_and_attend_static",
                                   "sv_block_repr", "sv_reuse_indices", "sv_sparse_ffn"])
def test_every_misaligned_pointer_is_rejected_by_name(entry):
    lib = sv.lib()
    align, call = _entry_calls()[entry]
    # every pointer in the header's declaration is covered
    decl = re.search(entry + r"\s*\(([^)]*)\)", re.sub(r"/\*.*?\*/", "", open(HEADER).read(),
                                                       flags=re.S)).group(1)
    ptr_args = {m.group(1) for m in re.finditer(r"\*\s*(\w+)", decl)}
    ptr_args -= {"shape", "budget", "stream"}
    assert ptr_args == set(align), sorted(ptr_args ^ set(align))
    for name, need in align.items():
        for off in sorted({need // 2, need - 4, 2} - {0}):
            if off % need == 0:
                continue
            a = _ptrs(align)
            a[name] += off
            assert call(a) == 3, (entry, name, off)
            msg = lib.sv_last_error().decode()
            assert f"{name} is not {need}-byte aligned" in msg, msg


def test_sixteen_byte_alignment_is_enough():
    # a pointer 16 bytes past a 256-byte boundary passes the alignment check and the call
    # goes on to the next one (here: a workspace one byte short), launching nothing
    lib = sv.lib()
    shape = _shape()
    need = sv.select_workspace_bytes(shape, 64)
    P = ctypes.c_void_p
    st = lib.sv_select_blocks(ctypes.byref(shape), ctypes.byref(sv.make_budget(4096, 64, 50)),
                              P(0x10000010), P(0x20000010), P(0x30000004), P(0x40000004), 64,
                              P(0x50000004), P(0x60000004), P(0x70000004), P(0x80000010),
                              need - 1, None)
    assert st == 4 and b"workspace" in lib.sv_last_error()


def test_last_error_is_per_thread():
    # the error message is thread-local: threads rejecting different arguments at the
    # same time each read back the message of their own last call (ctypes drops the
    # interpreter lock around foreign calls, so the calls overlap)
    import threading
    lib = sv.lib()
    align, call = _entry_calls()["sv_sparse_verify_attn"]
    names = sorted(align)
    start = threading.Barrier(16)
    bad = []

    def worker(t):
        name = names[t % len(names)]
        a = _ptrs(align)
        a[name] += 2
        start.wait()
        for _ in range(300):
            st = call(a)
            msg = lib.sv_last_error().decode()
            if st != 3 or f"{name} is not" not in msg:
                bad.append((t, name, st, msg))
                return

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(16)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not bad, bad[:3]
