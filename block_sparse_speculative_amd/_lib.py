"""ctypes binding of libsv.so: argument marshalling only.

Every function takes torch tensors (device memory) plus plain Python values, checks
what is cheap to check on the host (dtype, device, contiguity, shape), and calls the
C entry point of the same name on the current HIP stream. All computation happens
in the library's HIP kernels; there is no fallback. If libsv.so is missing, every
call raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# The in-tree build; SV_LIBRARY names another build of the same sources instead (the
# host-sanitizer build, say).
LIB_PATH = os.environ.get("SV_LIBRARY") or os.path.join(_PKG, "libsv.so")

SV_OK = 0
SV_F32, SV_BF16 = 0, 1

_STATUS = {0: "SV_OK", 1: "SV_ERR_NULL_ARG", 2: "SV_ERR_BAD_SHAPE", 3: "SV_ERR_UNSUPPORTED",
           4: "SV_ERR_WORKSPACE", 5: "SV_ERR_HIP"}


class Shape(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
                ("num_phys_blocks", ctypes.c_int32), ("num_draft", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class Budget(ctypes.Structure):
    _fields_ = [("dense_ctx_tokens", ctypes.c_int32), ("min_blocks", ctypes.c_int32),
                ("frac_per_mille", ctypes.c_int32), ("keep_first", ctypes.c_int32),
                ("keep_last", ctypes.c_int32)]


class AttnPlan(ctypes.Structure):
    _fields_ = [("num_splits", ctypes.c_int32), ("workgroups", ctypes.c_int32),
                ("tile_tokens", ctypes.c_int32), ("padded_rows", ctypes.c_int32),
                ("ring_kb", ctypes.c_int32), ("merge_mode", ctypes.c_int32)]

    def as_dict(self):
        return {name: int(getattr(self, name)) for name, _ in self._fields_}


# sv_merge_mode
MERGE_NONE, MERGE_IN_LAUNCH_WAIT, MERGE_IN_LAUNCH_LAST, MERGE_KERNEL = 0, 1, 2, 3


class FfnShape(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("d_ffn", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class SvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None

# (name, restype, argtypes) of every exported entry point, in header order.
_P = ctypes.c_void_p
_I = ctypes.c_int32
_SIG = [
    ("sv_abi_version", _I, []),
    ("sv_status_str", ctypes.c_char_p, [_I]),
    ("sv_last_error", ctypes.c_char_p, []),
    ("sv_budget_blocks", _I, [ctypes.POINTER(Budget), _I, _I]),
    ("sv_block_repr", _I, [ctypes.POINTER(Shape), _P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P]),
    ("sv_select_workspace_bytes", ctypes.c_size_t, [ctypes.POINTER(Shape), _I]),
    ("sv_select_blocks", _I, [ctypes.POINTER(Shape), ctypes.POINTER(Budget), _P, _P, _P, _P, _I,
                              _P, _P, _P, _P, ctypes.c_size_t, _P]),
    ("sv_attn_num_splits", _I, [ctypes.POINTER(Shape), _I, _I]),
    ("sv_attn_workspace_bytes", ctypes.c_size_t, [ctypes.POINTER(Shape), _I, _I]),
    ("sv_attn_plan_query", _I, [ctypes.POINTER(Shape), _I, _I, ctypes.POINTER(AttnPlan)]),
    ("sv_sparse_verify_attn", _I, [ctypes.POINTER(Shape), _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                   _P, _I, ctypes.c_float, _I, _P, _P, _P, ctypes.c_size_t, _P]),
    ("sv_select_and_attend_workspace_bytes", ctypes.c_size_t, [ctypes.POINTER(Shape), _I, _I]),
    ("sv_select_and_attend", _I, [ctypes.POINTER(Shape), ctypes.POINTER(Budget), _P, _P, _P, _P,
                                  _P, _P, _P, _P, _P, _I, ctypes.c_float, _I, _P, _P, _P, _P, _P,
                                  ctypes.c_size_t, _P]),
    ("sv_select_and_attend_static", _I, [ctypes.POINTER(Shape), ctypes.POINTER(Budget), _P, _P,
                                         _P, _P, _P, _P, _P, _P, _P, _I, ctypes.c_float, _I, _P,
                                         _P, _P, _P, _P]),
    ("sv_sparse_ffn_workspace_bytes", ctypes.c_size_t, [ctypes.POINTER(FfnShape)]),
    ("sv_sparse_ffn", _I, [ctypes.POINTER(FfnShape), _P, _P, _P, _P, ctypes.c_float, _P, _P, _P,
                           ctypes.c_size_t, _P]),
    ("sv_reuse_indices", _I, [ctypes.POINTER(Shape), _I, _P, _P, _P, _P, _P]),
]
EXPORTS = tuple(name for name, _, _ in _SIG)


def lib():
    """Load libsv.so (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} not found: build it with `python -m block_sparse_speculative_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, res, args in _SIG:
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def _check(status: int):
    if status != SV_OK:
        raise SvError(status, lib().sv_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype=None, shape: Optional[Sequence[int]] = None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def make_shape(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
               num_phys_blocks, num_draft, dtype) -> Shape:
    code = {torch.float32: SV_F32, torch.bfloat16: SV_BF16}.get(dtype, dtype)
    return Shape(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                 num_phys_blocks, num_draft, code)


def make_budget(dense_ctx_tokens, min_blocks, frac_per_mille, keep_first=1, keep_last=1) -> Budget:
    return Budget(dense_ctx_tokens, min_blocks, frac_per_mille, int(keep_first), int(keep_last))


def _elem(shape: Shape):
    return torch.float32 if shape.dtype == SV_F32 else torch.bfloat16


def abi_version() -> int:
    return lib().sv_abi_version()


def budget_blocks(budget: Budget, ctx_len: int, block_size: int) -> int:
    return lib().sv_budget_blocks(ctypes.byref(budget), int(ctx_len), int(block_size))


def select_workspace_bytes(shape: Shape, k_max: int) -> int:
    return lib().sv_select_workspace_bytes(ctypes.byref(shape), int(k_max))


def attn_num_splits(shape: Shape, k_max: int, num_splits: int = 0) -> int:
    return lib().sv_attn_num_splits(ctypes.byref(shape), int(k_max), int(num_splits))


def attn_workspace_bytes(shape: Shape, k_max: int, num_splits: int = 0) -> int:
    return lib().sv_attn_workspace_bytes(ctypes.byref(shape), int(k_max), int(num_splits))


def attn_plan(shape: Shape, k_max: int, num_splits: int = 0) -> dict:
    """sv_attn_plan_query: splits, workgroups, tile tokens, padded rows, LDS ring and
    merge mode of the attention launch for these arguments."""
    plan = AttnPlan()
    _check(lib().sv_attn_plan_query(ctypes.byref(shape), int(k_max), int(num_splits),
                                    ctypes.byref(plan)))
    return plan.as_dict()


def block_repr(shape: Shape, k_new, v_new, n_new, ctx_before, block_table, k_pool, v_pool,
               repr_pool, ctx_after=None):
    """sv_block_repr: write k_new/v_new [B, n_new_max, Hkv, D] into the pool at
    ctx_before (an append, or a rewrite of cached tokens when ctx_after [B] gives the
    sequence lengths afterwards) and refresh the representatives of the touched
    blocks."""
    B, Hkv, D = shape.num_seqs, shape.num_kv_heads, shape.head_dim
    e = _elem(shape)
    n_new_max = int(k_new.shape[1])
    _dev(k_new, "k_new", e, (B, n_new_max, Hkv, D))
    _dev(v_new, "v_new", e, (B, n_new_max, Hkv, D))
    _dev(n_new, "n_new", torch.int32, (B,))
    _dev(ctx_before, "ctx_before", torch.int32, (B,))
    _dev(block_table, "block_table", torch.int32, (B, shape.max_blocks_per_seq))
    P, bs = shape.num_phys_blocks, shape.block_size
    _dev(k_pool, "k_pool", e, (P, Hkv, bs, D))
    _dev(v_pool, "v_pool", e, (P, Hkv, bs, D))
    _dev(repr_pool, "repr_pool", torch.float32, (P, Hkv, D))
    if ctx_after is not None:
        _dev(ctx_after, "ctx_after", torch.int32, (B,))
    _check(lib().sv_block_repr(ctypes.byref(shape), _ptr(k_new), _ptr(v_new), n_new_max,
                               _ptr(n_new), _ptr(ctx_before), _ptr(ctx_after), _ptr(block_table),
                               _ptr(k_pool), _ptr(v_pool), _ptr(repr_pool), _stream()))


def select_blocks(shape: Shape, budget: Budget, q, repr_pool, block_table, ctx_lens, k_max: int,
                  idx, cnt, scores=None, ws=None):
    """sv_select_blocks. `ws` is a uint8 device tensor of at least
    select_workspace_bytes() bytes."""
    B, Hq, Hkv, D, T = (shape.num_seqs, shape.num_q_heads, shape.num_kv_heads, shape.head_dim,
                        shape.num_draft)
    _dev(q, "q", _elem(shape), (B, T, Hq, D))
    _dev(repr_pool, "repr_pool", torch.float32, (shape.num_phys_blocks, Hkv, D))
    _dev(block_table, "block_table", torch.int32, (B, shape.max_blocks_per_seq))
    _dev(ctx_lens, "ctx_lens", torch.int32, (B,))
    _dev(idx, "idx", torch.int32, (B, Hkv, k_max))
    _dev(cnt, "cnt", torch.int32, (B, Hkv))
    if scores is not None:
        _dev(scores, "scores", torch.float32, (B, Hkv, shape.max_blocks_per_seq))
    if ws is not None:
        _dev(ws, "ws")
    _check(lib().sv_select_blocks(ctypes.byref(shape), ctypes.byref(budget), _ptr(q),
                                  _ptr(repr_pool), _ptr(block_table), _ptr(ctx_lens), int(k_max),
                                  _ptr(idx), _ptr(cnt), _ptr(scores), _ptr(ws),
                                  0 if ws is None else ws.numel() * ws.element_size(), _stream()))


def sparse_verify_attn(shape: Shape, q, k_draft, v_draft, k_pool, v_pool, block_table, ctx_lens,
                       idx, cnt, k_max: int, scale: float, out, lse=None, ws=None,
                       num_splits: int = 0, draft_mask=None):
    """sv_sparse_verify_attn (draft_mask: None for chain drafts, else [B, T] int32
    visibility bits among the drafts)."""
    B, Hq, Hkv, D, T = (shape.num_seqs, shape.num_q_heads, shape.num_kv_heads, shape.head_dim,
                        shape.num_draft)
    e = _elem(shape)
    P, bs = shape.num_phys_blocks, shape.block_size
    _dev(q, "q", e, (B, T, Hq, D))
    _dev(k_draft, "k_draft", e, (B, T, Hkv, D))
    _dev(v_draft, "v_draft", e, (B, T, Hkv, D))
    _dev(k_pool, "k_pool", e, (P, Hkv, bs, D))
    _dev(v_pool, "v_pool", e, (P, Hkv, bs, D))
    _dev(block_table, "block_table", torch.int32, (B, shape.max_blocks_per_seq))
    _dev(ctx_lens, "ctx_lens", torch.int32, (B,))
    _dev(idx, "idx", torch.int32, (B, Hkv, k_max))
    _dev(cnt, "cnt", torch.int32, (B, Hkv))
    _dev(out, "out", e, (B, T, Hq, D))
    if lse is not None:
        _dev(lse, "lse", torch.float32, (B, T, Hq))
    if ws is not None:
        _dev(ws, "ws")
    if draft_mask is not None:
        _dev(draft_mask, "draft_mask", torch.int32, (B, T))
    _check(lib().sv_sparse_verify_attn(
        ctypes.byref(shape), _ptr(q), _ptr(k_draft), _ptr(v_draft), _ptr(draft_mask),
        _ptr(k_pool), _ptr(v_pool),
        _ptr(block_table), _ptr(ctx_lens), _ptr(idx), _ptr(cnt), int(k_max), float(scale),
        int(num_splits), _ptr(out), _ptr(lse), _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size(), _stream()))


def select_and_attend_workspace_bytes(shape: Shape, k_max: int, num_splits: int = 0) -> int:
    return lib().sv_select_and_attend_workspace_bytes(ctypes.byref(shape), int(k_max),
                                                      int(num_splits))


def select_and_attend(shape: Shape, budget: Budget, q, repr_pool, k_draft, v_draft, k_pool, v_pool,
                      block_table, ctx_lens, k_max: int, scale: float, idx, cnt, out, lse=None,
                      ws=None, num_splits: int = 0, draft_mask=None):
    """sv_select_and_attend: selection and attention of one layer; writes idx / cnt."""
    B, Hq, Hkv, D, T = (shape.num_seqs, shape.num_q_heads, shape.num_kv_heads, shape.head_dim,
                        shape.num_draft)
    e = _elem(shape)
    P, bs = shape.num_phys_blocks, shape.block_size
    _dev(q, "q", e, (B, T, Hq, D))
    _dev(repr_pool, "repr_pool", torch.float32, (P, Hkv, D))
    _dev(k_draft, "k_draft", e, (B, T, Hkv, D))
    _dev(v_draft, "v_draft", e, (B, T, Hkv, D))
    _dev(k_pool, "k_pool", e, (P, Hkv, bs, D))
    _dev(v_pool, "v_pool", e, (P, Hkv, bs, D))
    _dev(block_table, "block_table", torch.int32, (B, shape.max_blocks_per_seq))
    _dev(ctx_lens, "ctx_lens", torch.int32, (B,))
    _dev(idx, "idx", torch.int32, (B, Hkv, k_max))
    _dev(cnt, "cnt", torch.int32, (B, Hkv))
    _dev(out, "out", e, (B, T, Hq, D))
    if lse is not None:
        _dev(lse, "lse", torch.float32, (B, T, Hq))
    if ws is not None:
        _dev(ws, "ws")
    if draft_mask is not None:
        _dev(draft_mask, "draft_mask", torch.int32, (B, T))
    _check(lib().sv_select_and_attend(
        ctypes.byref(shape), ctypes.byref(budget), _ptr(q), _ptr(repr_pool), _ptr(k_draft),
        _ptr(v_draft), _ptr(draft_mask), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(ctx_lens), int(k_max),
        float(scale), int(num_splits), _ptr(idx), _ptr(cnt), _ptr(out), _ptr(lse), _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size(), _stream()))


STATIC_SCRATCH_BYTES = 32 << 20     # SV_STATIC_SCRATCH_BYTES
STATIC_SCRATCH_UNITS = 2048         # SV_STATIC_SCRATCH_UNITS


def select_and_attend_static(shape: Shape, budget: Budget, q, repr_pool, k_draft, v_draft,
                             k_pool, v_pool, block_table, ctx_lens, k_max: int, scale: float,
                             idx, cnt, out, lse=None, num_splits: int = 0, draft_mask=None):
    """sv_select_and_attend_static: sv_select_and_attend without a workspace (the library's
    static per-device scratch; allocates nothing)."""
    B, Hq, Hkv, D, T = (shape.num_seqs, shape.num_q_heads, shape.num_kv_heads, shape.head_dim,
                        shape.num_draft)
    e = _elem(shape)
    P, bs = shape.num_phys_blocks, shape.block_size
    _dev(q, "q", e, (B, T, Hq, D))
    _dev(repr_pool, "repr_pool", torch.float32, (P, Hkv, D))
    _dev(k_draft, "k_draft", e, (B, T, Hkv, D))
    _dev(v_draft, "v_draft", e, (B, T, Hkv, D))
    _dev(k_pool, "k_pool", e, (P, Hkv, bs, D))
    _dev(v_pool, "v_pool", e, (P, Hkv, bs, D))
    _dev(block_table, "block_table", torch.int32, (B, shape.max_blocks_per_seq))
    _dev(ctx_lens, "ctx_lens", torch.int32, (B,))
    _dev(idx, "idx", torch.int32, (B, Hkv, k_max))
    _dev(cnt, "cnt", torch.int32, (B, Hkv))
    _dev(out, "out", e, (B, T, Hq, D))
    if lse is not None:
        _dev(lse, "lse", torch.float32, (B, T, Hq))
    if draft_mask is not None:
        _dev(draft_mask, "draft_mask", torch.int32, (B, T))
    _check(lib().sv_select_and_attend_static(
        ctypes.byref(shape), ctypes.byref(budget), _ptr(q), _ptr(repr_pool), _ptr(k_draft),
        _ptr(v_draft), _ptr(draft_mask), _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
        _ptr(ctx_lens), int(k_max), float(scale), int(num_splits), _ptr(idx), _ptr(cnt),
        _ptr(out), _ptr(lse), _stream()))


def make_ffn_shape(num_tokens, d_model, d_ffn, dtype=torch.bfloat16) -> FfnShape:
    code = {torch.float32: SV_F32, torch.bfloat16: SV_BF16}.get(dtype, dtype)
    return FfnShape(num_tokens, d_model, d_ffn, code)


def sparse_ffn_workspace_bytes(shape: FfnShape) -> int:
    return lib().sv_sparse_ffn_workspace_bytes(ctypes.byref(shape))


def sparse_ffn(shape: FfnShape, x, w_gate, w_up, w_down_t, tau: float, y, keep_bits=None,
               ws=None):
    """sv_sparse_ffn: the threshold-pruned gated FFN (x [N, Dm]; w_gate, w_up, w_down_t
    [F, Dm]; y [N, Dm]; keep_bits [F] int32 viewed as uint32 bits, optional)."""
    N, Dm, F = shape.num_tokens, shape.d_model, shape.d_ffn
    _dev(x, "x", torch.bfloat16, (N, Dm))
    for name, t in (("w_gate", w_gate), ("w_up", w_up), ("w_down_t", w_down_t)):
        _dev(t, name, torch.bfloat16, (F, Dm))
    _dev(y, "y", torch.bfloat16, (N, Dm))
    if keep_bits is not None:
        _dev(keep_bits, "keep_bits", torch.int32, (F,))
    if ws is not None:
        _dev(ws, "ws")
    _check(lib().sv_sparse_ffn(ctypes.byref(shape), _ptr(x), _ptr(w_gate), _ptr(w_up),
                               _ptr(w_down_t), float(tau), _ptr(y), _ptr(keep_bits), _ptr(ws),
                               0 if ws is None else ws.numel() * ws.element_size(), _stream()))


def reuse_indices(shape: Shape, k_max: int, prev_idx, prev_cnt, idx, cnt):
    """sv_reuse_indices."""
    B, Hkv = shape.num_seqs, shape.num_kv_heads
    for name, t, shp in (("prev_idx", prev_idx, (B, Hkv, k_max)), ("prev_cnt", prev_cnt, (B, Hkv)),
                         ("idx", idx, (B, Hkv, k_max)), ("cnt", cnt, (B, Hkv))):
        _dev(t, name, torch.int32, shp)
    _check(lib().sv_reuse_indices(ctypes.byref(shape), int(k_max), _ptr(prev_idx),
                                  _ptr(prev_cnt), _ptr(idx), _ptr(cnt), _stream()))
