"""ctypes binding of libsparstar (include/sparstar.h).

Argument marshalling only: shapes and strides are read from torch tensors,
outputs are allocated with torch on the inputs' device when not given, and
the current HIP stream is passed through.  Every step of the method runs in
the library's kernels.  If the library has not been built, the first call
raises :class:`SparstarError`; nothing falls back to another implementation.
"""

from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional, Tuple

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsparstar.so")

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_LAYOUT, ERR_DENSITY, ERR_CAPACITY, ERR_HIP = range(8)
KERNEL_MFMA_BF16, KERNEL_F32 = 0, 1
BF16, F32 = 0, 1
POLICY_LATER_CLIP, POLICY_FIRST_CLIP = 0, 1

_c_i32, _c_i64, _c_f32, _c_dbl, _c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double, ctypes.c_void_p


class Problem(ctypes.Structure):
    """Mirror of sparstar_problem."""

    _fields_ = [
        ("batch", _c_i32), ("heads", _c_i32), ("head_dim", _c_i32), ("block", _c_i32),
        ("len_q", _c_i64), ("len_text", _c_i64), ("len_ref", _c_i64),
        ("dtype", _c_i32), ("out_dtype", _c_i32), ("softmax_scale", _c_f32), ("reserved", _c_i32),
        ("q_stride", _c_i64 * 3), ("k_stride", _c_i64 * 3), ("v_stride", _c_i64 * 3),
        ("o_stride", _c_i64 * 3),
    ]


class SparstarError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"libsparstar status {status}: {detail}")


_lib = None

# name -> (restype, argtypes)
_SIGS = {
    "sparstar_check_problem": (_c_i32, [ctypes.POINTER(Problem)]),
    "sparstar_num_q_blocks": (_c_i64, [ctypes.POINTER(Problem)]),
    "sparstar_num_k_blocks": (_c_i64, [ctypes.POINTER(Problem)]),
    "sparstar_num_retained": (_c_i64, [ctypes.POINTER(Problem), _c_i32]),
    "sparstar_budget": (_c_i64, [_c_i64, _c_dbl]),
    "sparstar_blocks_per_row": (_c_i64, [ctypes.POINTER(Problem), _c_dbl, _c_i32]),
    "sparstar_select_nnz": (_c_i64, [ctypes.POINTER(Problem), _c_dbl, _c_i32]),
    "sparstar_status_string": (ctypes.c_char_p, [_c_i32]),
    "sparstar_last_error": (ctypes.c_char_p, []),
    "sparstar_pool_score": (_c_i32, [ctypes.POINTER(Problem), _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp]),
    "sparstar_select_blocks": (_c_i32, [ctypes.POINTER(Problem), _c_vp, _c_dbl, _c_i32, _c_vp, _c_vp,
                                        _c_i64, _c_vp]),
    "sparstar_pool_blocks": (_c_i32, [ctypes.POINTER(Problem), _c_vp, _c_vp, _c_vp, _c_vp, _c_vp]),
    "sparstar_score_select": (_c_i32, [ctypes.POINTER(Problem), _c_vp, _c_vp, _c_dbl, _c_i32, _c_vp, _c_vp,
                                       _c_i64, _c_vp]),
    "sparstar_bsa_workspace_bytes": (_c_i64, [ctypes.POINTER(Problem)]),
    "sparstar_bsa_fwd": (_c_i32, [ctypes.POINTER(Problem), _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i64,
                                  _c_vp, _c_vp, _c_vp, _c_i64, _c_vp]),
    "dense_attn_fwd": (_c_i32, [ctypes.POINTER(Problem), _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i64,
                                _c_vp]),
    "sparstar_balance_workspace_bytes": (_c_i64, [ctypes.POINTER(Problem)]),
    "sparstar_attention_kernel": (_c_i32, [ctypes.POINTER(Problem)]),
    "sparstar_mfma_probe_sink_len": (_c_i64, []),
    "sparstar_mfma_probe": (_c_i32, [_c_i32, _c_vp, _c_i64, ctypes.POINTER(ctypes.c_double), _c_vp]),
    "sparstar_bsa_fwd_balanced": (_c_i32, [ctypes.POINTER(Problem), _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i64,
                                           _c_vp, _c_vp, _c_vp, _c_i64, _c_vp]),
    "sparstar_bsa_fwd_balanced_noalloc": (_c_i32, [ctypes.POINTER(Problem), _c_vp, _c_vp, _c_vp, _c_vp, _c_vp,
                                                   _c_i64, _c_vp, _c_vp, _c_vp]),
    "sparstar_block_mass": (_c_i32, [ctypes.POINTER(Problem), _c_vp, _c_vp, _c_vp, _c_vp, _c_vp]),
    "sparstar_selection_mass": (_c_i32, [ctypes.POINTER(Problem), _c_vp, _c_vp, _c_vp, _c_i64, _c_vp, _c_vp]),
    "sparstar_window_scores": (_c_i32, [ctypes.POINTER(Problem), _c_vp, _c_vp]),
    "sparstar_token_topk_mass": (_c_i32, [ctypes.POINTER(Problem), _c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64,
                                          _c_i64, _c_vp, _c_vp]),
}


def lib() -> ctypes.CDLL:
    """Load libsparstar.so (once); raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise SparstarError(ERR_UNSUPPORTED, f"{LIB_PATH} is missing; build it with "
                                "`python -m block_sparse_attention_aggregated_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != OK:
        raise SparstarError(status, lib().sparstar_last_error().decode())


def _dt(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return BF16
    if t == torch.float32:
        return F32
    raise SparstarError(ERR_UNSUPPORTED, f"dtype {t} is not supported (bf16 or float32)")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


@dataclass(frozen=True)
class Scale:
    """Segment lengths and block size of one scale (the rest comes from the tensors)."""

    len_text: int
    len_ref: int
    block: int = 128
    softmax_scale: Optional[float] = None   # default 1/sqrt(head_dim)


def problem(q: torch.Tensor, k: torch.Tensor, v: Optional[torch.Tensor], scale: Scale,
            out: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None) -> Problem:
    """Fill a sparstar_problem from Q [B,H,L_q,D], K/V [B,H,L_k,D] and an optional output."""
    if q.dim() != 4 or k.dim() != 4:
        raise SparstarError(ERR_SHAPE, "q and k must be [B, H, L, D]")
    B, H, L_q, D = q.shape
    if k.shape[0] != B or k.shape[1] != H or k.shape[3] != D:
        raise SparstarError(ERR_SHAPE, f"k shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    if k.shape[2] != scale.len_text + scale.len_ref + L_q:
        raise SparstarError(ERR_SHAPE, f"L_k = {k.shape[2]} but len_text + len_ref + L_q = "
                            f"{scale.len_text + scale.len_ref + L_q}")
    if v is not None and v.shape != k.shape:
        raise SparstarError(ERR_SHAPE, "v must have the shape of k")
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        if t is not None and t.stride(-1) != 1:
            raise SparstarError(ERR_LAYOUT, f"{name} must be contiguous in head_dim")
    p = Problem()
    p.batch, p.heads, p.head_dim, p.block = B, H, D, scale.block
    p.len_q, p.len_text, p.len_ref = L_q, scale.len_text, scale.len_ref
    p.dtype = _dt(q.dtype)
    if k.dtype != q.dtype or (v is not None and v.dtype != q.dtype):
        raise SparstarError(ERR_UNSUPPORTED, "q, k and v must share a dtype")
    od = out.dtype if out is not None else (out_dtype or q.dtype)
    p.out_dtype = _dt(od)
    p.softmax_scale = scale.softmax_scale if scale.softmax_scale is not None else 1.0 / math.sqrt(D)
    p.reserved = 0
    p.q_stride[:] = list(q.stride()[:3])
    p.k_stride[:] = list(k.stride()[:3])
    p.v_stride[:] = list((v if v is not None else k).stride()[:3])
    p.o_stride[:] = list(out.stride()[:3]) if out is not None else [H * L_q * D, L_q * D, D]
    return p


# ---------------------------------------------------------------- host-only helpers

def check_problem(p: Problem) -> int:
    return lib().sparstar_check_problem(ctypes.byref(p))


def num_q_blocks(p: Problem) -> int:
    return lib().sparstar_num_q_blocks(ctypes.byref(p))


def num_k_blocks(p: Problem) -> int:
    return lib().sparstar_num_k_blocks(ctypes.byref(p))


def num_retained(p: Problem, policy: int = POLICY_LATER_CLIP) -> int:
    return lib().sparstar_num_retained(ctypes.byref(p), policy)


def budget(n_candidates: int, density: float) -> int:
    return lib().sparstar_budget(n_candidates, density)


def blocks_per_row(p: Problem, density: float, policy: int = POLICY_LATER_CLIP) -> int:
    return lib().sparstar_blocks_per_row(ctypes.byref(p), density, policy)


def select_nnz(p: Problem, density: float, policy: int = POLICY_LATER_CLIP) -> int:
    return lib().sparstar_select_nnz(ctypes.byref(p), density, policy)


def balance_workspace_bytes(p: Problem) -> int:
    return lib().sparstar_balance_workspace_bytes(ctypes.byref(p))


def attention_kernel(p: Problem) -> int:
    """KERNEL_MFMA_BF16 or KERNEL_F32: which attention kernel the problem runs on (-1 if invalid)."""
    return lib().sparstar_attention_kernel(ctypes.byref(p))


def mfma_probe_sink_len() -> int:
    """Floats the sink of sparstar_mfma_probe needs on the current device (-1 if unknown)."""
    return lib().sparstar_mfma_probe_sink_len()


def sparstar_mfma_probe(rounds: int, sink: torch.Tensor) -> float:
    """One launch of the matrix-core rate probe on the current stream (a measurement helper,
    not a step of the method); returns the launch's multiply-add flops."""
    if sink.dtype != torch.float32 or not sink.is_contiguous():
        raise SparstarError(ERR_SHAPE, "sink must be contiguous float32")
    flops = ctypes.c_double(0.0)
    _check(lib().sparstar_mfma_probe(int(rounds), _ptr(sink), sink.numel(), ctypes.byref(flops),
                                     _stream(sink.device)))
    return flops.value


def status_string(s: int) -> str:
    return lib().sparstar_status_string(s).decode()


def last_error() -> str:
    return lib().sparstar_last_error().decode()


# ---------------------------------------------------------------- device calls

def sparstar_pool_score(q: torch.Tensor, k: torch.Tensor, scale: Scale, q_pool=None, k_pool=None,
                        scores=None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Block means of Q and K and the block scores (float32)."""
    p = problem(q, k, None, scale)
    B, H, _, D = q.shape
    nq, nk = num_q_blocks(p), num_k_blocks(p)
    dev = q.device
    if q_pool is None:
        q_pool = torch.empty((B, H, nq, D), dtype=torch.float32, device=dev)
    if k_pool is None:
        k_pool = torch.empty((B, H, nk, D), dtype=torch.float32, device=dev)
    if scores is None:
        scores = torch.empty((B, H, nq, nk), dtype=torch.float32, device=dev)
    for t, shape in ((q_pool, (B, H, nq, D)), (k_pool, (B, H, nk, D)), (scores, (B, H, nq, nk))):
        if tuple(t.shape) != shape or not t.is_contiguous() or t.dtype != torch.float32:
            raise SparstarError(ERR_SHAPE, f"expected contiguous float32 {shape}, got {tuple(t.shape)}")
    _check(lib().sparstar_pool_score(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(q_pool), _ptr(k_pool),
                                     _ptr(scores), _stream(dev)))
    return q_pool, k_pool, scores


def sparstar_select_blocks(scores: torch.Tensor, q: torch.Tensor, k: torch.Tensor, scale: Scale,
                           density: float, policy: int = POLICY_LATER_CLIP, row_ptr=None,
                           col_idx=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """CSR block lists (row_ptr int32 [rows+1], col_idx int32 [nnz]) from the scores."""
    p = problem(q, k, None, scale)
    B, H = q.shape[0], q.shape[1]
    nq, nk = num_q_blocks(p), num_k_blocks(p)
    if tuple(scores.shape) != (B, H, nq, nk) or not scores.is_contiguous():
        raise SparstarError(ERR_SHAPE, "scores must be contiguous [B, H, n_q, n_k]")
    nnz = select_nnz(p, density, policy)
    if nnz < 0:
        raise SparstarError(ERR_DENSITY, f"density {density} / policy {policy} rejected")
    dev = scores.device
    if row_ptr is None:
        row_ptr = torch.empty((B * H * nq + 1,), dtype=torch.int32, device=dev)
    if col_idx is None:
        col_idx = torch.empty((max(nnz, 1),), dtype=torch.int32, device=dev)
    _check(lib().sparstar_select_blocks(ctypes.byref(p), _ptr(scores), float(density), policy,
                                        _ptr(row_ptr), _ptr(col_idx), col_idx.numel(), _stream(dev)))
    return row_ptr, col_idx[:nnz]


def sparstar_pool_blocks(q: torch.Tensor, k: torch.Tensor, scale: Scale, q_pool=None,
                         k_pool=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Block means of Q and K (float32), without the scores."""
    p = problem(q, k, None, scale)
    B, H, _, D = q.shape
    nq, nk = num_q_blocks(p), num_k_blocks(p)
    dev = q.device
    if q_pool is None:
        q_pool = torch.empty((B, H, nq, D), dtype=torch.float32, device=dev)
    if k_pool is None:
        k_pool = torch.empty((B, H, nk, D), dtype=torch.float32, device=dev)
    for t, shape in ((q_pool, (B, H, nq, D)), (k_pool, (B, H, nk, D))):
        if tuple(t.shape) != shape or not t.is_contiguous() or t.dtype != torch.float32:
            raise SparstarError(ERR_SHAPE, f"expected contiguous float32 {shape}, got {tuple(t.shape)}")
    _check(lib().sparstar_pool_blocks(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(q_pool), _ptr(k_pool),
                                      _stream(dev)))
    return q_pool, k_pool


def sparstar_score_select(q_pool: torch.Tensor, k_pool: torch.Tensor, q: torch.Tensor, k: torch.Tensor,
                          scale: Scale, density: float, policy: int = POLICY_LATER_CLIP, row_ptr=None,
                          col_idx=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """CSR block lists from the block means, scores formed on chip (no score matrix)."""
    p = problem(q, k, None, scale)
    B, H, _, D = q.shape
    nq, nk = num_q_blocks(p), num_k_blocks(p)
    for t, shape in ((q_pool, (B, H, nq, D)), (k_pool, (B, H, nk, D))):
        if tuple(t.shape) != shape or not t.is_contiguous() or t.dtype != torch.float32:
            raise SparstarError(ERR_SHAPE, f"expected contiguous float32 {shape}, got {tuple(t.shape)}")
    nnz = select_nnz(p, density, policy)
    if nnz < 0:
        raise SparstarError(ERR_DENSITY, f"density {density} / policy {policy} rejected")
    dev = q_pool.device
    if row_ptr is None:
        row_ptr = torch.empty((B * H * nq + 1,), dtype=torch.int32, device=dev)
    if col_idx is None:
        col_idx = torch.empty((max(nnz, 1),), dtype=torch.int32, device=dev)
    _check(lib().sparstar_score_select(ctypes.byref(p), _ptr(q_pool), _ptr(k_pool), float(density), policy,
                                       _ptr(row_ptr), _ptr(col_idx), col_idx.numel(), _stream(dev)))
    return row_ptr, col_idx[:nnz]


def bsa_workspace_bytes(p: Problem) -> int:
    return lib().sparstar_bsa_workspace_bytes(ctypes.byref(p))


def sparstar_bsa_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, row_ptr: torch.Tensor,
                     col_idx: torch.Tensor, scale: Scale, out=None, out_dtype=None,
                     return_lse: bool = False, workspace="auto"):
    """Block-sparse attention forward over the CSR block lists.

    workspace: "auto" allocates the row-queue counters with torch (persistent grid, dynamic
    queues), a device tensor is used as given, None runs one workgroup per row (no workspace)."""
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    p = problem(q, k, v, scale, out=out)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if return_lse else None
    if row_ptr.dtype != torch.int32 or col_idx.dtype != torch.int32:
        raise SparstarError(ERR_UNSUPPORTED, "row_ptr and col_idx must be int32")
    rows = q.shape[0] * q.shape[1] * num_q_blocks(p)
    if row_ptr.numel() != rows + 1 or not row_ptr.is_contiguous() or not col_idx.is_contiguous():
        raise SparstarError(ERR_SHAPE, f"row_ptr must hold {rows + 1} entries, contiguous")
    if isinstance(workspace, str):
        workspace = torch.empty((max(bsa_workspace_bytes(p), 4) // 4,), dtype=torch.int32, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().sparstar_bsa_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(row_ptr), _ptr(col_idx),
                                  col_idx.numel(), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes,
                                  _stream(q.device)))
    return (out, lse) if return_lse else out


def sparstar_bsa_fwd_balanced(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, row_ptr: torch.Tensor,
                              col_idx: torch.Tensor, scale: Scale, out=None, out_dtype=None,
                              return_lse: bool = False, workspace=None):
    """sparstar_bsa_fwd with the rows started longest list first (uneven lists)."""
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    p = problem(q, k, v, scale, out=out)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if return_lse else None
    if row_ptr.dtype != torch.int32 or col_idx.dtype != torch.int32:
        raise SparstarError(ERR_UNSUPPORTED, "row_ptr and col_idx must be int32")
    rows = q.shape[0] * q.shape[1] * num_q_blocks(p)
    if row_ptr.numel() != rows + 1 or not row_ptr.is_contiguous() or not col_idx.is_contiguous():
        raise SparstarError(ERR_SHAPE, f"row_ptr must hold {rows + 1} entries, contiguous")
    need = balance_workspace_bytes(p)
    if workspace is None:
        workspace = torch.empty((max(need, 4) // 4,), dtype=torch.int32, device=q.device)
    _check(lib().sparstar_bsa_fwd_balanced(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(row_ptr),
                                           _ptr(col_idx), col_idx.numel(), _ptr(out), _ptr(lse), _ptr(workspace),
                                           workspace.numel() * workspace.element_size(), _stream(q.device)))
    return (out, lse) if return_lse else out


def sparstar_bsa_fwd_balanced_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, row_ptr: torch.Tensor,
                                      col_idx: torch.Tensor, scale: Scale, out: torch.Tensor,
                                      lse: Optional[torch.Tensor] = None) -> None:
    """sparstar_bsa_fwd_balanced with the library's own scratch: the caller passes every output."""
    p = problem(q, k, v, scale, out=out)
    if row_ptr.dtype != torch.int32 or col_idx.dtype != torch.int32:
        raise SparstarError(ERR_UNSUPPORTED, "row_ptr and col_idx must be int32")
    rows = q.shape[0] * q.shape[1] * num_q_blocks(p)
    if row_ptr.numel() != rows + 1 or not row_ptr.is_contiguous() or not col_idx.is_contiguous():
        raise SparstarError(ERR_SHAPE, f"row_ptr must hold {rows + 1} entries, contiguous")
    if lse is not None and (tuple(lse.shape) != tuple(q.shape[:3]) or lse.dtype != torch.float32
                            or not lse.is_contiguous()):
        raise SparstarError(ERR_SHAPE, "lse must be contiguous float32 [B, H, L_q]")
    _check(lib().sparstar_bsa_fwd_balanced_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(row_ptr),
                                                   _ptr(col_idx), col_idx.numel(), _ptr(out), _ptr(lse),
                                                   _stream(q.device)))


def dense_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: Scale, out=None,
                   out_dtype=None, return_lse: bool = False, workspace="auto"):
    """Dense attention forward over every key block (the density-1 baseline); workspace as for
    sparstar_bsa_fwd."""
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    p = problem(q, k, v, scale, out=out)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if return_lse else None
    if isinstance(workspace, str):
        workspace = torch.empty((max(bsa_workspace_bytes(p), 4) // 4,), dtype=torch.int32, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().dense_attn_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                _ptr(workspace), ws_bytes, _stream(q.device)))
    return (out, lse) if return_lse else out


def scale_forward(q, k, v, scale: Scale, density: float, policy: int = POLICY_LATER_CLIP,
                  out_dtype=None, return_lse: bool = False):
    """One SparSTAR scale: pool and score, select, block-sparse attention."""
    _, _, scores = sparstar_pool_score(q, k, scale)
    row_ptr, col_idx = sparstar_select_blocks(scores, q, k, scale, density, policy)
    res = sparstar_bsa_fwd(q, k, v, row_ptr, col_idx, scale, out_dtype=out_dtype, return_lse=return_lse)
    return res, (scores, row_ptr, col_idx)


# ---------------------------------------------------------------- retained attention mass

def sparstar_block_mass(q: torch.Tensor, k: torch.Tensor, lse: torch.Tensor, scale: Scale,
                        mass=None) -> torch.Tensor:
    """Dense softmax mass per (query block, key block), float32 [B, H, n_q, n_k]."""
    p = problem(q, k, None, scale)
    B, H = q.shape[0], q.shape[1]
    nq, nk = num_q_blocks(p), num_k_blocks(p)
    if tuple(lse.shape) != tuple(q.shape[:3]) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise SparstarError(ERR_SHAPE, "lse must be contiguous float32 [B, H, L_q]")
    if mass is None:
        mass = torch.empty((B, H, nq, nk), dtype=torch.float32, device=q.device)
    if tuple(mass.shape) != (B, H, nq, nk) or not mass.is_contiguous() or mass.dtype != torch.float32:
        raise SparstarError(ERR_SHAPE, "mass must be contiguous float32 [B, H, n_q, n_k]")
    _check(lib().sparstar_block_mass(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(lse), _ptr(mass),
                                     _stream(q.device)))
    return mass


def sparstar_selection_mass(mass: torch.Tensor, row_ptr: torch.Tensor, col_idx: torch.Tensor,
                            q: torch.Tensor, k: torch.Tensor, scale: Scale) -> torch.Tensor:
    """Mean retained mass per query block of a CSR selection, float32 [B*H*n_q]."""
    p = problem(q, k, None, scale)
    rows = q.shape[0] * q.shape[1] * num_q_blocks(p)
    if tuple(mass.shape) != (q.shape[0], q.shape[1], num_q_blocks(p), num_k_blocks(p)) or \
            not mass.is_contiguous():
        raise SparstarError(ERR_SHAPE, "mass must be contiguous [B, H, n_q, n_k]")
    if row_ptr.dtype != torch.int32 or col_idx.dtype != torch.int32 or row_ptr.numel() != rows + 1:
        raise SparstarError(ERR_SHAPE, f"row_ptr must be int32 [{rows + 1}], col_idx int32")
    out = torch.empty((rows,), dtype=torch.float32, device=mass.device)
    _check(lib().sparstar_selection_mass(ctypes.byref(p), _ptr(mass), _ptr(row_ptr), _ptr(col_idx),
                                         col_idx.numel(), _ptr(out), _stream(mass.device)))
    return out


def sparstar_window_scores(q: torch.Tensor, k: torch.Tensor, scale: Scale) -> torch.Tensor:
    """Sliding-window scores, float32 [B, H, n_q, n_k] (minus the block-centre distance)."""
    p = problem(q, k, None, scale)
    out = torch.empty((q.shape[0], q.shape[1], num_q_blocks(p), num_k_blocks(p)), dtype=torch.float32,
                      device=q.device)
    _check(lib().sparstar_window_scores(ctypes.byref(p), _ptr(out), _stream(q.device)))
    return out


def sparstar_token_topk_mass(q: torch.Tensor, k: torch.Tensor, lse: torch.Tensor, rows: torch.Tensor,
                             keep_tokens: int, k_tokens: int, scale: Scale) -> torch.Tensor:
    """Token-wise Top-K mass of the listed queries (rows: int64 (b*H + h)*L_q + t), float32."""
    p = problem(q, k, None, scale)
    if rows.dtype != torch.int64 or not rows.is_contiguous():
        raise SparstarError(ERR_SHAPE, "rows must be contiguous int64")
    if tuple(lse.shape) != tuple(q.shape[:3]) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise SparstarError(ERR_SHAPE, "lse must be contiguous float32 [B, H, L_q]")
    out = torch.empty((rows.numel(),), dtype=torch.float32, device=q.device)
    _check(lib().sparstar_token_topk_mass(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(lse), _ptr(rows),
                                          rows.numel(), int(keep_tokens), int(k_tokens), _ptr(out),
                                          _stream(q.device)))
    return out
