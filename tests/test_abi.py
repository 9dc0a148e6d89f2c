"""The C ABI on the CPU: the library loads, exports what include/sparstar.h
declares, computes the block bookkeeping like the oracle, and rejects bad
arguments before touching the GPU.  No call here reaches a kernel: every
device call is given an argument that validation refuses first."""

import ctypes
import math
import os
import re

import pytest
import torch

import oracle as O
from block_sparse_attention_aggregated_amd import inputs as I
from block_sparse_attention_aggregated_amd import sparstar as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparstar.h")

pytestmark = pytest.mark.skipif(not os.path.exists(S.LIB_PATH), reason="libsparstar.so not built")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol():
    names = _declared_functions()
    assert "sparstar_bsa_fwd" in names and "dense_attn_fwd" in names and len(names) == 26
    assert {"sparstar_mfma_probe", "sparstar_mfma_probe_sink_len"} <= set(names)
    assert {"sparstar_pool_blocks", "sparstar_score_select"} <= set(names)
    assert {"sparstar_block_mass", "sparstar_selection_mass", "sparstar_window_scores",
            "sparstar_token_topk_mass"} <= set(names)
    L = ctypes.CDLL(S.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    assert set(names) <= set(S._SIGS)


def _prob(cfg, dtype=S.BF16, out_dtype=None):
    p = S.Problem()
    p.batch, p.heads, p.head_dim, p.block = cfg.batch, cfg.heads, cfg.head_dim, cfg.block
    p.len_q, p.len_text, p.len_ref = cfg.len_q, cfg.len_text, cfg.len_ref
    p.dtype = dtype
    p.out_dtype = dtype if out_dtype is None else out_dtype
    p.softmax_scale = cfg.softmax_scale
    D = cfg.head_dim
    p.q_stride[:] = [cfg.heads * cfg.len_q * D, cfg.len_q * D, D]
    p.k_stride[:] = [cfg.heads * cfg.len_k * D, cfg.len_k * D, D]
    p.v_stride[:] = list(p.k_stride)
    p.o_stride[:] = list(p.q_stride)
    return p


@pytest.mark.parametrize("name", sorted(I.WORKLOADS))
def test_block_bookkeeping_matches_oracle(name):
    cfg = I.WORKLOADS[name]
    p = _prob(cfg, S.F32 if cfg.dtype == "f32" else S.BF16)
    assert S.check_problem(p) == S.OK
    b = cfg.block
    assert S.num_q_blocks(p) == O.num_blocks(cfg.len_q, b)
    assert S.num_k_blocks(p) == O.num_blocks(cfg.len_k, b)
    for pol in (S.POLICY_LATER_CLIP, S.POLICY_FIRST_CLIP):
        R, C = O.retained_and_candidates(cfg.len_text, cfg.len_ref, cfg.len_q, b, pol)
        assert R == list(range(len(R)))                      # retained set is a prefix
        assert S.num_retained(p, pol) == len(R)
        for rho in cfg.densities + (0.09375, 0.1875, 0.625, 1e-9):
            k = O.budget(len(C), rho)
            assert S.blocks_per_row(p, rho, pol) == len(R) + k
            assert S.select_nnz(p, rho, pol) == cfg.batch * cfg.heads * O.num_blocks(cfg.len_q, b) * (len(R) + k)


def test_appendix_shapes_720p():
    p = _prob(I.S720P)
    assert (S.num_q_blocks(p), S.num_k_blocks(p), S.num_retained(p)) == (563, 1129, 4)
    assert [S.blocks_per_row(p, r) for r in (0.1, 0.2, 0.4, 1.0)] == [117, 229, 454, 1129]
    assert S.select_nnz(p, 0.2) == 4_125_664


def test_budget_matches_oracle():
    for n in (0, 1, 2, 7, 8, 79, 488, 1125, 4096):
        for rho in (1e-9, 0.01, 0.09375, 0.1, 0.1875, 0.2, 0.25, 0.3, 1 / 3, 0.4, 0.5, 0.625, 0.999, 1.0):
            assert S.budget(n, rho) == O.budget(n, rho), (n, rho)
    for bad in (0.0, -0.1, 1.0000001, float("nan"), float("inf")):
        assert S.budget(10, bad) == -1


BOGUS = 0x10000  # never dereferenced: every call below fails validation first

# The calls below pass made-up device pointers that validation must refuse; on a
# machine with a visible GPU a regression there would launch on them, so these
# tests only run where no GPU is visible.
no_gpu = pytest.mark.skipif(torch.cuda.device_count() > 0,
                            reason="made-up pointers are only passed where no GPU is visible")


def _status(fn, *args):
    st = fn(*args)
    return st, S.last_error()


@pytest.mark.parametrize("mutate,code", [
    (lambda p: setattr(p, "head_dim", 96), S.ERR_UNSUPPORTED),
    (lambda p: setattr(p, "block", 32), S.ERR_UNSUPPORTED),
    (lambda p: setattr(p, "block", 512), S.ERR_UNSUPPORTED),
    (lambda p: setattr(p, "dtype", 7), S.ERR_UNSUPPORTED),
    (lambda p: setattr(p, "out_dtype", -1), S.ERR_UNSUPPORTED),
    (lambda p: setattr(p, "batch", -1), S.ERR_SHAPE),
    (lambda p: setattr(p, "len_q", -5), S.ERR_SHAPE),
    (lambda p: setattr(p, "len_text", -1), S.ERR_SHAPE),
    (lambda p: setattr(p, "softmax_scale", float("nan")), S.ERR_SHAPE),
    (lambda p: setattr(p, "softmax_scale", 0.0), S.ERR_SHAPE),
    (lambda p: setattr(p, "reserved", 1), S.ERR_SHAPE),
    (lambda p: p.q_stride.__setitem__(2, 100), S.ERR_LAYOUT),
    (lambda p: p.k_stride.__setitem__(1, 3), S.ERR_LAYOUT),
    (lambda p: p.o_stride.__setitem__(2, 64), S.ERR_LAYOUT),
    (lambda p: p.v_stride.__setitem__(0, -8), S.ERR_LAYOUT),
])
@no_gpu
def test_problem_validation(mutate, code):
    p = _prob(I.S192P)
    mutate(p)
    L = S.lib()
    assert S.check_problem(p) == code
    assert S.num_q_blocks(p) == -1
    b = ctypes.c_void_p(BOGUS)
    st, msg = _status(L.sparstar_pool_score, ctypes.byref(p), b, b, b, b, b, None)
    assert st == code and msg
    st, msg = _status(L.sparstar_select_blocks, ctypes.byref(p), b, 0.3, 0, b, b, 10**9, None)
    assert st == code and msg
    st, msg = _status(L.sparstar_bsa_fwd, ctypes.byref(p), b, b, b, b, b, 10, b, None, b, 256, None)
    assert st == code and msg
    st, msg = _status(L.dense_attn_fwd, ctypes.byref(p), b, b, b, b, None, b, 256, None)
    assert st == code and msg


@no_gpu
def test_null_and_alignment_and_density_and_capacity():
    p = _prob(I.S192P)
    L = S.lib()
    b = ctypes.c_void_p(BOGUS)
    odd = ctypes.c_void_p(BOGUS + 2)
    assert L.sparstar_pool_score(None, b, b, b, b, b, None) == S.ERR_NULL
    assert L.sparstar_pool_score(ctypes.byref(p), None, b, b, b, b, None) == S.ERR_NULL
    assert L.sparstar_pool_score(ctypes.byref(p), b, b, b, b, odd, None) == S.ERR_LAYOUT
    assert L.dense_attn_fwd(ctypes.byref(p), b, b, None, b, None, b, 256, None) == S.ERR_NULL
    assert L.dense_attn_fwd(ctypes.byref(p), b, odd, b, b, None, b, 256, None) == S.ERR_LAYOUT
    assert L.dense_attn_fwd(ctypes.byref(p), b, b, b, b, None, odd, 256, None) == S.ERR_LAYOUT
    assert L.dense_attn_fwd(ctypes.byref(p), b, b, b, b, None, b, 8, None) == S.ERR_CAPACITY
    assert L.sparstar_bsa_fwd(ctypes.byref(p), b, b, b, None, b, 10, b, None, b, 256, None) == S.ERR_NULL
    assert L.sparstar_bsa_fwd(ctypes.byref(p), b, b, b, b, b, -1, b, None, b, 256, None) == S.ERR_SHAPE
    assert L.sparstar_bsa_fwd(ctypes.byref(p), b, b, b, b, b, 10, b, ctypes.c_void_p(BOGUS + 1), b, 256, None) \
        == S.ERR_LAYOUT
    assert L.sparstar_bsa_fwd(ctypes.byref(p), b, b, b, b, b, 10, b, None, odd, 256, None) == S.ERR_LAYOUT
    assert S.bsa_workspace_bytes(p) == 256
    st = L.sparstar_bsa_fwd(ctypes.byref(p), b, b, b, b, b, 10, b, None, b, 255, None)
    assert st == S.ERR_CAPACITY and "workspace" in S.last_error()
    for rho in (0.0, -1.0, 1.5, float("nan")):
        assert L.sparstar_select_blocks(ctypes.byref(p), b, rho, 0, b, b, 10**9, None) == S.ERR_DENSITY
    assert L.sparstar_select_blocks(ctypes.byref(p), b, 0.3, 5, b, b, 10**9, None) == S.ERR_UNSUPPORTED
    nnz = S.select_nnz(p, 0.3)
    assert nnz == 16 * 40 * 28
    st = L.sparstar_select_blocks(ctypes.byref(p), b, 0.3, 0, b, b, nnz - 1, None)
    assert st == S.ERR_CAPACITY and "capacity" in S.last_error()
    assert L.sparstar_select_blocks(ctypes.byref(p), b, 0.3, 0, None, b, nnz, None) == S.ERR_NULL
    assert S.status_string(S.ERR_CAPACITY) == "output capacity too small"


@no_gpu
def test_fused_select_entry_points_validate_before_any_device_call():
    p = _prob(I.S192P)
    L = S.lib()
    b = ctypes.c_void_p(BOGUS)
    odd = ctypes.c_void_p(BOGUS + 4)
    nnz = S.select_nnz(p, 0.3)
    assert L.sparstar_pool_blocks(None, b, b, b, b, None) == S.ERR_NULL
    assert L.sparstar_pool_blocks(ctypes.byref(p), b, b, None, b, None) == S.ERR_NULL
    assert L.sparstar_pool_blocks(ctypes.byref(p), b, b, odd, b, None) == S.ERR_LAYOUT
    for rho in (0.0, 1.5, float("nan")):
        assert L.sparstar_score_select(ctypes.byref(p), b, b, rho, 0, b, b, nnz, None) == S.ERR_DENSITY
    assert L.sparstar_score_select(ctypes.byref(p), b, b, 0.3, 7, b, b, nnz, None) == S.ERR_UNSUPPORTED
    assert L.sparstar_score_select(ctypes.byref(p), None, b, 0.3, 0, b, b, nnz, None) == S.ERR_NULL
    assert L.sparstar_score_select(ctypes.byref(p), odd, b, 0.3, 0, b, b, nnz, None) == S.ERR_LAYOUT
    assert L.sparstar_score_select(ctypes.byref(p), b, b, 0.3, 0, b, b, nnz - 1, None) == S.ERR_CAPACITY
    # a strip's scores must fit LDS: 1,152 key blocks at most
    big = _prob(I.S720P.with_(block=64))                                        # n_k = 2,258
    st = L.sparstar_score_select(ctypes.byref(big), b, b, 0.2, 0, b, b, 10**9, None)
    assert st == S.ERR_UNSUPPORTED and "1152" in S.last_error()


@no_gpu
def test_mass_entry_points_validate_before_any_device_call():
    p = _prob(I.S192P)
    L = S.lib()
    b = ctypes.c_void_p(BOGUS)
    odd = ctypes.c_void_p(BOGUS + 2)
    assert L.sparstar_block_mass(None, b, b, b, b, None) == S.ERR_NULL
    assert L.sparstar_block_mass(ctypes.byref(p), b, b, None, b, None) == S.ERR_NULL
    assert L.sparstar_block_mass(ctypes.byref(p), odd, b, b, b, None) == S.ERR_LAYOUT
    assert L.sparstar_selection_mass(ctypes.byref(p), b, b, None, 10, b, None) == S.ERR_NULL
    assert L.sparstar_selection_mass(ctypes.byref(p), b, b, b, -1, b, None) == S.ERR_SHAPE
    assert L.sparstar_selection_mass(ctypes.byref(p), odd, b, b, 10, b, None) == S.ERR_LAYOUT
    assert L.sparstar_window_scores(ctypes.byref(p), None, None) == S.ERR_NULL
    assert L.sparstar_window_scores(ctypes.byref(p), ctypes.c_void_p(BOGUS + 4), None) == S.ERR_LAYOUT
    assert L.sparstar_token_topk_mass(ctypes.byref(p), b, b, b, b, -1, 0, 0, b, None) == S.ERR_SHAPE
    assert L.sparstar_token_topk_mass(ctypes.byref(p), b, b, b, b, 4, -1, 0, b, None) == S.ERR_SHAPE
    assert L.sparstar_token_topk_mass(ctypes.byref(p), b, b, b, None, 4, 0, 0, b, None) == S.ERR_NULL
    assert L.sparstar_token_topk_mass(ctypes.byref(p), b, b, b, ctypes.c_void_p(BOGUS + 4), 4, 0, 0, b,
                                      None) == S.ERR_LAYOUT
    # 256 bytes of queue counters, then the row order
    assert L.sparstar_balance_workspace_bytes(ctypes.byref(p)) == 256 + 16 * 40 * 4   # 4 segments of 10 blocks
    p64 = _prob(I.S192P_B64)                                                     # n_q = 79: 8 segments of 10
    assert L.sparstar_balance_workspace_bytes(ctypes.byref(p64)) == 256 + 16 * 8 * 10 * 4
    p256 = _prob(I.S192P_B256)                                                   # n_q = 20: 4 segments of 5
    assert L.sparstar_balance_workspace_bytes(ctypes.byref(p256)) == 256 + 16 * 4 * 5 * 4
    p.heads = 15                                                                 # odd head count: 8 segments of 5
    assert L.sparstar_balance_workspace_bytes(ctypes.byref(p)) == 256 + 15 * 8 * 5 * 4
    p.heads = 16
    assert L.sparstar_bsa_fwd_balanced(ctypes.byref(p), b, b, b, b, b, 10, b, None, None, 1 << 20, None) \
        == S.ERR_NULL
    assert L.sparstar_bsa_fwd_balanced(ctypes.byref(p), b, b, b, b, b, 10, b, None, b, 256 + 16 * 40 * 4 - 1,
                                       None) == S.ERR_CAPACITY
    assert L.sparstar_bsa_fwd_balanced(ctypes.byref(p), b, b, b, b, b, -1, b, None, b, 1 << 20, None) \
        == S.ERR_SHAPE
    # nothing listed: nothing to do, no device needed
    assert L.sparstar_token_topk_mass(ctypes.byref(p), None, None, None, None, 0, 0, 0, None, None) == S.OK


@no_gpu
def test_too_many_candidates_is_refused():
    cfg = I.S720P.with_(grid=(20, 90, 160), block=64)      # n_k - retained > 4096 candidates
    p = _prob(cfg)
    b = ctypes.c_void_p(BOGUS)
    st = S.lib().sparstar_select_blocks(ctypes.byref(p), b, 0.2, 0, b, b, 10**12, None)
    assert st == S.ERR_UNSUPPORTED


@no_gpu
def test_noalloc_refuses_problems_beyond_its_scratch():
    """The allocation-free call holds 1 MiB of queue counters and row order per device: a problem whose
    order does not fit is refused before anything touches a device, with a message saying why."""
    L = S.lib()
    b = ctypes.c_void_p(BOGUS)
    p = _prob(I.S720P)
    assert 256 + 4 * 32 * 4 * 141 <= 1 << 20
    big = _prob(I.S720P.with_(batch=16))                 # 16 * 32 heads * 4 segments * 141 rows
    assert S.balance_workspace_bytes(big) > 1 << 20
    st = L.sparstar_bsa_fwd_balanced_noalloc(ctypes.byref(big), b, b, b, b, b, 10, b, None, None)
    assert st == S.ERR_CAPACITY and "scratch" in S.last_error()
    assert L.sparstar_bsa_fwd_balanced_noalloc(None, b, b, b, b, b, 10, b, None, None) == S.ERR_NULL
    assert L.sparstar_bsa_fwd_balanced_noalloc(ctypes.byref(p), b, b, b, None, b, 10, b, None, None) \
        in (S.ERR_NULL, S.ERR_UNSUPPORTED, S.ERR_HIP)


def test_attention_kernel_choice():
    """The host names the kernel a problem runs on: bf16 at head_dim 128 on the MFMA kernel,
    float32 inputs and head_dim 64 (bf16 too) on the float32 kernel; invalid problems -1."""
    assert S.attention_kernel(_prob(I.S720P)) == S.KERNEL_MFMA_BF16
    assert S.attention_kernel(_prob(I.S720P_B64)) == S.KERNEL_MFMA_BF16
    assert S.attention_kernel(_prob(I.TINY, S.F32)) == S.KERNEL_F32
    assert S.attention_kernel(_prob(I.TINY, S.BF16)) == S.KERNEL_F32          # head_dim 64
    assert S.attention_kernel(_prob(I.S192P, S.F32)) == S.KERNEL_F32
    wide = _prob(I.S192P)
    wide.k_stride[2] = 1 << 18                                               # K/V extents past 2^31 bytes
    assert S.attention_kernel(wide) == S.KERNEL_F32
    bad = _prob(I.S192P)
    bad.block = 96
    assert S.attention_kernel(bad) == -1


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(S, "_lib", None)
    monkeypatch.setattr(S, "LIB_PATH", "/nonexistent/libsparstar.so")
    with pytest.raises(S.SparstarError):
        S.lib()


def test_mfma_probe_validates_before_any_device_call():
    L = S.lib()
    flops = ctypes.c_double(-1.0)
    b = ctypes.c_void_p(BOGUS)
    assert L.sparstar_mfma_probe(0, b, 1 << 20, ctypes.byref(flops), None) == S.ERR_SHAPE
    assert L.sparstar_mfma_probe(-5, b, 1 << 20, ctypes.byref(flops), None) == S.ERR_SHAPE
    assert L.sparstar_mfma_probe(10, None, 1 << 20, ctypes.byref(flops), None) == S.ERR_NULL
    assert L.sparstar_mfma_probe(10, ctypes.c_void_p(BOGUS + 2), 1 << 20, ctypes.byref(flops), None) == S.ERR_LAYOUT
    assert flops.value == -1.0   # nothing written on an error
