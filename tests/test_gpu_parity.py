"""GPU parity: every step of the HIP path against the float64 CPU oracle.

All calls go through the C ABI (ctypes binding).  Inputs come from the
seeded generator; the oracle reads the very values uploaded to the GPU."""

import math

import numpy as np
import pytest
import torch

import oracle as O
from block_sparse_attention_aggregated_amd import inputs as I
from block_sparse_attention_aggregated_amd import sparstar as S

from parity import (BF16_MAX_ABS, BF16_MEAN_ABS, F32_MAX_ABS, attention_errors, compare_row_selection,
                    csr_rows, excess_over_bf16_store, oracle_rows, to_f64)

pytestmark = pytest.mark.gpu

# LSE of bf16 inputs: float32 exp2/log and sums of float32 logits of bf16 data;
# 2e-3 is a few hundred float32 ulps at |lse| ~ 10-25.
LSE_BF16 = 2e-3

DEV = "cuda:0"
_CACHE = {}


def inputs(cfg):
    key = cfg
    if key not in _CACHE:
        if len(_CACHE) >= 2:
            _CACHE.clear()
            torch.cuda.empty_cache()
        _CACHE[key] = I.make_inputs(cfg, device=DEV)
        torch.cuda.synchronize()
    return _CACHE[key]


def scale_of(cfg):
    return S.Scale(cfg.len_text, cfg.len_ref, cfg.block, cfg.softmax_scale)


def head_np(t, h):
    return to_f64(t[0, h])


def print_case(*a):
    print("CASE", *a, flush=True)


# ---------------------------------------------------------------- pool + score

@pytest.mark.parametrize("cfg,heads", [(I.TINY, None), (I.S192P, None), (I.S480P, [0, 23])])
def test_pool_score_parity(cfg, heads):
    print_case("pool_score", cfg.name)
    Q, K, V = inputs(cfg)
    qp, kp, sc = S.sparstar_pool_score(Q, K, scale_of(cfg))
    torch.cuda.synchronize()
    b, sigma = cfg.block, cfg.softmax_scale
    for h in (range(cfg.heads) if heads is None else heads):
        q, k = head_np(Q, h), head_np(K, h)
        qbar, kbar = O.pool_blocks(q, b), O.pool_blocks(k, b)
        S_ref = O.block_scores(qbar, kbar, sigma)
        assert np.max(np.abs(to_f64(qp[0, h]) - qbar)) < 2e-6 * max(1.0, np.abs(qbar).max())
        assert np.max(np.abs(to_f64(kp[0, h]) - kbar)) < 2e-6 * max(1.0, np.abs(kbar).max())
        # float32 dot products of length D: error bounded by D * eps * sum |terms|
        bound = cfg.head_dim * 6e-8 * sigma * (np.abs(qbar) @ np.abs(kbar).T) + 1e-7
        err = np.abs(to_f64(sc[0, h]) - S_ref)
        assert np.all(err <= bound), float((err / bound).max())


# ---------------------------------------------------------------- selection

@pytest.mark.parametrize("cfg,rho,policy", [(I.TINY, 0.5, 0), (I.TINY, 1.0, 0), (I.TINY, 0.25, 1),
                                            (I.S192P, 0.3, 0), (I.S192P, 0.05, 1), (I.S192P, 1.0, 0)])
def test_select_bitexact_on_oracle_scores(cfg, rho, policy):
    """Given the same float32 scores, the GPU selection equals the oracle's exactly."""
    print_case("select exact", cfg.name, rho, policy)
    Q, K, V = inputs(cfg)
    b, sigma = cfg.block, cfg.softmax_scale
    S32 = torch.empty((1, cfg.heads, O.num_blocks(cfg.len_q, b), O.num_blocks(cfg.len_k, b)),
                      dtype=torch.float32)
    for h in range(cfg.heads):
        S32[0, h] = torch.from_numpy(O.block_scores(O.pool_blocks(head_np(Q, h), b),
                                                    O.pool_blocks(head_np(K, h), b), sigma))
    # plant exact ties to exercise the lower-index rule
    S32[0, 0, 0, -4:] = S32[0, 0, 0, -5]
    rp, ci = S.sparstar_select_blocks(S32.to(DEV), Q, K, scale_of(cfg), rho, policy)
    rows = csr_rows(rp, ci)
    R, C = O.retained_and_candidates(cfg.len_text, cfg.len_ref, cfg.len_q, b, policy)
    kk = O.budget(len(C), rho)
    nq = O.num_blocks(cfg.len_q, b)
    for h in range(cfg.heads):
        ref = O.select_blocks(S32[0, h].double().numpy(), R, C, kk)
        for i in range(nq):
            assert np.array_equal(rows[h * nq + i], ref[i]), (h, i)


@pytest.mark.parametrize("cfg,rho,heads", [(I.TINY, 0.5, None), (I.S192P, 0.3, None),
                                           (I.S480P, 0.25, [0, 11, 23])])
def test_select_parity_end_to_end(cfg, rho, heads):
    """GPU scores -> GPU selection vs the oracle's own scores and selection (tie rule)."""
    print_case("select e2e", cfg.name, rho)
    Q, K, V = inputs(cfg)
    sc = S.sparstar_pool_score(Q, K, scale_of(cfg))[2]
    rp, ci = S.sparstar_select_blocks(sc, Q, K, scale_of(cfg), rho)
    rows = csr_rows(rp, ci)
    b = cfg.block
    nq = O.num_blocks(cfg.len_q, b)
    swaps = 0
    for h in (range(cfg.heads) if heads is None else heads):
        res = O.scale_head(head_np(Q, h), head_np(K, h), head_np(V, h), cfg.len_text, cfg.len_ref, b,
                           cfg.softmax_scale, rho, rows=[])
        for i in range(nq):
            swaps += compare_row_selection(rows[h * nq + i], res["sets"][i], res["scores"][i],
                                           len(res["retained"]), res["k"])
    print(f"near-tie swaps: {swaps}")


# ---------------------------------------------------------------- attention

def _check_attention(cfg, Q, K, V, rows_lists, out, lse, heads, sample_rows, bf16_in):
    b, sigma = cfg.block, cfg.softmax_scale
    nq = O.num_blocks(cfg.len_q, b)
    worst_max, worst_excess, worst_lse, sum_abs, n = 0.0, -1.0, 0.0, 0.0, 0
    bf16_store = out.dtype == torch.bfloat16
    for h in heads:
        q, k, v = head_np(Q, h), head_np(K, h), head_np(V, h)
        lists = rows_lists[h * nq:(h + 1) * nq]
        rows = range(nq) if sample_rows is None else sample_rows(h)
        ref_o, ref_l = oracle_rows(q, k, v, lists, rows, b, sigma)
        got = to_f64(out[0, h])
        got_l = to_f64(lse[0, h]) if lse is not None else None
        for i in rows:
            s, e = O.block_range(i, cfg.len_q, b)
            mx, mean = attention_errors(got[s:e], ref_o[i])
            worst_max = max(worst_max, mx)
            if bf16_store:
                worst_excess = max(worst_excess, excess_over_bf16_store(got[s:e], ref_o[i]))
            sum_abs += mean * (e - s) * cfg.head_dim
            n += (e - s) * cfg.head_dim
            if got_l is not None:
                worst_lse = max(worst_lse, float(np.max(np.abs(got_l[s:e] - ref_l[i]))))
    mean_abs = sum_abs / max(n, 1)
    print(f"max-abs {worst_max:.3e} mean-abs {mean_abs:.3e} over {n // cfg.head_dim} queries"
          + (f"; beyond the bf16 store rounding {worst_excess:.3e}" if bf16_store else "")
          + (f"; lse max-abs {worst_lse:.3e}" if lse is not None else ""))
    assert worst_lse < (LSE_BF16 if bf16_in else 1e-5)
    if bf16_in:
        assert mean_abs <= BF16_MEAN_ABS
        assert (worst_excess if bf16_store else worst_max) <= BF16_MAX_ABS
    else:
        assert worst_max <= F32_MAX_ABS
    return worst_max, mean_abs


@pytest.mark.parametrize("cfg,rho,out_dtype,heads,nsample", [
    (I.TINY, 0.5, torch.float32, None, None),
    (I.TINY, 1.0, torch.float32, None, None),
    (I.S192P, 0.3, torch.bfloat16, None, None),
    (I.S192P, 0.3, torch.float32, [0, 7, 15], None),
    (I.S480P, 0.25, torch.bfloat16, [0, 9, 23], 12),
    (I.S480P, 0.25, torch.float32, [0, 9, 23], 12),
])
def test_bsa_parity_on_gpu_csr(cfg, rho, out_dtype, heads, nsample):
    """bsa_fwd against oracle attention over the GPU's own block lists."""
    print_case("bsa", cfg.name, rho, out_dtype)
    Q, K, V = inputs(cfg)
    (out, lse), (_, rp, ci) = S.scale_forward(Q, K, V, scale_of(cfg), rho, out_dtype=out_dtype,
                                               return_lse=True)
    torch.cuda.synchronize()
    lists = csr_rows(rp, ci)
    nq = O.num_blocks(cfg.len_q, cfg.block)
    sampler = None
    if nsample:
        def sampler(h):
            rng = np.random.default_rng(1000 + h)
            return sorted({0, nq - 1, *rng.choice(nq, nsample, replace=False).tolist()})
    _check_attention(cfg, Q, K, V, lists, out, lse, range(cfg.heads) if heads is None else heads,
                     sampler, cfg.dtype == "bf16")


def test_bsa_end_to_end_against_oracle_selection():
    """Where the selections agree, the GPU output meets the bounds against the oracle's own sets."""
    cfg = I.S192P
    print_case("bsa e2e", cfg.name)
    Q, K, V = inputs(cfg)
    out = S.scale_forward(Q, K, V, scale_of(cfg), 0.3)[0]
    torch.cuda.synchronize()
    for h in (0, 5):
        res = O.scale_head(head_np(Q, h), head_np(K, h), head_np(V, h), cfg.len_text, cfg.len_ref,
                           cfg.block, cfg.softmax_scale, 0.3)
        got = to_f64(out[0, h])
        mx, mean = attention_errors(got, res["out"])
        assert excess_over_bf16_store(got, res["out"]) <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, (h, mx, mean)


@pytest.mark.parametrize("cfg,heads,nsample", [(I.TINY, None, None), (I.S192P, [0, 15], 8)])
def test_dense_parity(cfg, heads, nsample):
    print_case("dense", cfg.name)
    Q, K, V = inputs(cfg)
    out, lse = S.dense_attn_fwd(Q, K, V, scale_of(cfg), out_dtype=torch.float32, return_lse=True)
    torch.cuda.synchronize()
    nq, nk = O.num_blocks(cfg.len_q, cfg.block), O.num_blocks(cfg.len_k, cfg.block)
    lists = [np.arange(nk)] * (nq * cfg.heads)
    sampler = None
    if nsample:
        def sampler(h):
            rng = np.random.default_rng(7 + h)
            return sorted({0, nq - 1, *rng.choice(nq, nsample, replace=False).tolist()})
    _check_attention(cfg, Q, K, V, lists, out, lse, range(cfg.heads) if heads is None else heads,
                     sampler, cfg.dtype == "bf16")


@pytest.mark.parametrize("cfg", [I.TINY, I.S192P])
def test_bsa_full_csr_equals_dense_bitwise(cfg):
    print_case("full csr == dense", cfg.name)
    Q, K, V = inputs(cfg)
    sc = S.sparstar_pool_score(Q, K, scale_of(cfg))[2]
    rp, ci = S.sparstar_select_blocks(sc, Q, K, scale_of(cfg), 1.0)
    a = S.sparstar_bsa_fwd(Q, K, V, rp, ci, scale_of(cfg))
    d = S.dense_attn_fwd(Q, K, V, scale_of(cfg))
    torch.cuda.synchronize()
    assert torch.equal(a, d)


# ---------------------------------------------------------------- properties and edge cases

def test_determinism_and_nan_poison():
    cfg = I.S192P
    print_case("determinism", cfg.name)
    Q, K, V = inputs(cfg)
    outs = []
    for _ in range(2):
        o = torch.full(Q.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
        lse = torch.full(Q.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
        _, _, sc = S.sparstar_pool_score(Q, K, scale_of(cfg))
        rp, ci = S.sparstar_select_blocks(sc, Q, K, scale_of(cfg), 0.3)
        res = S.sparstar_bsa_fwd(Q, K, V, rp, ci, scale_of(cfg), out=o, return_lse=True)
        torch.cuda.synchronize()
        assert not torch.isnan(res[0]).any() and not torch.isnan(res[1]).any()
        outs.append((sc.clone(), rp.clone(), ci.clone(), res[0].clone(), res[1].clone()))
    for x, y in zip(*outs):
        assert torch.equal(x, y)


def _custom_inputs(L_text, L_ref, L_q, H, D, dtype, seed=3):
    g = torch.Generator().manual_seed(seed)
    L_k = L_text + L_ref + L_q
    Q = torch.randn((1, H, L_q, D), generator=g).to(dtype)
    K = torch.randn((1, H, L_k, D), generator=g).to(dtype)
    V = torch.randn((1, H, L_k, D), generator=g).to(dtype)
    return Q.to(DEV), K.to(DEV), V.to(DEV)


@pytest.mark.parametrize("L_text,L_ref,L_q,H,D,b,dtype,rho", [
    (0, 37, 200, 2, 128, 128, torch.bfloat16, 0.5),     # no text, partial blocks, 1-token-odd tail
    (100, 0, 129, 2, 128, 128, torch.bfloat16, 0.3),    # no reference; a 1-token query block
    (512, 1000, 1000, 3, 128, 128, torch.bfloat16, 0.2),
    (16, 256, 255, 2, 64, 64, torch.bfloat16, 0.5),     # float32 kernel with bf16 inputs
    (7, 100, 300, 2, 128, 128, torch.float32, 0.4),     # float32 kernel, D = b = 128
    (0, 0, 1, 1, 128, 128, torch.bfloat16, 1.0),        # a single token
])
def test_ragged_shapes(L_text, L_ref, L_q, H, D, b, dtype, rho):
    print_case("ragged", L_text, L_ref, L_q, H, D, b, dtype, rho)
    Q, K, V = _custom_inputs(L_text, L_ref, L_q, H, D, dtype)
    scale = S.Scale(L_text, L_ref, b, 1 / math.sqrt(D))
    (out, lse), (sc, rp, ci) = S.scale_forward(Q, K, V, scale, rho, out_dtype=torch.float32,
                                                 return_lse=True)
    torch.cuda.synchronize()
    lists = csr_rows(rp, ci)
    nq = O.num_blocks(L_q, b)
    for h in range(H):
        q, k, v = head_np(Q, h), head_np(K, h), head_np(V, h)
        res = O.scale_head(q, k, v, L_text, L_ref, b, 1 / math.sqrt(D), rho, rows=[])
        for i in range(nq):
            compare_row_selection(lists[h * nq + i], res["sets"][i], res["scores"][i],
                                  len(res["retained"]), res["k"])
        ref_o, ref_l = oracle_rows(q, k, v, lists[h * nq:(h + 1) * nq], range(nq), b, 1 / math.sqrt(D))
        got = to_f64(out[0, h])
        for i in range(nq):
            s, e = O.block_range(i, L_q, b)
            mx, _ = attention_errors(got[s:e], ref_o[i])
            assert mx <= (BF16_MAX_ABS if dtype == torch.bfloat16 else F32_MAX_ABS), (h, i, mx)
            assert np.max(np.abs(to_f64(lse[0, h])[s:e] - ref_l[i])) < LSE_BF16


@pytest.mark.parametrize("D,b,dtype", [(128, 128, torch.bfloat16), (128, 64, torch.bfloat16),
                                       (128, 256, torch.bfloat16), (64, 64, torch.float32)])
def test_irregular_csr(D, b, dtype):
    """Uneven block lists: empty rows, one block, every block, duplicates and
    out-of-range indices (skipped, also right after a valid entry, where the
    kernel has read the next entry ahead), rows in any order; the last key
    block is partial at every block size."""
    L_text, L_ref, L_q, H = 64, 700, 600, 2
    print_case("irregular csr", D, b, dtype)
    Q, K, V = _custom_inputs(L_text, L_ref, L_q, H, D, dtype, seed=11)
    scale = S.Scale(L_text, L_ref, b, 1 / math.sqrt(D))
    nq, nk = O.num_blocks(L_q, b), O.num_blocks(L_text + L_ref + L_q, b)
    rng = np.random.default_rng(5)
    lists = []
    for r in range(H * nq):
        kind = r % 6
        if kind == 0:
            lists.append(np.zeros(0, dtype=np.int64))
        elif kind == 1:
            lists.append(np.array([nk - 1]))
        elif kind == 2:
            lists.append(np.arange(nk)[::-1])
        elif kind == 3:
            lists.append(np.array([3, 3, 5]))
        elif kind == 4:
            lists.append(np.array([-1, 2, nk, 1000]))
        else:
            lists.append(rng.choice(nk, rng.integers(1, nk + 1), replace=False))
    rp = np.zeros(len(lists) + 1, dtype=np.int32)
    rp[1:] = np.cumsum([len(x) for x in lists])
    ci = np.concatenate(lists).astype(np.int32)
    out, lse = S.sparstar_bsa_fwd(Q, K, V, torch.from_numpy(rp).to(DEV), torch.from_numpy(ci).to(DEV),
                                  scale, out_dtype=torch.float32, return_lse=True)
    torch.cuda.synchronize()
    tol = BF16_MAX_ABS if dtype == torch.bfloat16 else F32_MAX_ABS
    for h in range(H):
        q, k, v = head_np(Q, h), head_np(K, h), head_np(V, h)
        got, got_l = to_f64(out[0, h]), to_f64(lse[0, h])
        for i in range(nq):
            s, e = O.block_range(i, L_q, b)
            blocks = [j for j in lists[h * nq + i] if 0 <= j < nk]
            if not blocks:
                assert np.all(got[s:e] == 0) and np.all(np.isneginf(got_l[s:e]))
                continue
            o_ref, l_ref, _ = O.attend_row(q[s:e], k, v, blocks, b, 1 / math.sqrt(D))
            assert np.max(np.abs(got[s:e] - o_ref)) <= tol, (h, i)
            assert np.max(np.abs(got_l[s:e] - l_ref)) < LSE_BF16


@pytest.mark.parametrize("D,b,dtype,H,L_q", [(128, 128, torch.bfloat16, 3, 1000), (128, 64, torch.bfloat16, 3, 1000),
                                             (128, 256, torch.bfloat16, 3, 1000), (64, 64, torch.float32, 3, 1000),
                                             (128, 128, torch.bfloat16, 2, 1000), (128, 256, torch.bfloat16, 4, 1000),
                                             (128, 128, torch.bfloat16, 16, 16384)])
def test_balanced_equals_plain_bitwise(D, b, dtype, H, L_q):
    """Rows started longest list first give the same outputs, bit for bit, as the plain call:
    uneven random lists plus the irregular kinds (empty, duplicates, out of range); odd head
    counts use 8 segments per head, even ones at b = 128 and 256 use 4.  The 16-head problem has
    enough rows for the persistent queues; the small ones run one workgroup per row."""
    L_text, L_ref = 64, 900
    print_case("balanced", D, b, dtype, H, L_q)
    Q, K, V = _custom_inputs(L_text, L_ref, L_q, H, D, dtype, seed=12)
    scale = S.Scale(L_text, L_ref, b, 1 / math.sqrt(D))
    nq, nk = O.num_blocks(L_q, b), O.num_blocks(L_text + L_ref + L_q, b)
    rng = np.random.default_rng(8)
    lists = []
    for r in range(H * nq):
        if r % 7 == 0:
            lists.append(np.zeros(0, dtype=np.int64))
        elif r % 7 == 1:
            lists.append(np.array([2, 2, -5, nk + 3]))
        else:
            lists.append(np.sort(rng.choice(nk, rng.integers(1, nk + 1), replace=False)))
    rp = np.zeros(len(lists) + 1, dtype=np.int32)
    rp[1:] = np.cumsum([len(x) for x in lists])
    rp_t = torch.from_numpy(rp).to(DEV)
    ci_t = torch.from_numpy(np.concatenate(lists).astype(np.int32)).to(DEV)
    a, la = S.sparstar_bsa_fwd(Q, K, V, rp_t, ci_t, scale, return_lse=True)
    nseg = 4 if b != 64 and H % 2 == 0 else 8               # segments per head
    per = -(-nq // nseg)
    ws = torch.full((64 + H * nseg * per,), -7, dtype=torch.int32, device=DEV)   # counters, then the order
    assert S.balance_workspace_bytes(S.problem(Q, K, V, scale)) == ws.numel() * 4
    c, lc = S.sparstar_bsa_fwd_balanced(Q, K, V, rp_t, ci_t, scale, return_lse=True, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, c) and torch.equal(la, lc)
    order = ws[64:].cpu().numpy().reshape(H, nseg, per)
    lens = np.diff(rp).reshape(H, nq)
    for h in range(H):
        for x in range(nseg):
            seg = order[h, x]
            blocks = list(range(x * per, min((x + 1) * per, nq)))
            got = seg[:len(blocks)]
            assert sorted(got.tolist()) == blocks and np.all(seg[len(blocks):] == -1)
            ln = lens[h, got]
            assert np.all(np.diff(ln) <= 0)                      # longest first
            for u in range(len(got) - 1):                       # stable among equal lengths
                if ln[u] == ln[u + 1]:
                    assert got[u] < got[u + 1]


@pytest.mark.parametrize("b", [64, 128, 256])
def test_static_and_dynamic_queues_bitwise(b):
    """The two ways of handing out rows (one workgroup per row without a workspace, a persistent grid
    on per-XCD atomic queues with one) compute every row the same way: equal bit for bit, on the
    selection's lists, on irregular ones (empty rows, duplicates, out-of-range entries) and dense.
    The problem has enough rows for the queues (at least two rounds of resident workgroups per XCD);
    the counters left in the workspace show which way ran: a smaller problem, with fewer rows than
    that, runs one workgroup per row even with a workspace and leaves the counters alone."""
    L_text, L_ref, L_q, H = 64, 1000, 16384, 16
    print_case("static vs dynamic queues", b)
    Q, K, V = _custom_inputs(L_text, L_ref, L_q, H, 128, torch.bfloat16, seed=21)
    scale = S.Scale(L_text, L_ref, b, 1 / math.sqrt(128))
    STALE = 12345
    ws = torch.full((64,), STALE, dtype=torch.int32, device=DEV)          # stale counters: the call sets them
    _, _, scores = S.sparstar_pool_score(Q, K, scale)
    rp, ci = S.sparstar_select_blocks(scores, Q, K, scale, 0.3)
    a, la = S.sparstar_bsa_fwd(Q, K, V, rp, ci, scale, return_lse=True, workspace=ws)
    c, lc = S.sparstar_bsa_fwd(Q, K, V, rp, ci, scale, return_lse=True, workspace=None)
    torch.cuda.synchronize()
    assert torch.equal(a, c) and torch.equal(la, lc)
    assert not torch.all(ws[:8] == STALE), "the persistent queues did not run"
    nq, nk = O.num_blocks(L_q, b), O.num_blocks(L_text + L_ref + L_q, b)
    rng = np.random.default_rng(4)
    lists = [np.zeros(0, np.int64) if r % 5 == 0 else np.array([1, 1, -3, nk]) if r % 5 == 1
             else np.sort(rng.choice(nk, rng.integers(1, nk + 1), replace=False)) for r in range(H * nq)]
    rp_np = np.zeros(len(lists) + 1, dtype=np.int32)
    rp_np[1:] = np.cumsum([len(x) for x in lists])
    rp_t = torch.from_numpy(rp_np).to(DEV)
    ci_t = torch.from_numpy(np.concatenate(lists).astype(np.int32)).to(DEV)
    ws.fill_(STALE)
    d, ld = S.sparstar_bsa_fwd(Q, K, V, rp_t, ci_t, scale, return_lse=True, workspace=ws)
    e, le = S.sparstar_bsa_fwd(Q, K, V, rp_t, ci_t, scale, return_lse=True, workspace=None)
    torch.cuda.synchronize()
    assert torch.equal(d, e) and torch.equal(ld, le)
    assert not torch.all(ws[:8] == STALE)
    # the dense path: persistent queues and one workgroup per row
    ws.fill_(-5)
    f, lf = S.dense_attn_fwd(Q, K, V, scale, return_lse=True, workspace=ws)
    g, lg = S.dense_attn_fwd(Q, K, V, scale, return_lse=True, workspace=None)
    torch.cuda.synchronize()
    assert torch.equal(f, g) and torch.equal(lf, lg)
    assert not torch.all(ws[:8] == -5)
    # too few rows for the queues: one workgroup per row, the counters untouched
    Qs, Ks, Vs = Q[:, :2, :1024].contiguous(), K[:, :2, :L_text + L_ref + 1024].contiguous(), \
        V[:, :2, :L_text + L_ref + 1024].contiguous()
    ws.fill_(STALE)
    h1 = S.dense_attn_fwd(Qs, Ks, Vs, scale, workspace=ws)
    h2 = S.dense_attn_fwd(Qs, Ks, Vs, scale, workspace=None)
    torch.cuda.synchronize()
    assert torch.equal(h1, h2) and torch.all(ws == STALE)


def test_balanced_on_the_selection():
    cfg = I.S192P
    Q, K, V = inputs(cfg)
    (out, lse), (_, rp, ci) = S.scale_forward(Q, K, V, scale_of(cfg), 0.3, return_lse=True)
    c, lc = S.sparstar_bsa_fwd_balanced(Q, K, V, rp, ci, scale_of(cfg), return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(out, c) and torch.equal(lse, lc)


@pytest.mark.parametrize("order", ["rising", "falling"])
def test_bsa_reference_max_jumps(order):
    """Key blocks whose scores sit far above those of the first block a row
    visits (by up to ~10^3 in exp2 units, enough to overflow exp2 against the
    first block's max), so the kernel must raise its reference max and rescale
    mid-row; and the mirror case where the first block holds the largest
    scores.  Output and LSE against the oracle."""
    L_text, L_ref, L_q, H, D, b = 0, 896, 256, 2, 128, 128
    print_case("max jumps", order)
    g = torch.Generator().manual_seed(23)
    L_k = L_text + L_ref + L_q
    Q = torch.randn((1, H, L_q, D), generator=g)
    K = torch.randn((1, H, L_k, D), generator=g)
    V = torch.randn((1, H, L_k, D), generator=g)
    gains = ([1.0, 1.0, 4.0, 1.0, 16.0, 2.0, 64.0, 1.0, 1.0] if order == "rising"   # per key block
             else [64.0, 16.0, 4.0, 2.0, 1.0, 1.0, 1.0, 1.0, 1.0])
    for j, gj in enumerate(gains):
        K[:, :, j * b:(j + 1) * b] *= gj
    Q, K, V = (t.to(torch.bfloat16).to(DEV) for t in (Q, K, V))
    scale = S.Scale(L_text, L_ref, b, 1 / math.sqrt(D))
    nq, nk = O.num_blocks(L_q, b), O.num_blocks(L_k, b)
    lists = [np.arange(nk) for _ in range(H * nq)]
    rp = np.zeros(len(lists) + 1, dtype=np.int32)
    rp[1:] = np.cumsum([len(x) for x in lists])
    ci = np.concatenate(lists).astype(np.int32)
    out, lse = S.sparstar_bsa_fwd(Q, K, V, torch.from_numpy(rp).to(DEV), torch.from_numpy(ci).to(DEV),
                                  scale, out_dtype=torch.float32, return_lse=True)
    torch.cuda.synchronize()
    for h in range(H):
        q, k, v = head_np(Q, h), head_np(K, h), head_np(V, h)
        got, got_l = to_f64(out[0, h]), to_f64(lse[0, h])
        for i in range(nq):
            s, e = O.block_range(i, L_q, b)
            o_ref, l_ref, _ = O.attend_row(q[s:e], k, v, list(range(nk)), b, 1 / math.sqrt(D))
            assert np.max(np.abs(got[s:e] - o_ref)) <= BF16_MAX_ABS, (h, i)
            # logits up to ~200: float32 dot products of length 128 with |k| up to ~256
            assert np.max(np.abs(got_l[s:e] - l_ref)) < 2e-2


def test_strided_views():
    """Q/K/V as views into a packed [B, L, H, D] buffer and a strided output."""
    cfg = I.TINY.with_(dtype="bf16", head_dim=128, block=128, grid=(2, 8, 16), ref_grid=(2, 8, 16))
    print_case("strided", cfg.name)
    Q, K, V = I.make_inputs(cfg, device=DEV)
    Qp = Q.transpose(1, 2).contiguous().transpose(1, 2)    # [B,H,L,D] view of [B,L,H,D] memory
    Kp = K.transpose(1, 2).contiguous().transpose(1, 2)
    Vp = V.transpose(1, 2).contiguous().transpose(1, 2)
    outp = torch.empty((1, cfg.len_q, cfg.heads, 128), dtype=torch.bfloat16, device=DEV).transpose(1, 2)
    sc = scale_of(cfg)
    ref = S.scale_forward(Q, K, V, sc, 0.5)[0]
    _, _, scs = S.sparstar_pool_score(Qp, Kp, sc)
    rp, ci = S.sparstar_select_blocks(scs, Qp, Kp, sc, 0.5)
    S.sparstar_bsa_fwd(Qp, Kp, Vp, rp, ci, sc, out=outp)
    torch.cuda.synchronize()
    assert torch.equal(outp, ref)


# ---------------------------------------------------------------- clip policies and the schedule

@pytest.mark.parametrize("name,heads", [("720p_clip1_s0", 2), ("720p_clip1_s3", 2), ("720p_clip1_s1", None),
                                        ("480p_clip1_s3", 2), ("480p_clip2_s0", 2), ("480p_clip2_s3", 4)])
def test_clip_schedule_end_to_end(name, heads):
    """A sparsified scale of a first or later clip at its density in the decreasing
    schedule.  First clip: text and image blocks retained, the current scale ranked;
    later clip: text retained, preceding clip and current scale ranked jointly.
    Selection on every row of the checked heads, attention on sampled query blocks,
    against the oracle under the same policy."""
    cfg = I.WORKLOADS[name] if heads is None else I.WORKLOADS[name].with_(heads=heads)
    rho = cfg.densities[0]
    print_case("clip schedule", cfg.name, cfg.heads, rho, cfg.policy)
    Q, K, V = inputs(cfg)
    (out, lse), (sc, rp, ci) = S.scale_forward(Q, K, V, scale_of(cfg), rho, policy=cfg.policy,
                                               return_lse=True)
    torch.cuda.synchronize()
    lists = csr_rows(rp, ci)
    b = cfg.block
    nq = O.num_blocks(cfg.len_q, b)
    R, C = O.retained_and_candidates(cfg.len_text, cfg.len_ref, cfg.len_q, b, cfg.policy)
    kk = O.budget(len(C), rho)
    assert len(R) == S.num_retained(S.problem(Q, K, V, scale_of(cfg)), cfg.policy)
    check_heads = range(cfg.heads) if heads is not None else [0, cfg.heads - 1]
    swaps = 0
    for h in check_heads:
        S_ref = O.block_scores(O.pool_blocks(head_np(Q, h), b), O.pool_blocks(head_np(K, h), b),
                               cfg.softmax_scale)
        ref_sets = O.select_blocks(S_ref, R, C, kk)
        for i in range(nq):
            swaps += compare_row_selection(lists[h * nq + i], ref_sets[i], S_ref[i], len(R), kk)
    print(f"retained {len(R)} candidates {len(C)} budget {kk}; near-tie swaps {swaps}")

    def sampler(h):
        rng = np.random.default_rng(200 + h)
        return sorted({0, nq - 1, *rng.choice(nq, 4, replace=False).tolist()})
    _check_attention(cfg, Q, K, V, lists, out, lse, list(check_heads), sampler, True)
    # the same kernel on the same lists with a float32-stored output: the plain gate
    out32 = S.sparstar_bsa_fwd(Q, K, V, rp, ci, scale_of(cfg), out_dtype=torch.float32)
    torch.cuda.synchronize()
    _check_attention(cfg, Q, K, V, lists, out32, None, list(check_heads), sampler, True)


# ---------------------------------------------------------------- block sizes 64 and 256

@pytest.mark.parametrize("name,heads,nsample", [("192p_b64", [0, 15], 12), ("192p_b256", [0, 15], None),
                                                ("tiny_f32_b256", None, None)])
def test_block_sizes_end_to_end(name, heads, nsample):
    """Block sizes of the pages' ablation beside the deployed 128: pooled scores, selection
    (near-tie rule) and attention against the oracle, and the dense path equal to a full
    block list bit for bit (bf16: the MFMA kernel at 2 and 8 wavefronts per workgroup)."""
    cfg = I.WORKLOADS[name]
    rho = cfg.densities[0]
    print_case("block size", cfg.name, cfg.block, rho)
    Q, K, V = inputs(cfg)
    sc = scale_of(cfg)
    bf16_in = cfg.dtype == "bf16"
    qp, kp, scores = S.sparstar_pool_score(Q, K, sc)
    rp, ci = S.sparstar_select_blocks(scores, Q, K, sc, rho)
    out, lse = S.sparstar_bsa_fwd(Q, K, V, rp, ci, sc, out_dtype=torch.float32, return_lse=True)
    torch.cuda.synchronize()
    b = cfg.block
    nq, nk = O.num_blocks(cfg.len_q, b), O.num_blocks(cfg.len_k, b)
    R, C = O.retained_and_candidates(cfg.len_text, cfg.len_ref, cfg.len_q, b)
    kk = O.budget(len(C), rho)
    lists = csr_rows(rp, ci)
    check_heads = range(cfg.heads) if heads is None else heads
    for h in check_heads:
        q, k = head_np(Q, h), head_np(K, h)
        qbar, kbar = O.pool_blocks(q, b), O.pool_blocks(k, b)
        S_ref = O.block_scores(qbar, kbar, cfg.softmax_scale)
        assert np.max(np.abs(to_f64(qp[0, h]) - qbar)) < 2e-6 * max(1.0, np.abs(qbar).max())
        bound = cfg.head_dim * 6e-8 * cfg.softmax_scale * (np.abs(qbar) @ np.abs(kbar).T) + 1e-7
        assert np.all(np.abs(to_f64(scores[0, h]) - S_ref) <= bound)
        ref_sets = O.select_blocks(S_ref, R, C, kk)
        for i in range(nq):
            compare_row_selection(lists[h * nq + i], ref_sets[i], S_ref[i], len(R), kk)
    sampler = None
    if nsample:
        def sampler(h):
            rng = np.random.default_rng(300 + h)
            return sorted({0, nq - 1, *rng.choice(nq, nsample, replace=False).tolist()})
    _check_attention(cfg, Q, K, V, lists, out, lse, list(check_heads), sampler, bf16_in)
    # the dense path is the sparse path over every block
    full_rp = torch.arange(0, (cfg.heads * nq + 1) * nk, nk, dtype=torch.int32, device=DEV)
    full_ci = torch.arange(nk, dtype=torch.int32, device=DEV).repeat(cfg.heads * nq)
    a = S.sparstar_bsa_fwd(Q, K, V, full_rp, full_ci, sc)
    d = S.dense_attn_fwd(Q, K, V, sc)
    torch.cuda.synchronize()
    assert torch.equal(a, d)


# ---------------------------------------------------------------- seeded random shapes

def _random_cases(n=12, seed=2024):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        b = int(rng.choice([64, 128, 256]))
        f32 = i % 4 == 3
        cases.append(dict(L_text=int(rng.integers(0, 600)), L_ref=int(rng.integers(0, 2500)),
                          L_q=int(rng.integers(1, 2500)), H=int(rng.integers(1, 4)), D=64 if f32 else 128, b=b,
                          dtype=torch.float32 if f32 else torch.bfloat16, rho=float(rng.uniform(0.05, 1.0)),
                          policy=int(rng.integers(0, 2)), seed=100 + i))
    return cases


@pytest.mark.parametrize("case", _random_cases(), ids=lambda c: f"b{c['b']}_q{c['L_q']}_p{c['policy']}")
def test_random_shapes_end_to_end(case):
    """Seeded random segment lengths, block sizes, densities and policies: selection
    (near-tie rule) and attention against the oracle, every row."""
    c = case
    print_case("random shape", c)
    Q, K, V = _custom_inputs(c["L_text"], c["L_ref"], c["L_q"], c["H"], c["D"], c["dtype"], seed=c["seed"])
    sigma = 1 / math.sqrt(c["D"])
    scale = S.Scale(c["L_text"], c["L_ref"], c["b"], sigma)
    (out, lse), (scores, rp, ci) = S.scale_forward(Q, K, V, scale, c["rho"], policy=c["policy"],
                                                   out_dtype=torch.float32, return_lse=True)
    torch.cuda.synchronize()
    b = c["b"]
    nq = O.num_blocks(c["L_q"], b)
    R, C = O.retained_and_candidates(c["L_text"], c["L_ref"], c["L_q"], b, c["policy"])
    kk = O.budget(len(C), c["rho"])
    lists = csr_rows(rp, ci)
    tol = BF16_MAX_ABS if c["dtype"] == torch.bfloat16 else F32_MAX_ABS
    for h in range(c["H"]):
        q, k, v = head_np(Q, h), head_np(K, h), head_np(V, h)
        S_ref = O.block_scores(O.pool_blocks(q, b), O.pool_blocks(k, b), sigma)
        ref_sets = O.select_blocks(S_ref, R, C, kk)
        got, got_l = to_f64(out[0, h]), to_f64(lse[0, h])
        for i in range(nq):
            compare_row_selection(lists[h * nq + i], ref_sets[i], S_ref[i], len(R), kk)
            s, e = O.block_range(i, c["L_q"], b)
            o_ref, l_ref, _ = O.attend_row(q[s:e], k, v, list(lists[h * nq + i]), b, sigma)
            assert np.max(np.abs(got[s:e] - o_ref)) <= tol, (h, i)
            assert np.max(np.abs(got_l[s:e] - l_ref)) < LSE_BF16, (h, i)


# ---------------------------------------------------------------- fused score-then-select

def _fused_equals_unfused(Q, K, sc, rho, policy):
    qp, kp, scores = S.sparstar_pool_score(Q, K, sc)
    rp, ci = S.sparstar_select_blocks(scores, Q, K, sc, rho, policy)
    qp2, kp2 = S.sparstar_pool_blocks(Q, K, sc)
    rp2, ci2 = S.sparstar_score_select(qp2, kp2, Q, K, sc, rho, policy)
    torch.cuda.synchronize()
    assert torch.equal(qp, qp2) and torch.equal(kp, kp2)
    assert torch.equal(rp, rp2)
    assert torch.equal(ci, ci2), int((ci != ci2).sum())


@pytest.mark.parametrize("name,rho", [("tiny_f32", 0.5), ("tiny_f32", 1.0), ("192p", 0.3), ("192p_b64", 0.3),
                                      ("192p_b256", 0.3), ("tiny_f32_b256", 0.5), ("480p", 0.25),
                                      ("720p_clip1_s1", None), ("480p_clip2_s3", None), ("720p", 0.2)])
def test_fused_score_select_equals_unfused_bitwise(name, rho):
    """The fused kernel forms each score with the score kernel's float32 operations and ranks
    with the same row selector: pooled blocks and block lists equal the unfused path's bit for
    bit (the unfused path is checked against the oracle elsewhere)."""
    cfg = I.WORKLOADS[name]
    rho = cfg.densities[0] if rho is None else rho
    print_case("fused select", cfg.name, rho, cfg.policy)
    Q, K, V = inputs(cfg)
    _fused_equals_unfused(Q, K, scale_of(cfg), rho, cfg.policy)


@pytest.mark.parametrize("name,heads", [("192p", None), ("480p", [0, 12, 23]), ("720p", [0, 15, 31]),
                                        ("720p_clip1_s1", [0, 31])])
def test_fused_score_select_against_oracle(name, heads):
    """The fused kernel's block lists against the oracle directly: pooled blocks within the pooling
    bound, and every row of the checked heads equal to the oracle's selection on its float64 scores
    but for near-ties (within 1e-4 relative of the row's k-th best score)."""
    cfg = I.WORKLOADS[name]
    rho = cfg.densities[0] if name != "720p" else 0.2
    print_case("fused select vs oracle", cfg.name, rho, cfg.policy)
    Q, K, V = inputs(cfg)
    sc = scale_of(cfg)
    qp, kp = S.sparstar_pool_blocks(Q, K, sc)
    rp, ci = S.sparstar_score_select(qp, kp, Q, K, sc, rho, cfg.policy)
    torch.cuda.synchronize()
    lists = csr_rows(rp, ci)
    b = cfg.block
    nq = O.num_blocks(cfg.len_q, b)
    R, C = O.retained_and_candidates(cfg.len_text, cfg.len_ref, cfg.len_q, b, cfg.policy)
    kk = O.budget(len(C), rho)
    swaps = 0
    for h in (range(cfg.heads) if heads is None else heads):
        qbar, kbar = O.pool_blocks(head_np(Q, h), b), O.pool_blocks(head_np(K, h), b)
        assert np.max(np.abs(to_f64(qp[0, h]) - qbar)) < 2e-6 * max(1.0, np.abs(qbar).max())
        assert np.max(np.abs(to_f64(kp[0, h]) - kbar)) < 2e-6 * max(1.0, np.abs(kbar).max())
        S_ref = O.block_scores(qbar, kbar, cfg.softmax_scale)
        ref_sets = O.select_blocks(S_ref, R, C, kk)
        for i in range(nq):
            swaps += compare_row_selection(lists[h * nq + i], ref_sets[i], S_ref[i], len(R), kk)
    print(f"fused selection: near-tie swaps {swaps}")


def test_fused_score_select_random_shapes():
    """The seeded random problems of the end-to-end test whose key blocks fit the fused kernel:
    equal to the unfused path bit for bit (partial strips, both policies, D = 64 and 128)."""
    n = 0
    for c in _random_cases():
        n_k = O.num_blocks(c["L_text"] + c["L_ref"] + c["L_q"], c["b"])
        if n_k > 1152:
            continue
        print_case("fused select random", c)
        Q, K, V = _custom_inputs(c["L_text"], c["L_ref"], c["L_q"], c["H"], c["D"], c["dtype"], seed=c["seed"])
        sc = S.Scale(c["L_text"], c["L_ref"], c["b"], 1 / math.sqrt(c["D"]))
        _fused_equals_unfused(Q, K, sc, c["rho"], c["policy"])
        n += 1
    assert n >= 8


# ---------------------------------------------------------------- graph capture

def test_step_captured_in_a_graph_replays_exactly():
    """The whole step (pool + score, select, attention) launches no allocation, memset or
    synchronisation, so it can be captured in a HIP graph: every replay, with eager work on
    the same buffers in between, equals the eager step bit for bit."""
    cfg = I.S192P
    sc = scale_of(cfg)
    Q, K, V = inputs(cfg)
    ref, (ref_s, ref_rp, ref_ci) = S.scale_forward(Q, K, V, sc, 0.3)
    qp, kp, scores = S.sparstar_pool_score(Q, K, sc)
    rp, ci = S.sparstar_select_blocks(scores, Q, K, sc, 0.3)
    out = torch.empty_like(Q)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        S.sparstar_pool_score(Q, K, sc, qp, kp, scores)
        S.sparstar_select_blocks(scores, Q, K, sc, 0.3, row_ptr=rp, col_idx=ci)
        S.sparstar_bsa_fwd(Q, K, V, rp, ci, sc, out=out)
    for rep in range(3):
        out.fill_(float("nan"))
        scores.zero_()
        ci.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(scores, ref_s) and torch.equal(rp, ref_rp) and torch.equal(ci, ref_ci), rep
        assert torch.equal(out, ref), rep



def test_queued_attention_captured_in_a_graph_replays_exactly():
    """The attention on the persistent grid (480p: 732 rows per XCD queue, so the atomic queues are
    used) and the balanced call, captured in one HIP graph with caller-owned workspaces: the queue
    counters are set by a kernel inside the graph, so every replay, with eager work on the same
    buffers in between, equals the eager calls bit for bit."""
    cfg = I.S480P
    sc = scale_of(cfg)
    Q, K, V = inputs(cfg)
    print_case("graph queues", cfg.name)
    _, _, scores = S.sparstar_pool_score(Q, K, sc)
    rp, ci = S.sparstar_select_blocks(scores, Q, K, sc, 0.25)
    p = S.problem(Q, K, V, sc)
    qws = torch.zeros((S.bsa_workspace_bytes(p) // 4,), dtype=torch.int32, device=DEV)
    bws = torch.zeros((S.balance_workspace_bytes(p) // 4,), dtype=torch.int32, device=DEV)
    ref, ref_lse = S.sparstar_bsa_fwd(Q, K, V, rp, ci, sc, return_lse=True, workspace=qws)
    ref_b = S.sparstar_bsa_fwd_balanced(Q, K, V, rp, ci, sc, workspace=bws)
    assert torch.equal(ref, ref_b)
    out, out_b = torch.empty_like(Q), torch.empty_like(Q)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _, lse_graph = S.sparstar_bsa_fwd(Q, K, V, rp, ci, sc, out=out, return_lse=True, workspace=qws)
        S.sparstar_bsa_fwd_balanced(Q, K, V, rp, ci, sc, out=out_b, workspace=bws)
    for rep in range(3):
        out.fill_(float("nan"))
        out_b.fill_(float("nan"))
        lse_graph.fill_(float("nan"))
        qws.fill_(-7)   # stale counters: the graph must set them itself
        bws.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref) and torch.equal(lse_graph, ref_lse), rep
        assert torch.equal(out_b, ref), rep
        # eager work on the same buffers between replays
        S.sparstar_bsa_fwd(Q, K, V, rp, ci, sc, out=out, workspace=qws)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), rep



def test_mfma_probe_runs_and_counts_its_flops():
    """The matrix-core rate probe (a measurement helper): its sink size follows the CU count, a
    launch fills every lane's value with a finite number, and its flop count is the formula's."""
    n = S.mfma_probe_sink_len()
    props = torch.cuda.get_device_properties(0)
    assert n == 2 * props.multi_processor_count * 256
    sink = torch.full((n,), float("nan"), dtype=torch.float32, device=DEV)
    flops = S.sparstar_mfma_probe(4, sink)
    torch.cuda.synchronize()
    assert torch.isfinite(sink).all()
    assert flops == 2 * props.multi_processor_count * 4 * 4 * 64 * (2 * 32 * 32 * 16)
    with pytest.raises(S.SparstarError):
        S.sparstar_mfma_probe(4, sink[: n - 1])


def test_persistent_queues_repeat_bitwise():
    """Launch after launch on the persistent grid (480p: 732 rows per XCD queue, rows handed out in
    finishing order): 100 launches reusing one workspace, each output equal to the first bit for
    bit, since every row is computed whole by one workgroup whichever workgroup pops it."""
    cfg = I.S480P
    sc = scale_of(cfg)
    Q, K, V = inputs(cfg)
    print_case("repeat queues", cfg.name)
    _, _, scores = S.sparstar_pool_score(Q, K, sc)
    rp, ci = S.sparstar_select_blocks(scores, Q, K, sc, 0.25)
    ws = torch.zeros((S.bsa_workspace_bytes(S.problem(Q, K, V, sc)) // 4,), dtype=torch.int32, device=DEV)
    ref = S.sparstar_bsa_fwd(Q, K, V, rp, ci, sc, workspace=ws)
    out = torch.empty_like(ref)
    bad = 0
    for _ in range(100):
        S.sparstar_bsa_fwd(Q, K, V, rp, ci, sc, out=out, workspace=ws)
        bad += int(not torch.equal(out, ref))
    assert bad == 0

# ---------------------------------------------------------------- full size (sampled)

_SCORES = {}


def _oracle_scores(cfg, Q, K, h):
    """Float64 oracle block scores of one head (kept across the densities of one workload)."""
    if any(key[0] != cfg.name for key in _SCORES):
        _SCORES.clear()
    if (cfg.name, h) not in _SCORES:
        b = cfg.block
        _SCORES[(cfg.name, h)] = O.block_scores(O.pool_blocks(head_np(Q, h), b), O.pool_blocks(head_np(K, h), b),
                                                cfg.softmax_scale)
    return _SCORES[(cfg.name, h)]


def _full_size_check(cfg, rho, rows_per_head, heads=None):
    """The timed launch configuration at full size, against the oracle:
    * selection on every row of every head (near-tie rule);
    * attention on `rows_per_head` query blocks of every head (first, last partial, seeded random),
      the oracle fed the GPU's own block lists, for the bf16-stored output that the benchmark times
      (max-abs beyond the store's own rounding) and for the float32-stored output of the same kernel
      on the same lists (the plain max-abs 1e-2 / mean-abs 1e-3 gate)."""
    Q, K, V = inputs(cfg)
    sc = scale_of(cfg)
    qp, kp, scores = S.sparstar_pool_score(Q, K, sc)
    rp, ci = S.sparstar_select_blocks(scores, Q, K, sc, rho, cfg.policy)
    out_bf, lse = S.sparstar_bsa_fwd(Q, K, V, rp, ci, sc, return_lse=True)
    out_f32 = S.sparstar_bsa_fwd(Q, K, V, rp, ci, sc, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert out_bf.dtype == torch.bfloat16
    lists = csr_rows(rp, ci)
    b = cfg.block
    nq = O.num_blocks(cfg.len_q, b)
    R, C = O.retained_and_candidates(cfg.len_text, cfg.len_ref, cfg.len_q, b, cfg.policy)
    kk = O.budget(len(C), rho)
    heads = range(cfg.heads) if heads is None else heads
    swaps = 0
    for h in heads:
        S_ref = _oracle_scores(cfg, Q, K, h)
        ref_sets = O.select_blocks(S_ref, R, C, kk)
        for i in range(nq):
            swaps += compare_row_selection(lists[h * nq + i], ref_sets[i], S_ref[i], len(R), kk)
    print(f"{cfg.name} rho {rho}: selection on {len(heads) * nq} rows, {swaps} near-tie swaps")

    def sampler(h):
        rng = np.random.default_rng(100 + h)
        pick = rng.choice(np.arange(1, nq - 1), rows_per_head - 2, replace=False).tolist()
        return sorted({0, nq - 1, *pick})
    mx_bf, mean_bf = _check_attention(cfg, Q, K, V, lists, out_bf, lse, list(heads), sampler, True)
    mx_32, mean_32 = _check_attention(cfg, Q, K, V, lists, out_f32, None, list(heads), sampler, True)
    print(f"{cfg.name} rho {rho}: raw max-abs bf16-stored {mx_bf:.3e} (mean {mean_bf:.3e}), "
          f"float32-stored {mx_32:.3e} (mean {mean_32:.3e})")
    return out_bf, rp, ci


@pytest.mark.slow
@pytest.mark.parametrize("rho", [0.1, 0.2, 0.4])
def test_full_size_720p(rho):
    """The 72,000-token 720p final scale at each sparse density: every head, every row's selection,
    32 heads x 16 query blocks of attention, bf16- and float32-stored output."""
    print_case("full size 720p", rho)
    _full_size_check(I.S720P, rho, 16)


@pytest.mark.slow
def test_full_size_720p_dense():
    """Density 1 at 720p: dense_attn_fwd against the oracle's plain softmax over every key
    (32 heads x 4 query blocks: first, last partial, two seeded), both output dtypes; the selection
    at density 1 lists every block, and the sparse kernel over it equals the dense one bit for bit."""
    cfg = I.S720P
    print_case("full size 720p dense")
    Q, K, V = inputs(cfg)
    sc = scale_of(cfg)
    d_bf, lse = S.dense_attn_fwd(Q, K, V, sc, return_lse=True)
    d_32 = S.dense_attn_fwd(Q, K, V, sc, out_dtype=torch.float32)
    torch.cuda.synchronize()
    nq, nk = O.num_blocks(cfg.len_q, cfg.block), O.num_blocks(cfg.len_k, cfg.block)
    lists = [np.arange(nk)] * (nq * cfg.heads)

    def sampler(h):
        rng = np.random.default_rng(7 + h)
        return sorted({0, nq - 1, *rng.choice(np.arange(1, nq - 1), 2, replace=False).tolist()})
    mx_bf, _ = _check_attention(cfg, Q, K, V, lists, d_bf, lse, range(cfg.heads), sampler, True)
    mx_32, _ = _check_attention(cfg, Q, K, V, lists, d_32, None, range(cfg.heads), sampler, True)
    print(f"dense 720p: raw max-abs bf16-stored {mx_bf:.3e}, float32-stored {mx_32:.3e}")
    _, _, scores = S.sparstar_pool_score(Q, K, sc)
    rp, ci = S.sparstar_select_blocks(scores, Q, K, sc, 1.0)
    a = S.sparstar_bsa_fwd(Q, K, V, rp, ci, sc)
    torch.cuda.synchronize()
    assert int(rp[-1]) == cfg.heads * nq * nk
    assert torch.equal(ci.view(cfg.heads * nq, nk).cpu(),
                       torch.arange(nk, dtype=torch.int32).repeat(cfg.heads * nq, 1))
    assert torch.equal(a, d_bf)


@pytest.mark.slow
@pytest.mark.parametrize("idx", [0, 1, 2, 3])
def test_full_size_sweep(idx):
    """The four scales of the 720p clip-pyramid sweep (per-scale seeds; scales 1 and 2 have their own
    partial last query and key blocks), each with fresh selection at density 0.2: every head, every
    row's selection, 32 heads x 16 query blocks of attention, both output dtypes."""
    cfg = I.SWEEP[idx]
    print_case("full size sweep", cfg.name)
    _full_size_check(cfg, 0.2, 16)


@pytest.mark.slow
@pytest.mark.parametrize("cfg", [I.S720P_B64, I.S720P_B256], ids=lambda x: x.name)
def test_full_size_block_sizes(cfg):
    """The 720p scale at the block sizes 64 and 256 of the pages' ablation: selection on every row of
    four heads, attention on 6 query blocks of each, both output dtypes."""
    print_case("full size", cfg.name)
    _full_size_check(cfg, 0.2, 6, heads=[0, 11, 20, cfg.heads - 1])
