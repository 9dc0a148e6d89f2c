"""GPU parity of the retained-attention-mass measures against the float64 oracle.

All calls go through the C ABI.  The block mass, the token-wise bound and the
selection masses are compared with oracle/retained_mass.py on the same seeded
inputs; the selections derived from them (block oracle, window, random) go
through the same selector as the method's own and are compared bit for bit
on the same float32 inputs."""

import numpy as np
import pytest
import torch

import oracle as O
from oracle import retained_mass as RM
from block_sparse_attention_aggregated_amd import inputs as I
from block_sparse_attention_aggregated_amd import sparstar as S

from parity import csr_rows, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# Block mass: float32 exp2 of float32 logits (bf16 or float32 data) against float64, with
# the GPU's own float32 log-sum-exp: relative error of a few 1e-6 per weight.
MASS_RTOL = 1e-4
TOPK_ATOL = 1e-4


def print_case(*a):
    print("CASE", *a, flush=True)


def scale_of(cfg):
    return S.Scale(cfg.len_text, cfg.len_ref, cfg.block, cfg.softmax_scale)


def head_np(t, h):
    return to_f64(t[0, h])


def _dense_lse(cfg, Q, K, V):
    _, lse = S.dense_attn_fwd(Q, K, V, scale_of(cfg), out_dtype=torch.float32, return_lse=True)
    return lse


def _oracle_mass_row(q, k, i, cfg):
    s, e = O.block_range(i, cfg.len_q, cfg.block)
    return RM.block_mass(q[s:e], k, cfg.block, cfg.softmax_scale)[0]


@pytest.mark.parametrize("cfg,heads,rows", [(I.TINY, None, None), (I.S192P, [0, 15], None),
                                            (I.S480P, [7], [0, 1, 100, 243]), (I.S192P_B256, [3], None),
                                            (I.S192P_B64, [5], [0, 1, 40, 78])])
def test_block_mass_parity(cfg, heads, rows):
    print_case("block_mass", cfg.name)
    Q, K, V = I.make_inputs(cfg, device=DEV)
    lse = _dense_lse(cfg, Q, K, V)
    M = S.sparstar_block_mass(Q, K, lse, scale_of(cfg))
    torch.cuda.synchronize()
    nq = O.num_blocks(cfg.len_q, cfg.block)
    n_real = np.array([RM.real_queries(i, cfg.len_q, cfg.block) for i in range(nq)], dtype=np.float64)
    Mg = M.double().cpu().numpy()
    # invariant on every row of every head: each query's mass sums to 1
    assert np.allclose(Mg.sum(axis=3), n_real[None, None, :], rtol=MASS_RTOL, atol=0)
    worst = 0.0
    for h in (range(cfg.heads) if heads is None else heads):
        q, k = head_np(Q, h), head_np(K, h)
        for i in (range(nq) if rows is None else rows):
            ref = _oracle_mass_row(q, k, i, cfg)
            err = np.abs(Mg[0, h, i] - ref)
            assert np.all(err <= MASS_RTOL * ref + 1e-7 * n_real[i]), (h, i, float(err.max()))
            worst = max(worst, float((err / np.maximum(ref, 1e-30)).max()))
    print(f"worst relative error {worst:.2e}")


def test_block_mass_is_deterministic():
    cfg = I.S192P
    Q, K, V = I.make_inputs(cfg, device=DEV)
    lse = _dense_lse(cfg, Q, K, V)
    a = S.sparstar_block_mass(Q, K, lse, scale_of(cfg))
    b = S.sparstar_block_mass(Q, K, lse, scale_of(cfg))
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("cfg,rho", [(I.TINY, 0.5), (I.S192P, 0.3)])
def test_selections_and_their_mass(cfg, rho):
    """Block oracle, window and random selections through the GPU selector: bit-exact against
    the oracle's selector on the same float32 inputs; their retained masses against float64
    sums of the GPU block mass; and the ordering token bound >= block oracle >= the others."""
    print_case("selections", cfg.name, rho)
    sc = scale_of(cfg)
    Q, K, V = I.make_inputs(cfg, device=DEV)
    lse = _dense_lse(cfg, Q, K, V)
    M = S.sparstar_block_mass(Q, K, lse, sc)
    W = S.sparstar_window_scores(Q, K, sc)
    gen = torch.Generator(device=DEV).manual_seed(1234)
    Rn = torch.rand(M.shape, generator=gen, device=DEV, dtype=torch.float32)
    _, _, scores = S.sparstar_pool_score(Q, K, sc)
    sel = {name: S.sparstar_select_blocks(x, Q, K, sc, rho) for name, x in
           (("oracle", M), ("qk", scores), ("window", W), ("random", Rn))}
    masses = {name: S.sparstar_selection_mass(M, rp, ci, Q, K, sc) for name, (rp, ci) in sel.items()}
    torch.cuda.synchronize()

    b, nq, nk = cfg.block, O.num_blocks(cfg.len_q, cfg.block), O.num_blocks(cfg.len_k, cfg.block)
    R, C = O.retained_and_candidates(cfg.len_text, cfg.len_ref, cfg.len_q, b)
    kk = O.budget(len(C), rho)
    W_ref = RM.window_scores(nq, nk, cfg.len_text, cfg.len_ref, b)
    assert np.array_equal(W[0, 0].cpu().numpy(), W_ref.astype(np.float32))
    assert torch.equal(W, W[0:1, 0:1].expand_as(W))
    Mn, Rnn = M.cpu().numpy(), Rn.cpu().numpy()
    for h in range(cfg.heads):
        for name, src in (("oracle", Mn[0, h]), ("window", W_ref), ("random", Rnn[0, h])):
            ref_sets = O.select_blocks(src.astype(np.float32).astype(np.float64), R, C, kk)
            got = csr_rows(*sel[name])[h * nq:(h + 1) * nq]
            for i in range(nq):
                assert list(got[i]) == list(ref_sets[i]), (name, h, i)
        for name in sel:
            lists = csr_rows(*sel[name])[h * nq:(h + 1) * nq]
            ref = RM.selection_mass(Mn[0, h].astype(np.float64), lists, cfg.len_q, b)
            got = masses[name].cpu().numpy()[h * nq:(h + 1) * nq]
            assert np.allclose(got, ref, rtol=1e-6, atol=1e-7), name

    # ordering (per row; float32 sums of the same block masses)
    m = {n: x.cpu().numpy() for n, x in masses.items()}
    for other in ("qk", "window", "random"):
        assert np.all(m["oracle"] >= m[other] - 1e-6), other
    # token-wise bound on the first query of every block of head 0 (and the block's last real one)
    t_rows = sorted({min(i * b + off, cfg.len_q - 1) for i in range(nq) for off in (0, b - 1)})
    rows = torch.tensor(t_rows, dtype=torch.int64, device=DEV)
    tok = S.sparstar_token_topk_mass(Q, K, lse, rows, len(R) * b, kk * b, sc).cpu().numpy()
    q, k = head_np(Q, 0), head_np(K, 0)
    ref = RM.token_topk_mass(q[t_rows], k, cfg.softmax_scale, len(R) * b, kk * b)
    assert np.allclose(tok, ref, rtol=0, atol=TOPK_ATOL), float(np.abs(tok - ref).max())
    # the bound holds query by query against the per-query mass of the block oracle's blocks
    w = RM.softmax_weights(q[t_rows], k, cfg.softmax_scale)
    oracle_lists = csr_rows(*sel["oracle"])[:nq]
    for n, t in enumerate(t_rows):
        blocks = oracle_lists[t // b]
        kept = sum(w[n, j * b:min((j + 1) * b, cfg.len_k)].sum() for j in blocks)
        assert tok[n] >= kept - TOPK_ATOL
    print({n: float(x[:nq].mean()) for n, x in m.items()}, "token bound", float(tok.mean()))


def test_token_topk_edge_cases():
    """K = 0 keeps the retained tokens only; K >= candidates keeps everything (1); an index
    outside the queries gives NaN."""
    cfg = I.TINY
    sc = scale_of(cfg)
    Q, K, V = I.make_inputs(cfg, device=DEV)
    lse = _dense_lse(cfg, Q, K, V)
    rows = torch.tensor([0, 5, cfg.len_q - 1, cfg.len_q, 2 * cfg.len_q - 1, -1, 2 * cfg.len_q],
                        dtype=torch.int64, device=DEV)
    full = S.sparstar_token_topk_mass(Q, K, lse, rows, 64, 10 ** 9, sc).cpu().numpy()
    none = S.sparstar_token_topk_mass(Q, K, lse, rows, 64, 0, sc).cpu().numpy()
    assert np.allclose(full[:5], 1.0, atol=1e-5)
    assert np.all(np.isnan(full[5:])) and np.all(np.isnan(none[5:]))
    for n, qi in enumerate([0, 5, cfg.len_q - 1, cfg.len_q, 2 * cfg.len_q - 1]):
        h, t = divmod(qi, cfg.len_q)
        w = RM.softmax_weights(head_np(Q, h)[t:t + 1], head_np(K, h), cfg.softmax_scale)[0]
        assert none[n] == pytest.approx(w[:64].sum(), abs=1e-5)


@pytest.mark.slow
def test_block_mass_full_size_720p():
    """The 720p launch: every row sums to its real queries; two sampled query blocks of two
    heads against the oracle."""
    cfg = I.S720P
    print_case("block_mass full size", cfg.name)
    Q, K, V = I.make_inputs(cfg, device=DEV)
    lse = _dense_lse(cfg, Q, K, V)
    M = S.sparstar_block_mass(Q, K, lse, scale_of(cfg))
    torch.cuda.synchronize()
    nq = O.num_blocks(cfg.len_q, cfg.block)
    n_real = np.array([RM.real_queries(i, cfg.len_q, cfg.block) for i in range(nq)], dtype=np.float64)
    rs = M.sum(dim=3, dtype=torch.float64).cpu().numpy()
    assert np.allclose(rs, n_real[None, None, :], rtol=MASS_RTOL, atol=0), float(np.abs(rs / n_real - 1).max())
    for h in (0, cfg.heads - 1):
        q, k = head_np(Q, h), head_np(K, h)
        for i in (0, nq - 1):
            ref = _oracle_mass_row(q, k, i, cfg)
            got = M[0, h, i].double().cpu().numpy()
            assert np.all(np.abs(got - ref) <= MASS_RTOL * ref + 1e-7 * n_real[i]), (h, i)
