"""Pins of the retained-attention-mass oracle (oracle/retained_mass.py).

Each pin checks the oracle against something other than itself: closed
forms (row sums, constant keys, a hand-computed two-key softmax), the
optimality of the block oracle by exhaustive search, the ordering the
definitions imply (token-wise bound >= block oracle >= any other selection),
and a window geometry that can be read off by hand.  A last test plants a
mistake in each function and checks that some pin fails."""

import itertools
import math

import numpy as np
import pytest

import oracle as O
from oracle import retained_mass as RM


def _rand(L, D, seed):
    return np.random.default_rng(seed).standard_normal((L, D))


def test_block_mass_rows_sum_to_real_queries():
    """Each query's weights sum to 1, so row i sums to the real queries of block i."""
    q, k, b = _rand(200, 16, 1), _rand(437, 16, 2), 64       # partial last query and key blocks
    M = RM.block_mass(q, k, b, 0.25)
    assert M.shape == (4, 7)
    want = [64, 64, 64, 8]
    assert np.allclose(M.sum(axis=1), want, rtol=0, atol=1e-12)
    assert [RM.real_queries(i, 200, b) for i in range(4)] == want


def test_block_mass_constant_keys():
    """Identical keys: every weight is 1/L_k, so M[i, j] = n_real(i) * |B_j| / L_k."""
    q = _rand(70, 8, 3)
    k = np.tile(_rand(1, 8, 4), (100, 1))
    M = RM.block_mass(q, k, 32, 0.5)
    n_real = np.array([32, 32, 6])[:, None]
    kb = np.array([32, 32, 32, 4])[None, :]
    assert np.allclose(M, n_real * kb / 100.0, rtol=0, atol=1e-13)


def test_block_mass_two_keys_by_hand():
    """Logits 0 and ln 3 give weights 1/4 and 3/4 (softmax of two values)."""
    q = np.array([[1.0, 0.0]])
    k = np.array([[0.0, 0.0], [math.log(3.0), 0.0]])
    M = RM.block_mass(q, k, 1, 1.0)
    assert np.allclose(M, [[0.25, 0.75]], atol=1e-15)
    assert np.allclose(RM.token_topk_mass(q, k, 1.0, 0, 1), [0.75], atol=1e-15)
    assert np.allclose(RM.token_topk_mass(q, k, 1.0, 1, 0), [0.25], atol=1e-15)


def test_block_oracle_is_optimal_by_exhaustive_search():
    """No other k-subset of the candidates keeps more mass than the oracle's."""
    q, k, b = _rand(24, 8, 5), _rand(70, 8, 6) * 2.0, 8       # n_k = 9 key blocks
    M = RM.block_mass(q, k, b, 0.5)
    R, C = [0], list(range(1, 9))
    for kk in (1, 3, 5):
        sets = RM.block_oracle_sets(M, R, C, kk)
        got = RM.selection_mass(M, sets, 24, b)
        for i in range(M.shape[0]):
            best = max(sum(M[i, j] for j in R + list(sub)) for sub in itertools.combinations(C, kk))
            assert got[i] * RM.real_queries(i, 24, b) == pytest.approx(best, abs=1e-12)


def test_bound_ordering_and_full_budget():
    """token-wise Top-K >= block oracle >= aggregated-QK, window, random; all equal 1 at the
    full budget (every block, every token)."""
    L_text, L_ref, L_q, b, D = 16, 96, 90, 16, 16          # partial last query block (10)
    rng = np.random.default_rng(7)
    q, k = rng.standard_normal((L_q, D)), rng.standard_normal((L_text + L_ref + L_q, D)) * 1.5
    sigma = 0.3
    n_q, n_k = O.num_blocks(L_q, b), O.num_blocks(k.shape[0], b)
    R, C = O.retained_and_candidates(L_text, L_ref, L_q, b)
    M = RM.block_mass(q, k, b, sigma)
    for rho in (0.1, 0.3, 0.6, 1.0):
        kk = O.budget(len(C), rho)
        oracle = RM.selection_mass(M, RM.block_oracle_sets(M, R, C, kk), L_q, b)
        S = O.block_scores(O.pool_blocks(q, b), O.pool_blocks(k, b), sigma)
        qk = RM.selection_mass(M, O.select_blocks(S, R, C, kk), L_q, b)
        win = RM.selection_mass(M, O.select_blocks(RM.window_scores(n_q, n_k, L_text, L_ref, b), R, C, kk),
                                L_q, b)
        rnd = RM.selection_mass(M, O.select_blocks(rng.random((n_q, n_k)), R, C, kk), L_q, b)
        tok = np.array([RM.token_topk_mass(q[i * b:(i + 1) * b], k, sigma, len(R) * b, kk * b).mean()
                        for i in range(n_q)])
        assert np.all(tok >= oracle - 1e-12)
        for other in (qk, win, rnd):
            assert np.all(oracle >= other - 1e-12)
        if rho == 1.0:
            for x in (tok, oracle, qk, win, rnd):
                assert np.allclose(x, 1.0, atol=1e-12)


def test_token_topk_one_token_is_the_largest_candidate_weight():
    q, k = _rand(5, 8, 8), _rand(40, 8, 9)
    w = RM.softmax_weights(q, k, 0.7)
    got = RM.token_topk_mass(q, k, 0.7, 10, 1)
    assert np.allclose(got, w[:, :10].sum(1) + w[:, 10:].max(1), atol=1e-15)
    # more tokens never keep less
    assert np.all(RM.token_topk_mass(q, k, 0.7, 10, 7) >= got)


def test_window_geometry_by_hand():
    """L_text + L_ref = 3 blocks: query block i is centred on key block 3 + i, which scores 0;
    one block either way scores -b.  With k = 3 the window is {2+i, 3+i, 4+i}, clipped at the
    end of the keys (the nearest remaining block then being the lower one)."""
    b, L_text, L_ref, L_q = 8, 8, 16, 40
    n_q, n_k = O.num_blocks(L_q, b), O.num_blocks(L_text + L_ref + L_q, b)
    W = RM.window_scores(n_q, n_k, L_text, L_ref, b)
    for i in range(n_q):
        assert W[i, 3 + i] == 0.0 and W[i, 2 + i] == -b
    R, C = [0], list(range(1, n_k))
    sets = O.select_blocks(W, R, C, 3)
    assert list(sets[0]) == [0, 2, 3, 4]
    assert list(sets[n_q - 1]) == [0, 5, 6, 7]     # i = 4: 6, 7 and (5 vs none above) 5


# ---------------------------------------------------------------- planted mistakes

def _mass_pins_fail(monkeypatch, name, bad):
    monkeypatch.setattr(RM, name, bad)
    pins = [test_block_mass_rows_sum_to_real_queries, test_block_mass_constant_keys,
            test_block_mass_two_keys_by_hand, test_block_oracle_is_optimal_by_exhaustive_search,
            test_bound_ordering_and_full_budget, test_token_topk_one_token_is_the_largest_candidate_weight,
            test_window_geometry_by_hand]
    for pin in pins:
        try:
            pin()
        except Exception:
            return True
    return False


def test_planted_mass_mistakes_are_caught(monkeypatch):
    orig = {n: getattr(RM, n) for n in ("block_mass", "selection_mass", "token_topk_mass", "window_scores",
                                        "real_queries", "block_oracle_sets", "softmax_weights")}

    def mass_unnormalised(q, k, b, sigma):               # exp without the softmax denominator
        L_q, L_k = q.shape[0], k.shape[0]
        n_q, n_k = -(-L_q // b), -(-L_k // b)
        lg = sigma * (q @ k.T)
        w = np.exp(lg - lg.max(1, keepdims=True))
        return np.array([[w[i * b:(i + 1) * b, j * b:(j + 1) * b].sum() for j in range(n_k)] for i in range(n_q)])

    def mass_drops_last_key(q, k, b, sigma):             # off-by-one in the key block range
        M = orig["block_mass"](q, k[:-1], b, sigma)
        return M if M.shape[1] == -(-k.shape[0] // b) else np.pad(M, ((0, 0), (0, 1)))

    def selection_by_nominal_b(M, sets, L_q, b):         # divides a partial block by b
        return np.array([sum(M[i, j] for j in sets[i]) / b for i in range(M.shape[0])])

    def topk_smallest(q, k, sigma, keep, kt):            # wrong end of the sort
        w = orig["softmax_weights"](q, k, sigma)
        c = np.sort(w[:, keep:], axis=1)[:, :kt]
        return w[:, :keep].sum(1) + c.sum(1)

    def window_without_offset(n_q, n_k, L_text, L_ref, b):   # query centres not shifted past text+ref
        return orig["window_scores"](n_q, n_k, 0, 0, b)

    def oracle_by_smallest(M, R, C, kk):                 # wrong sign
        return orig["block_oracle_sets"](-M, R, C, kk)

    planted = [("block_mass", mass_unnormalised), ("block_mass", mass_drops_last_key),
               ("selection_mass", selection_by_nominal_b), ("token_topk_mass", topk_smallest),
               ("window_scores", window_without_offset), ("block_oracle_sets", oracle_by_smallest)]
    for name, bad in planted:
        with monkeypatch.context() as mp:
            assert _mass_pins_fail(mp, name, bad), f"planted mistake in {name} ({bad.__name__}) not caught"
