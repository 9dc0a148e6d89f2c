"""The allocation-free entry point against the balanced call it mirrors, through the C ABI: two
calls in a row, the second on a smaller problem, each equal bit for bit to
sparstar_bsa_fwd_balanced with its own workspace (output and LSE)."""

import math

import numpy as np
import pytest
import torch

from block_sparse_attention_aggregated_amd import sparstar as S

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _problem(L_text, L_ref, L_q, H, b, seed, uneven):
    g = torch.Generator().manual_seed(seed)
    L_k = L_text + L_ref + L_q
    Q, K, V = (torch.randn((1, H, n, 128), generator=g).to(torch.bfloat16).to(DEV) for n in (L_q, L_k, L_k))
    scale = S.Scale(L_text, L_ref, b, 1 / math.sqrt(128))
    if not uneven:
        _, _, scores = S.sparstar_pool_score(Q, K, scale)
        rp, ci = S.sparstar_select_blocks(scores, Q, K, scale, 0.3)
        return Q, K, V, scale, rp, ci
    nq, nk = -(-L_q // b), -(-L_k // b)
    rng = np.random.default_rng(seed)
    lists = [np.zeros(0, np.int64) if r % 9 == 0 else np.sort(rng.choice(nk, rng.integers(1, nk + 1), replace=False))
             for r in range(H * nq)]
    rp = np.zeros(len(lists) + 1, dtype=np.int32)
    rp[1:] = np.cumsum([len(x) for x in lists])
    return (Q, K, V, scale, torch.from_numpy(rp).to(DEV),
            torch.from_numpy(np.concatenate(lists).astype(np.int32)).to(DEV))


@pytest.mark.parametrize("uneven", [False, True])
def test_noalloc_equals_balanced_on_two_calls(uneven):
    # the first problem has enough rows per XCD for the persistent queues, the second (smaller) one runs
    # one workgroup per row
    cases = [(512, 3000, 16384, 16, 128, 31), (64, 700, 900, 2, 128, 32)]
    for L_text, L_ref, L_q, H, b, seed in cases:
        print("CASE noalloc", L_text, L_ref, L_q, H, b, seed, "uneven" if uneven else "selection", flush=True)
        Q, K, V, scale, rp, ci = _problem(L_text, L_ref, L_q, H, b, seed, uneven)
        ref, ref_lse = S.sparstar_bsa_fwd_balanced(Q, K, V, rp, ci, scale, return_lse=True)
        out = torch.full_like(Q, float("nan"))
        lse = torch.full(Q.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
        S.sparstar_bsa_fwd_balanced_noalloc(Q, K, V, rp, ci, scale, out, lse)
        torch.cuda.synchronize()
        assert torch.equal(out, ref) and torch.equal(lse, ref_lse)


def test_noalloc_captured_in_a_graph_replays_exactly():
    """The callers the allocation-free entry point is for include code under HIP graph capture:
    captured once (its queues engaged: 256 rows per XCD queue), every replay, with eager calls
    of it in between, equals the balanced call with its own workspace bit for bit."""
    print("CASE noalloc graph", flush=True)
    Q, K, V, scale, rp, ci = _problem(512, 3000, 16384, 16, 128, 31, True)
    ref, ref_lse = S.sparstar_bsa_fwd_balanced(Q, K, V, rp, ci, scale, return_lse=True)
    out = torch.empty_like(Q)
    lse = torch.empty(Q.shape[:3], dtype=torch.float32, device=DEV)
    S.sparstar_bsa_fwd_balanced_noalloc(Q, K, V, rp, ci, scale, out, lse)  # first call on the device: eager
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        S.sparstar_bsa_fwd_balanced_noalloc(Q, K, V, rp, ci, scale, out, lse)
    for rep in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref) and torch.equal(lse, ref_lse), rep
        out.fill_(float("nan"))
        S.sparstar_bsa_fwd_balanced_noalloc(Q, K, V, rp, ci, scale, out, lse)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), rep
