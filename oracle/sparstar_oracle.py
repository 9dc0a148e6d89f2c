"""CPU oracle for one SparSTAR attention scale (test infrastructure only).

This is the slow, plain float64 reference that the HIP library is checked
against.  Only the tests, the package's smoke check and the benchmark's CPU
baseline leg may import it; the library itself never does, and this module
shares no code with the library (it imports neither the package nor its
kernels).  Inputs are numpy arrays of one (batch, head): q [L_q, D],
k [L_k, D], v [L_k, D], already rounded to the workload dtype; they are
widened to float64 here and every step runs in float64.

The steps follow "SparSTAR: Sparse Attention for SpaceTime AutoRegressive
Video Synthesis" (full text), written out from its definitions:

1. key layout  -- section 3 "Spacetime Sparse Attention": keys and values are
   text, the preceding clip's final scale, then the current-scale tokens,
   which are the queries as well; L_k = L_text + L_ref + L_q.
2. partition   -- section 5 "Original-order block partition": contiguous
   blocks of b tokens in kernel order, n = ceil(L / b), not aligned to the
   segment boundaries.
3. pooling     -- same paragraph: block means, the final partial block
   zero-padded and divided by the nominal b.
4. segment sets -- same paragraph: J_text and J_ref are the key blocks that
   intersect the text and reference token ranges.
5. score       -- section 5 "Per-head aggregated query-key score": one score
   per (query block, key block) pair, per head, from the pooled query and
   key.  The formula did not survive extraction; the reading used is the
   scaled inner product of the pooled vectors, S_ij = sigma * <qbar_i, kbar_j>.
6. policy      -- section 5 "Clip-Dependent Retained and Selectable Blocks"
   and appendix A.7 "Later-clip schedule": for clip c >= 2 the text blocks
   are retained, reference and current blocks are ranked jointly; for clip 1
   text and reference blocks are retained and only current blocks ranked.
7. budget      -- density rho applies to the ranked (candidate) blocks:
   k = ceil(rho * |C|), at least 1, at most |C|.
8. selection   -- per query block: retained set plus the k best candidates,
   ranked by score, equal scores going to the lower block index; the row's
   block list is kept in ascending order (the forward fields kv_num_blocks /
   kv_indices of section 5 "Forward-Only Sparse Execution").
9. attention   -- every query of block i attends, with a plain softmax over
   materialised logits, to the real key tokens of its selected blocks; the
   padded tail of a partial key block is not a key.  No causal mask (section
   3: every query attends to all visible keys).

Parity against the authors' implementation is unpinned: their code is not
released (appendix B.2).  The oracle's own pins are in the tests.
"""

from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np

LATER_CLIP = 0   # clip c >= 2: text retained; reference + current ranked jointly
FIRST_CLIP = 1   # clip 1: text + reference retained; current ranked


def key_length(len_text: int, len_ref: int, len_q: int) -> int:
    """Step 1: the key sequence is [text | reference | current]."""
    return len_text + len_ref + len_q


def num_blocks(length: int, b: int) -> int:
    """Step 2: n = ceil(L / b)."""
    return -(-length // b)


def block_range(j: int, length: int, b: int) -> Tuple[int, int]:
    """Step 2: token index range [start, stop) of block j."""
    return j * b, min((j + 1) * b, length)


def pool_blocks(x: np.ndarray, b: int) -> np.ndarray:
    """Step 3: block means over the nominal block length b.

    A final partial block is zero-padded, so its sum covers only the real
    tokens but is still divided by b.
    """
    x = np.asarray(x, dtype=np.float64)
    L, D = x.shape
    n = num_blocks(L, b)
    out = np.zeros((n, D), dtype=np.float64)
    for j in range(n):
        s, e = block_range(j, L, b)
        out[j] = x[s:e].sum(axis=0) / b
    return out


def block_scores(qbar: np.ndarray, kbar: np.ndarray, sigma: float) -> np.ndarray:
    """Step 5: S[i, j] = sigma * <qbar_i, kbar_j>, shape [n_q, n_k]."""
    return sigma * (np.asarray(qbar, np.float64) @ np.asarray(kbar, np.float64).T)


def intersecting_blocks(lo: int, hi: int, len_k: int, b: int) -> List[int]:
    """Step 4: {j : B_j intersects [lo, hi)} over the key blocks."""
    out = []
    for j in range(num_blocks(len_k, b)):
        s, e = block_range(j, len_k, b)
        if s < hi and lo < e and lo < hi:
            out.append(j)
    return out


def retained_and_candidates(len_text: int, len_ref: int, len_q: int, b: int,
                            policy: int = LATER_CLIP) -> Tuple[List[int], List[int]]:
    """Steps 4 and 6: the retained block set R and the ranked candidates C."""
    L_k = key_length(len_text, len_ref, len_q)
    j_text = intersecting_blocks(0, len_text, L_k, b)
    j_ref = intersecting_blocks(len_text, len_text + len_ref, L_k, b)
    if policy == LATER_CLIP:
        retained = set(j_text)
    elif policy == FIRST_CLIP:
        retained = set(j_text) | set(j_ref)
    else:
        raise ValueError(f"unknown policy {policy}")
    cands = [j for j in range(num_blocks(L_k, b)) if j not in retained]
    return sorted(retained), cands


def budget(n_candidates: int, density: float) -> int:
    """Step 7: k = clamp(ceil(rho * |C|), 1, |C|); 0 when there is nothing to rank.

    The 1e-6 guard keeps a product such as 0.2 * 1125 = 225.00000000000003
    from rounding up to 226.
    """
    if not (0.0 < density <= 1.0):
        raise ValueError("density must lie in (0, 1]")
    if n_candidates == 0:
        return 0
    return min(n_candidates, max(1, math.ceil(density * n_candidates - 1e-6)))


def select_row(scores_row: np.ndarray, retained: Sequence[int], cands: Sequence[int],
               k: int) -> np.ndarray:
    """Step 8: retained blocks plus the k best candidates, ascending block indices.

    Candidates are sorted by (-score, block index): higher scores first and,
    among exactly equal scores, the lower block index first.
    """
    c = np.asarray(cands, dtype=np.int64)
    order = np.lexsort((c, -np.asarray(scores_row, np.float64)[c]))  # primary key last
    chosen = set(int(j) for j in retained) | set(int(j) for j in c[order[:k]])
    return np.array(sorted(chosen), dtype=np.int64)


def select_blocks(scores: np.ndarray, retained: Sequence[int], cands: Sequence[int],
                  k: int) -> List[np.ndarray]:
    """Step 8 for every query block of one head."""
    return [select_row(scores[i], retained, cands, k) for i in range(scores.shape[0])]


def attend_row(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray, blocks: Sequence[int],
               b: int, sigma: float):
    """Step 9 for the queries of one block over the given key blocks.

    Returns (out [t, D], lse [t], probs [t, n_keys]) where probs are the
    softmax weights over the gathered real key tokens, in gathered order.
    """
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    L_k = k.shape[0]
    idx = np.concatenate([np.arange(*block_range(j, L_k, b)) for j in blocks]) \
        if len(blocks) else np.zeros(0, dtype=np.int64)
    logits = sigma * (np.asarray(q_rows, np.float64) @ k[idx].T)     # [t, n_keys]
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    z = e.sum(axis=1, keepdims=True)
    probs = e / z
    out = probs @ v[idx]
    lse = (m + np.log(z))[:, 0]
    return out, lse, probs


def sparse_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                     row_blocks: Sequence[Sequence[int]], b: int, sigma: float,
                     rows: Sequence[int] | None = None):
    """Step 9 for one head: O [L_q, D] and LSE [L_q] (rows not asked for stay NaN)."""
    q = np.asarray(q, np.float64)
    L_q, D = q.shape
    O = np.full((L_q, D), np.nan)
    lse = np.full((L_q,), np.nan)
    for i in (range(num_blocks(L_q, b)) if rows is None else rows):
        s, e = block_range(i, L_q, b)
        O[s:e], lse[s:e], _ = attend_row(q[s:e], k, v, row_blocks[i], b, sigma)
    return O, lse


def dense_row_blocks(len_q: int, len_k: int, b: int) -> List[np.ndarray]:
    """Every key block for every query block: the density-1 attention pattern."""
    return [np.arange(num_blocks(len_k, b))] * num_blocks(len_q, b)


def scale_head(q, k, v, len_text: int, len_ref: int, b: int, sigma: float,
               density: float, policy: int = LATER_CLIP, rows=None) -> dict:
    """Steps 1-9 for one (batch, head)."""
    L_q = q.shape[0]
    assert k.shape[0] == key_length(len_text, len_ref, L_q) == v.shape[0]
    qbar = pool_blocks(q, b)
    kbar = pool_blocks(k, b)
    S = block_scores(qbar, kbar, sigma)
    R, C = retained_and_candidates(len_text, len_ref, L_q, b, policy)
    kk = budget(len(C), density)
    sets = select_blocks(S, R, C, kk)
    O, lse = sparse_attention(q, k, v, sets, b, sigma, rows=rows)
    return dict(qbar=qbar, kbar=kbar, scores=S, retained=R, candidates=C, k=kk,
                sets=sets, out=O, lse=lse)


def executed_flops(len_q: int, len_k: int, b: int, head_dim: int, row_blocks) -> int:
    """Attention FLOPs over the executed block pairs of one head.

    Each pair (i, j) costs 2 * |B_i| * |B_j| * D for the logits and as much
    for the weighted sum of values, counting real tokens only.
    """
    tot = 0
    for i, blocks in enumerate(row_blocks):
        s, e = block_range(i, len_q, b)
        for j in blocks:
            ks, ke = block_range(j, len_k, b)
            tot += 4 * (e - s) * (ke - ks) * head_dim
    return tot
