"""CPU oracle for retained attention mass (test infrastructure only).

The quality proxy of "SparSTAR: Sparse Attention for SpaceTime
AutoRegressive Video Synthesis" (full text), section 4 "Analysis"
("Cross-Scale Pattern Consistency within a Clip", Figure 3; "Pattern
Persistence across Clip Boundaries") and section 1 (the gap to the token-wise
upper bound split into a blockization and a scoring term): the share of each
query's dense softmax mass that a key selection keeps.  Same rules as the
main oracle module: float64 throughout, one (batch, head) at a time, only the
tests, the smoke check and the benchmark's CPU leg use it, and it shares no
code with the library.

Definitions written out here (the pages name the measures but print no
formula; the readings are the plainest ones):

* weights    w_ts = softmax over all L_k real keys of sigma * q_t.k_s (the
               dense attention of query t).
* block mass M[i, j] = sum over the real queries t of query block i and the
               real keys s of key block j of w_ts.  Each query's weights sum
               to 1, so row i of M sums to the number of real queries of
               block i.
* retained mass of a selection (a block list per query block): the mean over
               the real queries of block i of the mass on the listed blocks,
               sum_{j in A_i} M[i, j] / n_real(i).
* exact block oracle: the retained blocks plus the k candidates of largest
               M[i, j] (equal masses to the lower index).  Mass is additive
               over blocks, so no other k-candidate set keeps more.
* token-wise Top-K bound: per query, the mass of the retained blocks' tokens
               plus the k*b largest candidate-token weights: no selection of k
               candidate blocks (at most k*b tokens) keeps more.
* sliding window: the k candidates whose centres lie closest, in key-sequence
               position, to the query block's centre (the current-scale tokens
               are keys L_text + L_ref + t), equal distances to the lower index.
* random blocks: the k candidates with the largest of a given array of
               uniform random numbers (the random numbers are an input).
"""

from __future__ import annotations

from typing import Sequence

import numpy as np

from .sparstar_oracle import block_range, num_blocks, select_blocks


def softmax_weights(q_rows: np.ndarray, k: np.ndarray, sigma: float) -> np.ndarray:
    """Dense attention weights [n, L_k] of the queries q_rows [n, D] over every key."""
    logits = sigma * (np.asarray(q_rows, np.float64) @ np.asarray(k, np.float64).T)
    logits -= logits.max(axis=1, keepdims=True)
    w = np.exp(logits)
    return w / w.sum(axis=1, keepdims=True)


def block_mass(q: np.ndarray, k: np.ndarray, b: int, sigma: float) -> np.ndarray:
    """M[i, j]: dense softmax mass of the real queries of block i on the real keys of block j."""
    L_q, L_k = q.shape[0], k.shape[0]
    n_q, n_k = num_blocks(L_q, b), num_blocks(L_k, b)
    M = np.zeros((n_q, n_k), dtype=np.float64)
    for i in range(n_q):
        s, e = block_range(i, L_q, b)
        w = softmax_weights(q[s:e], k, sigma).sum(axis=0)       # [L_k], summed over the block's queries
        for j in range(n_k):
            ks, ke = block_range(j, L_k, b)
            M[i, j] = w[ks:ke].sum()
    return M


def real_queries(i: int, len_q: int, b: int) -> int:
    s, e = block_range(i, len_q, b)
    return e - s


def selection_mass(M: np.ndarray, sets: Sequence[Sequence[int]], len_q: int, b: int) -> np.ndarray:
    """Mean retained mass per query block of the block lists `sets` (entries counted as listed)."""
    return np.array([sum(M[i, j] for j in sets[i]) / real_queries(i, len_q, b) for i in range(M.shape[0])])


def block_oracle_sets(M: np.ndarray, retained: Sequence[int], cands: Sequence[int], k: int):
    """Retained blocks plus the k candidates of largest exact block mass."""
    return select_blocks(M, retained, cands, k)


def token_topk_mass(q_rows: np.ndarray, k: np.ndarray, sigma: float, keep_tokens: int,
                    k_tokens: int) -> np.ndarray:
    """Per query: mass of the key tokens [0, keep_tokens) plus the k_tokens largest
    weights among the key tokens [keep_tokens, L_k)."""
    w = softmax_weights(q_rows, k, sigma)
    L_k = w.shape[1]
    keep = min(keep_tokens, L_k)
    cand = w[:, keep:]
    kt = min(k_tokens, cand.shape[1])
    top = np.sort(cand, axis=1)[:, cand.shape[1] - kt:] if kt > 0 else np.zeros((w.shape[0], 0))
    return w[:, :keep].sum(axis=1) + top.sum(axis=1)


def window_scores(n_q: int, n_k: int, len_text: int, len_ref: int, b: int) -> np.ndarray:
    """Minus the distance between block centres in key-sequence position: key block j is
    centred at j*b + b/2, query block i at len_text + len_ref + i*b + b/2."""
    i = np.arange(n_q, dtype=np.float64)[:, None]
    j = np.arange(n_k, dtype=np.float64)[None, :]
    return -np.abs((j * b + b / 2) - (len_text + len_ref + i * b + b / 2))
