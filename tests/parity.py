"""Helpers for the GPU-vs-oracle parity tests (not a test module).

Comparison rules:
* selection: the per-row counts must be equal; in each row the listed blocks
  must equal the oracle's, except for candidate swaps a (GPU only) / b (oracle
  only) whose oracle scores lie within 1e-4 relative of the row's k-th best
  oracle candidate score (a near-tie the float32 GPU scores may order
  differently from the float64 oracle);
* attention: max-abs and mean-abs error over the real query rows; bf16 inputs
  1e-2 / 1e-3, float32 inputs 1e-5 max-abs.  A bf16-stored output carries, on
  top of the kernel's error, the rounding of the store itself (up to half a
  bf16 spacing, 1.6e-2 for values in [4, 8)); for it the max-abs bound is
  1e-2 plus that half spacing, element by element.  The float32-stored output
  of the same kernel is held to the plain bounds.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle as O

TIE_REL = 1e-4
BF16_MAX_ABS, BF16_MEAN_ABS = 1e-2, 1e-3
F32_MAX_ABS = 1e-5


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def csr_rows(row_ptr: torch.Tensor, col_idx: torch.Tensor):
    rp = row_ptr.cpu().numpy().astype(np.int64)
    ci = col_idx.cpu().numpy().astype(np.int64)
    return [ci[rp[r]:rp[r + 1]] for r in range(len(rp) - 1)]


def compare_row_selection(gpu: np.ndarray, ref: np.ndarray, scores_row: np.ndarray, n_keep: int,
                          k: int) -> int:
    """Number of tie-swapped candidates; raises AssertionError on a real mismatch."""
    assert len(gpu) == len(ref), (len(gpu), len(ref))
    assert np.all(np.diff(gpu) > 0), "GPU row not strictly ascending"
    assert list(gpu[:n_keep]) == list(range(n_keep)), "retained prefix missing"
    g, o = set(gpu.tolist()), set(ref.tolist())
    extra, missing = g - o, o - g
    if not extra and not missing:
        return 0
    cands = np.arange(n_keep, len(scores_row))
    s_sorted = np.sort(scores_row[cands])[::-1]
    s_k = s_sorted[k - 1]
    for j in extra | missing:
        assert j >= n_keep
        tol = TIE_REL * max(abs(scores_row[j]), abs(s_k))
        assert abs(scores_row[j] - s_k) < tol, \
            f"block {j}: score {scores_row[j]!r} vs k-th {s_k!r} is not a near-tie"
    return len(extra)


def attention_errors(gpu_out: np.ndarray, ref_out: np.ndarray):
    d = np.abs(gpu_out - ref_out)
    return float(d.max()), float(d.mean())


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half the spacing of bfloat16 numbers at |x|: the most a correct rounding to bf16 moves x."""
    _, e = np.frexp(np.abs(x))          # |x| = m * 2**e with m in [0.5, 1)
    return np.where(x == 0, 0.0, np.ldexp(1.0, e - 9))


def excess_over_bf16_store(gpu_out: np.ndarray, ref_out: np.ndarray) -> float:
    """Largest error left after allowing for the final rounding of the output to bf16."""
    return float(np.max(np.abs(gpu_out - ref_out) - bf16_half_ulp(ref_out)))


def oracle_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, row_lists, rows, b: int, sigma: float):
    """Oracle attention (out, lse) for the given query-block rows of one head."""
    outs, lses = {}, {}
    for i in rows:
        s, e = O.block_range(i, q.shape[0], b)
        blocks = [j for j in row_lists[i] if 0 <= j < O.num_blocks(k.shape[0], b)]
        outs[i], lses[i], _ = O.attend_row(q[s:e], k, v, blocks, b, sigma)
    return outs, lses
