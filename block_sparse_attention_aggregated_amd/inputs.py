"""Seeded synthetic inputs for one SparSTAR scale, and the named workloads.

This module is shared by the HIP path's tests and benchmark and by the CPU
oracle's tests.  It holds no part of the method's arithmetic: no block
partition, pooling, scoring, selection or attention.  It only draws Q, K, V.

What the inputs stand in for.  The pages measure on activations of the 8B
InfinityStar model under VBench prompts (SparSTAR full text, section 6
"Experimental Setup"); neither model nor prompts are available, so seeded
tensors of the same shapes and a comparable structure stand in for them:

* keys and values are laid out as ``[text | reference | current]``: text
  conditioning, the preceding clip's final scale, then the current-scale
  tokens, which are also the queries (SparSTAR full text, section 3
  "Spacetime Sparse Attention");
* visual tokens follow spatiotemporal raster order t*H*W + h*W + w (section 5
  "Original-order block partition");
* every element is N(0, 1), plus, on visual tokens, a smooth sinusoidal
  positional vector over normalised (t, h, w) coordinates, so that query and
  key blocks near each other in space and time score higher (a stand-in for
  the locality spacetime RoPE gives InfinityStar attention, InfinityStar
  summary page, "Approach");
* two key positions outside the text are scaled by 4 (attention sinks).

Recipe, per (batch 0, head h), with ``rng = default_rng(SeedSequence([seed, h]))``
and draws taken in this order: Q/K phase set (D uniforms on [0, 2*pi)), V
phase set (D uniforms), Q normals (L_q x D), K normals (L_k x D), V normals
(L_k x D), then the 2 sink positions (without replacement from
[L_text, L_k)).  The positional vector of a visual token at grid cell
(t, h, w) of a T x Hg x Wg grid is

    p_d = A * sin(2*pi*f_d*u_{d mod 3} + phi_d),  f_d = 1 + ((d div 3) mod 4),
    (u_0, u_1, u_2) = ((t+1/2)/T - s, (h+1/2)/Hg, (w+1/2)/Wg)

with s = 1 for the reference (preceding-clip) tokens and s = 0 for current
tokens.  bf16 workloads are rounded from float32 to bfloat16 with
round-to-nearest-even (torch's cast); the tiny workload stays float32.
"""

from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

DEFAULT_SEED = 41


@dataclass(frozen=True)
class ScaleConfig:
    """One attention scale: shapes, block size, densities and dtype."""

    name: str
    heads: int
    head_dim: int
    block: int
    grid: Tuple[int, int, int]        # current scale (T, Hg, Wg): the queries
    ref_grid: Tuple[int, int, int]    # preceding clip's final scale
    len_text: int
    densities: Tuple[float, ...]
    dtype: str                        # "bf16" or "f32" (Q, K, V)
    batch: int = 1
    seed: int = DEFAULT_SEED
    n_sinks: int = 2
    sink_gain: float = 4.0
    pos_amplitude: float = 1.0
    policy: int = 0                   # 0: later clip (text kept), 1: first clip (text + ref kept)

    @property
    def len_q(self) -> int:
        return self.grid[0] * self.grid[1] * self.grid[2]

    @property
    def len_ref(self) -> int:
        return self.ref_grid[0] * self.ref_grid[1] * self.ref_grid[2]

    @property
    def len_k(self) -> int:
        return self.len_text + self.len_ref + self.len_q

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def with_(self, **kw) -> "ScaleConfig":
        return dataclasses.replace(self, **kw)


# The five workloads.  Grids, head counts, text lengths and densities are the
# synthetic stand-ins for InfinityStar scales: 72,000 tokens is the 720p final
# scale (SparSTAR full text, section 1), 128-token blocks are the deployed
# block size (section 6 "Implementation and hardware").
TINY = ScaleConfig("tiny_f32", heads=2, head_dim=64, block=64, grid=(4, 8, 8),
                   ref_grid=(4, 8, 8), len_text=16, densities=(0.5, 1.0), dtype="f32")
S192P = ScaleConfig("192p", heads=16, head_dim=128, block=128, grid=(20, 12, 21),
                    ref_grid=(20, 12, 21), len_text=512, densities=(0.3,), dtype="bf16")
S480P = ScaleConfig("480p", heads=24, head_dim=128, block=128, grid=(20, 30, 52),
                    ref_grid=(20, 30, 52), len_text=512, densities=(0.25,), dtype="bf16")
S720P = ScaleConfig("720p", heads=32, head_dim=128, block=128, grid=(20, 45, 80),
                    ref_grid=(20, 45, 80), len_text=512, densities=(0.1, 0.2, 0.4, 1.0),
                    dtype="bf16")
SWEEP_GRIDS = ((20, 23, 40), (20, 30, 53), (20, 38, 67), (20, 45, 80))
SWEEP = tuple(
    ScaleConfig(f"720p_sweep_s{i}", heads=32, head_dim=128, block=128, grid=g,
                ref_grid=(20, 45, 80), len_text=512, densities=(0.2,), dtype="bf16",
                seed=DEFAULT_SEED + i)
    for i, g in enumerate(SWEEP_GRIDS))

# First clip of a 720p video under the pages' decreasing schedule: the four
# sparsified scales keep the text and the final image-pyramid scale
# (1 x 45 x 80 = 3,600 tokens, here in the reference segment) dense and rank the
# current-scale blocks at densities 0.625, 0.1875, 0.1875, 0.09375 (SparSTAR
# full text, section 5 "Clip-Dependent Retained and Selectable Blocks";
# appendix A.7).  The image tokens take the reference coordinates of the
# recipe below (one frame, shifted by one clip).
CLIP1_DENSITIES = (0.625, 0.1875, 0.1875, 0.09375)
CLIP1 = tuple(
    ScaleConfig(f"720p_clip1_s{i}", heads=32, head_dim=128, block=128, grid=g,
                ref_grid=(1, 45, 80), len_text=512, densities=(d,), dtype="bf16",
                seed=DEFAULT_SEED + 10 + i, policy=1)
    for i, (g, d) in enumerate(zip(SWEEP_GRIDS, CLIP1_DENSITIES)))

# Second clip of a ten-second 720p video: the same four scales as SWEEP (same
# inputs), the preceding clip's final scale ranked jointly with the current
# scale, at the same decreasing schedule (appendix A.7).
CLIP2 = tuple(c.with_(name=f"720p_clip2_s{i}", densities=(d,))
              for i, (c, d) in enumerate(zip(SWEEP, CLIP1_DENSITIES)))

# 480p: the five-second setting sparsifies the four finest scales of its one
# clip, the ten-second setting those of its second clip, whose keys hold the
# first clip's final scale (appendix A.6).  The pages' scale grids are not in
# the text; the four grids below scale the final 30 x 52 grid by the 720p
# sweep's side ratios (about 1/2, 2/3, 5/6, 1).  32 heads as in the 8B backbone
# (appendix A.5).
GRIDS_480P = ((20, 15, 26), (20, 20, 35), (20, 25, 44), (20, 30, 52))
CLIP1_480P = tuple(
    ScaleConfig(f"480p_clip1_s{i}", heads=32, head_dim=128, block=128, grid=g,
                ref_grid=(1, 30, 52), len_text=512, densities=(d,), dtype="bf16",
                seed=DEFAULT_SEED + 20 + i, policy=1)
    for i, (g, d) in enumerate(zip(GRIDS_480P, CLIP1_DENSITIES)))
CLIP2_480P = tuple(
    ScaleConfig(f"480p_clip2_s{i}", heads=32, head_dim=128, block=128, grid=g,
                ref_grid=(20, 30, 52), len_text=512, densities=(d,), dtype="bf16",
                seed=DEFAULT_SEED + 30 + i)
    for i, (g, d) in enumerate(zip(GRIDS_480P, CLIP1_DENSITIES)))

# Block-size ablation (appendix D.2 "Block-Size Ablation": 64 and 256 beside the
# deployed 128): the 192p and tiny shapes for parity, the 720p final scale at
# density 0.2 for timing.
S192P_B64 = S192P.with_(name="192p_b64", block=64)
S192P_B256 = S192P.with_(name="192p_b256", block=256)
TINY_B256 = TINY.with_(name="tiny_f32_b256", block=256)
S720P_B64 = S720P.with_(name="720p_b64", block=64, densities=(0.2,))
S720P_B256 = S720P.with_(name="720p_b256", block=256, densities=(0.2,))
BLOCK_SIZES = (S192P_B64, S192P_B256, TINY_B256, S720P_B64, S720P_B256)

WORKLOADS = {c.name: c for c in (TINY, S192P, S480P, S720P) + SWEEP + CLIP1 + CLIP2 + CLIP1_480P + CLIP2_480P
             + BLOCK_SIZES}
SEQUENCES = {"sweep": SWEEP, "clip1": CLIP1, "clip2": CLIP2, "clip1_480p": CLIP1_480P,
             "clip2_480p": CLIP2_480P}


def grid_coords(grid: Sequence[int], t_shift: float) -> np.ndarray:
    """Normalised (tau, eta, omega) of every cell of a grid, raster order, [N, 3] f64."""
    T, Hg, Wg = grid
    t = (np.arange(T, dtype=np.float64) + 0.5) / T - t_shift
    h = (np.arange(Hg, dtype=np.float64) + 0.5) / Hg
    w = (np.arange(Wg, dtype=np.float64) + 0.5) / Wg
    tt, hh, ww = np.meshgrid(t, h, w, indexing="ij")
    return np.stack([tt.ravel(), hh.ravel(), ww.ravel()], axis=1)


def positional(coords: np.ndarray, phases: np.ndarray, amplitude: float) -> np.ndarray:
    """Sinusoidal positional vectors [N, D] (float64) for coordinates [N, 3]."""
    D = phases.shape[0]
    d = np.arange(D)
    freq = 1.0 + ((d // 3) % 4)
    u = coords[:, d % 3]                                   # [N, D]
    return amplitude * np.sin(2.0 * np.pi * freq[None, :] * u + phases[None, :])


@dataclass
class HeadInputs:
    """One head's float32 draws before any dtype rounding."""

    q: np.ndarray        # [L_q, D]
    k: np.ndarray        # [L_k, D]
    v: np.ndarray        # [L_k, D]
    sinks: np.ndarray    # key positions scaled by sink_gain


def draw_head(cfg: ScaleConfig, head: int, batch: int = 0) -> HeadInputs:
    """Draw one head in float32, following the module recipe."""
    seed_words = [cfg.seed, head] if batch == 0 else [cfg.seed, head, batch]
    rng = np.random.default_rng(np.random.SeedSequence(seed_words))
    D = cfg.head_dim
    phase_qk = rng.uniform(0.0, 2.0 * np.pi, size=D)
    phase_v = rng.uniform(0.0, 2.0 * np.pi, size=D)
    q = rng.standard_normal((cfg.len_q, D), dtype=np.float32)
    k = rng.standard_normal((cfg.len_k, D), dtype=np.float32)
    v = rng.standard_normal((cfg.len_k, D), dtype=np.float32)
    sinks = rng.choice(np.arange(cfg.len_text, cfg.len_k), size=cfg.n_sinks, replace=False)

    cur = grid_coords(cfg.grid, 0.0)
    ref = grid_coords(cfg.ref_grid, 1.0)
    A = cfg.pos_amplitude
    p_cur_qk = positional(cur, phase_qk, A).astype(np.float32)
    q += p_cur_qk
    r0, r1 = cfg.len_text, cfg.len_text + cfg.len_ref
    k[r0:r1] += positional(ref, phase_qk, A).astype(np.float32)
    k[r1:] += p_cur_qk
    v[r0:r1] += positional(ref, phase_v, A).astype(np.float32)
    v[r1:] += positional(cur, phase_v, A).astype(np.float32)
    k[sinks] *= np.float32(cfg.sink_gain)
    return HeadInputs(q=q, k=k, v=v, sinks=np.sort(sinks))


def _round(x: np.ndarray, dtype: str):
    import torch
    t = torch.from_numpy(x)
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def make_inputs(cfg: ScaleConfig, device: str = "cpu", heads: Optional[Iterable[int]] = None,
                workers: int = 0):
    """Q [B,H,L_q,D], K, V [B,H,L_k,D] as torch tensors in the workload dtype.

    Heads are drawn independently (each from its own seed), ``workers``
    threads at a time (0: up to 16, bounded by the CPU count), and copied
    into the tensors as they finish, so host memory stays near ``workers``
    heads of float32 draws even at the 720p sizes.  ``heads`` restricts the
    draw to a subset (the other heads are left uninitialised).
    """
    import concurrent.futures as cf

    import torch
    tdtype = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    B, H, D = cfg.batch, cfg.heads, cfg.head_dim
    Q = torch.empty((B, H, cfg.len_q, D), dtype=tdtype, device=device)
    K = torch.empty((B, H, cfg.len_k, D), dtype=tdtype, device=device)
    V = torch.empty((B, H, cfg.len_k, D), dtype=tdtype, device=device)
    jobs = [(b, h) for b in range(B) for h in (range(H) if heads is None else heads)]
    if workers <= 0:
        import os
        workers = max(1, min(16, len(os.sched_getaffinity(0)), len(jobs)))

    def draw(job):
        b, h = job
        hi = draw_head(cfg, h, b)
        return job, [_round(x, cfg.dtype) for x in (hi.q, hi.k, hi.v)]

    with cf.ThreadPoolExecutor(workers) as ex:
        for i in range(0, len(jobs), workers):
            for (b, h), (q, k, v) in ex.map(draw, jobs[i:i + workers]):
                Q[b, h].copy_(q)
                K[b, h].copy_(k)
                V[b, h].copy_(v)
    return Q, K, V


def head_f64(cfg: ScaleConfig, head: int, batch: int = 0):
    """One head's rounded values widened to float64 numpy arrays (q, k, v)."""
    import torch
    hi = draw_head(cfg, head, batch)
    return tuple(_round(x, cfg.dtype).to(torch.float64).numpy() for x in (hi.q, hi.k, hi.v))
