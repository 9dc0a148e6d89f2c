"""Benchmark one SparSTAR scale on one MI355X.

    python bench.py [--workload 720p] [--density 0.2] [--steps K] [--warmup W]

A step is one pass of the whole hot path over one scale: sparstar_pool_score
(block means + block scores), sparstar_select_blocks (per-row top-k -> CSR)
and sparstar_bsa_fwd (block-sparse attention), on one stream, with the
inputs already resident in HBM.  Prints one JSON line:

  value        effective TFLOP/s over the executed blocks for the whole step
               (4 * |B_i| * |B_j| * D per executed block pair, real tokens;
               pooling, scoring and selection time included in the denominator)
  ms_per_step  ms per scale
  roofline     bsa_fwd (the dominant kernel) against bf16 MFMA peak, timed with
               HIP events on the stream the kernels run on
  cpu_baseline the float64 CPU oracle on a bounded sample of the same scale,
               extrapolated to the whole scale (a baseline, not a target)

--dense times dense_attn_fwd instead (the density-1 baseline); --mass measures
the retained attention mass of the selection strategies and times the
block-mass pass.  --gpus > 1 is refused: this path runs on one GPU and shards
by head with no exchange.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ms/scale and effective TFLOP/s (executed blocks) at 72k-token 720p scale"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "bsa_fwd_traffic.json")
KERNEL_SRC = os.path.join(ROOT, "block_sparse_attention_aggregated_amd", "csrc", "attn_mfma.hip")


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="720p",
                    help="720p (default), 480p, 192p, tiny_f32, sweep (four 720p-video scales of a later "
                         "clip), clip1 (the same scales of a first clip under the decreasing schedule), or "
                         "one scale by name")
    ap.add_argument("--density", type=float, default=None,
                    help="default: 0.2 at 720p and sweep, each scale's own density otherwise")
    ap.add_argument("--out-dtype", choices=("bf16", "f32"), default=None)
    ap.add_argument("--dense", action="store_true", help="time dense_attn_fwd (density 1 baseline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=16,
                    help="query blocks per head the oracle attends in its sample")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="also run a plain device copy of this many MiB (HBM counter calibration)")
    ap.add_argument("--uneven", action="store_true",
                    help="time bsa_fwd over seeded random block lists of uneven length (same mean as the "
                         "density) instead of the selection's uniform ones; the selector is not run")
    ap.add_argument("--random-even", action="store_true",
                    help="with --uneven: random lists of the selection's length for every row (the control)")
    ap.add_argument("--balanced", action="store_true",
                    help="run the attention through sparstar_bsa_fwd_balanced (rows started longest list first)")
    ap.add_argument("--longest-first", action="store_true",
                    help="with --uneven: give the longest lists to the rows the kernel dispatches first")
    ap.add_argument("--fused-select", action="store_true",
                    help="score and select in one kernel (sparstar_pool_blocks + sparstar_score_select) "
                         "instead of sparstar_pool_score + sparstar_select_blocks")
    ap.add_argument("--mass", action="store_true",
                    help="retained attention mass of the selection strategies instead (times block_mass)")
    ap.add_argument("--mass-queries", type=int, default=512,
                    help="sampled queries for the token-wise Top-K bound in --mass mode")
    ap.add_argument("--json-out", default=None)
    return ap.parse_args()


def workload_configs(name):
    from block_sparse_attention_aggregated_amd import inputs as I
    if name in I.SEQUENCES:
        return list(I.SEQUENCES[name])
    return [I.WORKLOADS[name]]


def exec_flops(cfg, row_ptr, col_idx) -> int:
    """Executed-pair FLOPs from the CSR: 4 * |B_i| * |B_j| * D over real tokens."""
    b = cfg.block
    nq = -(-cfg.len_q // b)
    nk = -(-cfg.len_k // b)
    klen = np.minimum(b, cfg.len_k - np.arange(nk) * b).astype(np.int64)
    qlen = np.minimum(b, cfg.len_q - np.arange(nq) * b).astype(np.int64)
    rp = row_ptr.cpu().numpy().astype(np.int64)
    ci = col_idx.cpu().numpy().astype(np.int64)[:rp[-1]]
    cs = np.concatenate([[0], np.cumsum(klen[ci])])
    row_keys = cs[rp[1:]] - cs[rp[:-1]]
    rows_q = np.tile(qlen, cfg.batch * cfg.heads)
    return int(4 * cfg.head_dim * np.sum(rows_q * row_keys))


def scoring_bytes(cfg) -> int:
    """Algorithmic bytes of pool_score: read Q and K once, write the pooled blocks and scores."""
    el = 2 if cfg.dtype == "bf16" else 4
    b = cfg.block
    nq, nk = -(-cfg.len_q // b), -(-cfg.len_k // b)
    BH = cfg.batch * cfg.heads
    return BH * ((cfg.len_q + cfg.len_k) * cfg.head_dim * el + (nq + nk) * cfg.head_dim * 4 + nq * nk * 4)


def traffic_record():
    """Measured HBM bytes per bsa_fwd launch, if taken on the current kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        rec = json.load(f)
    src = hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()
    return rec if rec.get("kernel_sha256") == src else None


def cpu_baseline(cfg, density, policy, Q, K, V, rows_per_head):
    """Time the float64 oracle on a bounded sample of the scale: pooling, scoring and
    selection of every head, and attention of rows_per_head query blocks per head
    (first, last and seeded random ones); the attention time is extrapolated to all
    rows by executed FLOPs.  About 10-20 s of CPU work at 720p."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = 1
    b, sigma = cfg.block, cfg.softmax_scale
    nq = O.num_blocks(cfg.len_q, b)
    rng = np.random.default_rng(0)
    t_sel = t_att = 0.0
    flops_rows = flops_all = 0
    n_rows = 0
    for bi in range(cfg.batch):
        for h in range(cfg.heads):
            q = Q[bi, h].cpu().double().numpy()
            k = K[bi, h].cpu().double().numpy()
            v = V[bi, h].cpu().double().numpy()
            t0 = time.perf_counter()
            res = O.scale_head(q, k, v, cfg.len_text, cfg.len_ref, b, sigma, density, policy, rows=[])
            t_sel += time.perf_counter() - t0
            pick = rng.choice(nq, max(0, min(nq, rows_per_head) - 2), replace=False).tolist()
            rows = sorted({0, nq - 1, *pick})[:max(rows_per_head, 1)]
            t0 = time.perf_counter()
            O.sparse_attention(q, k, v, res["sets"], b, sigma, rows=rows)
            t_att += time.perf_counter() - t0
            n_rows += len(rows)
            flops_rows += O.executed_flops(cfg.len_q, cfg.len_k, b, cfg.head_dim,
                                           [res["sets"][i] if i in rows else [] for i in range(nq)])
            flops_all += O.executed_flops(cfg.len_q, cfg.len_k, b, cfg.head_dim, res["sets"])
    t_total = t_sel + t_att * flops_all / max(flops_rows, 1)
    return {
        "value": flops_all / t_total / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
        "ms_per_scale_extrapolated": t_total * 1e3,
        "sample": (f"float64 numpy oracle on the same inputs: pooling+scoring+selection of all "
                   f"{cfg.batch * cfg.heads} heads ({t_sel:.1f} s) and attention of {n_rows} of "
                   f"{cfg.batch * cfg.heads * nq} query blocks ({rows_per_head} per head: first, last, "
                   f"seeded random; {t_att:.1f} s), attention extrapolated to all rows by executed FLOPs"),
    }


def run_mass(args):
    """Retained attention mass of the block oracle, aggregated-QK (the method), a sliding window and
    random blocks on one scale, plus the token-wise Top-K bound on sampled queries; times the block-mass
    pass (QK^T over every key, exp2 and block sums) with HIP events on its stream."""
    import torch

    from block_sparse_attention_aggregated_amd import inputs as I
    from block_sparse_attention_aggregated_amd import sparstar as S

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = workload_configs(args.workload)[-1]
    density = args.density if args.density is not None else (0.2 if args.workload == "720p" else cfg.densities[0])
    sc = S.Scale(cfg.len_text, cfg.len_ref, cfg.block, cfg.softmax_scale)
    print(f"# generating {cfg.name} inputs", file=sys.stderr, flush=True)
    Q, K, V = I.make_inputs(cfg, device=dev)
    _, lse = S.dense_attn_fwd(Q, K, V, sc, return_lse=True)
    mass = S.sparstar_block_mass(Q, K, lse, sc)
    for _ in range(args.warmup):
        S.sparstar_block_mass(Q, K, lse, sc, mass=mass)
    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    print(f"# timing {args.steps} block_mass launches", file=sys.stderr, flush=True)
    for e0, e1 in ev:
        e0.record(stream)
        S.sparstar_block_mass(Q, K, lse, sc, mass=mass)
        e1.record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    flops = 2 * cfg.batch * cfg.heads * cfg.len_q * cfg.len_k * cfg.head_dim   # Q K^T over every key

    # selections: block oracle (exact block mass), aggregated-QK, window, random
    gen = torch.Generator(device=dev).manual_seed(1234)
    rnd = torch.rand(mass.shape, generator=gen, device=dev, dtype=torch.float32)
    _, _, scores = S.sparstar_pool_score(Q, K, sc)
    window = S.sparstar_window_scores(Q, K, sc)
    res = {}
    for name, src in (("block_oracle", mass), ("aggregated_qk", scores), ("window", window), ("random", rnd)):
        rp, ci = S.sparstar_select_blocks(src, Q, K, sc, density, cfg.policy)
        res[name] = float(S.sparstar_selection_mass(mass, rp, ci, Q, K, sc).mean())
    p = S.problem(Q, K, None, sc)
    r = S.num_retained(p, cfg.policy)
    kk = S.blocks_per_row(p, density, cfg.policy) - r
    g = torch.Generator(device=dev).manual_seed(99)
    rows = torch.randint(0, cfg.batch * cfg.heads * cfg.len_q, (args.mass_queries,), generator=g, device=dev)
    tok = S.sparstar_token_topk_mass(Q, K, lse, rows, r * cfg.block, kk * cfg.block, sc)
    # the same queries under the block oracle's blocks, for the gap at matched queries
    torch.cuda.synchronize()
    res["token_topk_bound_sampled"] = float(tok.mean())
    rec = {
        "metric": "retained attention mass (mean over query blocks) and block-mass pass time",
        "value": res["aggregated_qk"], "unit": "fraction of dense softmax mass", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": cfg.name, "heads": cfg.heads, "density": density, "block": cfg.block,
                   "policy": "first clip" if cfg.policy == 1 else "later clip",
                   "token_bound_queries": args.mass_queries},
        "retained_mass": res,
        "gaps": {"blockization (token bound - block oracle)": res["token_topk_bound_sampled"] - res["block_oracle"],
                 "scoring (block oracle - aggregated QK)": res["block_oracle"] - res["aggregated_qk"]},
        "roofline": {"kernel": "sparstar_block_mass", "bound": "mfma", "achieved": flops / (ms * 1e-3) / 1e12,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, "traffic": None,
                     "flop_per_launch": flops, "exp2_per_launch": cfg.batch * cfg.heads * cfg.len_q * cfg.len_k},
    }
    line = json.dumps(rec)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")


def dispatch_order(B, H, n_q, block, xcds=8):
    """Rows in the order bsa_fwd's workgroups are numbered: with S segments per head (4 at blocks
    128 and 256 when B*H is even, else 8) and per = ceil(n_q / S), workgroup w = 8 m + x runs
    query block (x % S) * per + m % per of head (8 / S) (m // per) + x // S (a workgroup past n_q
    or past the last head exits)."""
    segments = 4 if block != 64 and (B * H) % 2 == 0 else 8
    per = -(-n_q // segments)
    at_once = xcds // segments
    order = []
    for w in range(-(-(B * H) // at_once) * per * xcds):
        m, x = divmod(w, xcds)
        hset, mm = divmod(m, per)
        bh = hset * at_once + x // segments
        qi = (x % segments) * per + mm
        if bh < B * H and qi < n_q:
            order.append(bh * n_q + qi)
    return np.array(order)


def uneven_lists(n_rows, n_k, r, k, seed=7, even=False, first=None):
    """Seeded block lists (row_ptr, col_idx as numpy int32) whose candidate counts are uniform on
    [1, 2k - 1] (mean k), or all k if `even`: the retained prefix [0, r) plus that many distinct
    random candidates of [r, n_k), ascending.  An input recipe for timing, not a selection."""
    rng = np.random.default_rng(seed)
    n_c = n_k - r
    counts = rng.integers(1, min(2 * k - 1, n_c) + 1, size=n_rows)
    if even:
        counts[:] = k
    if first is not None:          # longest lists to the rows dispatched first
        srt = np.sort(counts)[::-1]
        counts = np.empty_like(srt)
        counts[first] = srt
    keys = rng.random((n_rows, n_c), dtype=np.float32)
    rank = np.argsort(keys, axis=1)
    rows = []
    for i in range(n_rows):
        pick = np.sort(rank[i, :counts[i]]) + r
        rows.append(np.concatenate([np.arange(r), pick]))
    row_ptr = np.zeros(n_rows + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum([len(x) for x in rows])
    return row_ptr.astype(np.int32), np.concatenate(rows).astype(np.int32), counts


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the path shards by head with "
              "no exchange, so N GPUs would each run this same benchmark at H/N heads.", file=sys.stderr)
        sys.exit(2)
    if args.mass:
        run_mass(args)
        return
    import torch

    from block_sparse_attention_aggregated_amd import inputs as I
    from block_sparse_attention_aggregated_amd import sparstar as S

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfgs = workload_configs(args.workload)
    fixed = args.density if args.density is not None else (0.2 if args.workload in ("720p", "sweep") else None)
    print(f"# generating {args.workload} inputs", file=sys.stderr, flush=True)
    scales = []
    for cfg in cfgs:
        Q, K, V = I.make_inputs(cfg, device=dev)
        od = {"bf16": torch.bfloat16, "f32": torch.float32, None: Q.dtype}[args.out_dtype]
        sc = S.Scale(cfg.len_text, cfg.len_ref, cfg.block, cfg.softmax_scale)
        density = fixed if fixed is not None else cfg.densities[0]
        qp, kp, scores = S.sparstar_pool_score(Q, K, sc)
        rp, ci = S.sparstar_select_blocks(scores, Q, K, sc, density, cfg.policy)
        if args.uneven:
            p = S.problem(Q, K, None, sc)
            r = S.num_retained(p, cfg.policy)
            k = S.blocks_per_row(p, density, cfg.policy) - r
            n_rows = cfg.batch * cfg.heads * S.num_q_blocks(p)
            print(f"# drawing uneven block lists for {n_rows} rows", file=sys.stderr, flush=True)
            first = dispatch_order(cfg.batch, cfg.heads, S.num_q_blocks(p), cfg.block) if args.longest_first else None
            rp_np, ci_np, counts = uneven_lists(n_rows, S.num_k_blocks(p), r, k, even=args.random_even, first=first)
            rp, ci = torch.from_numpy(rp_np).to(dev), torch.from_numpy(ci_np).to(dev)
            print(f"# candidates per row: min {counts.min()} mean {counts.mean():.1f} max {counts.max()} "
                  f"(uniform selection: {k})", file=sys.stderr, flush=True)
        out = torch.empty(Q.shape, dtype=od, device=dev)
        ws = torch.empty((S.balance_workspace_bytes(S.problem(Q, K, None, sc)) // 4,), dtype=torch.int32, device=dev)
        scales.append(dict(cfg=cfg, Q=Q, K=K, V=V, sc=sc, qp=qp, kp=kp, scores=scores, rp=rp, ci=ci, out=out,
                           density=density, policy=cfg.policy, ws=ws))
    torch.cuda.synchronize()
    for s in scales:
        s["flops"] = (4 * s["cfg"].head_dim * s["cfg"].batch * s["cfg"].heads * s["cfg"].len_q * s["cfg"].len_k
                      if args.dense else exec_flops(s["cfg"], s["rp"], s["ci"]))
    stream = torch.cuda.current_stream(dev)

    def step(events=None):
        for n, s in enumerate(scales):
            if events is not None:
                events[n][0].record(stream)
            if args.dense:
                if events is not None:
                    events[n][1].record(stream)
                    events[n][2].record(stream)
                S.dense_attn_fwd(s["Q"], s["K"], s["V"], s["sc"], out=s["out"])
            else:
                if args.fused_select:
                    S.sparstar_pool_blocks(s["Q"], s["K"], s["sc"], s["qp"], s["kp"])
                else:
                    S.sparstar_pool_score(s["Q"], s["K"], s["sc"], s["qp"], s["kp"], s["scores"])
                if events is not None:
                    events[n][1].record(stream)
                if args.fused_select and not args.uneven:
                    S.sparstar_score_select(s["qp"], s["kp"], s["Q"], s["K"], s["sc"], s["density"], s["policy"],
                                            row_ptr=s["rp"], col_idx=s["ci"])
                elif not args.uneven:
                    S.sparstar_select_blocks(s["scores"], s["Q"], s["K"], s["sc"], s["density"], s["policy"],
                                             row_ptr=s["rp"], col_idx=s["ci"])
                if events is not None:
                    events[n][2].record(stream)
                if args.balanced:
                    S.sparstar_bsa_fwd_balanced(s["Q"], s["K"], s["V"], s["rp"], s["ci"], s["sc"], out=s["out"],
                                                workspace=s["ws"])
                else:
                    S.sparstar_bsa_fwd(s["Q"], s["K"], s["V"], s["rp"], s["ci"], s["sc"], out=s["out"])
            if events is not None:
                events[n][3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [[[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in scales] for _ in range(args.steps)]
    print(f"# timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(ev[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    per_scale = []
    for n, s in enumerate(scales):
        pool = np.array([e[n][0].elapsed_time(e[n][1]) for e in ev])
        sel = np.array([e[n][1].elapsed_time(e[n][2]) for e in ev])
        att = np.array([e[n][2].elapsed_time(e[n][3]) for e in ev])
        tot = np.array([e[n][0].elapsed_time(e[n][3]) for e in ev])
        cfg = s["cfg"]
        per_scale.append({
            "scale": cfg.name, "len_q": cfg.len_q, "len_k": cfg.len_k, "density": s["density"],
            "policy": "first clip" if s["policy"] == 1 else "later clip",
            "ms_pool_score": float(pool.mean()), "ms_select": float(sel.mean()),
            "ms_attention": float(att.mean()), "ms_attention_median": float(np.median(att)),
            "ms_scale": float(tot.mean()),
            "exec_tflop": s["flops"] / 1e12,
            "attention_tflops": s["flops"] / (att.mean() * 1e-3) / 1e12,
            "scoring_gbs": ((scoring_bytes(cfg) / (pool.mean() * 1e-3) / 1e9)
                            if not args.dense and not args.fused_select else None),
        })
    flops = sum(s["flops"] for s in scales)
    ms_step = wall * 1e3 / args.steps      # bracketed by device synchronisation
    ms_step_events = sum(p["ms_scale"] for p in per_scale)
    att_ms = sum(p["ms_attention"] for p in per_scale)
    achieved = flops / (att_ms * 1e-3) / 1e12
    traffic = traffic_record()
    cfg0 = cfgs[-1]
    rec = {
        "metric": METRIC,
        "value": flops / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg0.dtype == "bf16" else "f32",
        "data": "synthetic (seeded Gaussian + sinusoidal (t,h,w) locality + 2 sink keys; stands in for "
                "InfinityStar activations)",
        "config": {
            "workload": ("720p final scale: 72,000 queries, keys 512 text + 72,000 preceding-clip + "
                         "72,000 current" if args.workload == "720p" else args.workload),
            "heads": cfg0.heads, "head_dim": cfg0.head_dim, "block": cfg0.block,
            "density": scales[0]["density"] if len(scales) == 1 else [s["density"] for s in scales],
            "mode": ("dense" if args.dense else (("sparse, random lists of equal length" if args.random_even else
                                                  "sparse, uneven random lists") if args.uneven else "sparse"))
                    + (", balanced (longest list first)" if args.balanced else "")
                    + (", fused score-then-select" if args.fused_select else ""),
            "out_dtype": str(scales[0]["out"].dtype).replace("torch.", ""),
            "parallelism": "single GPU",
        },
        "ms_per_scale": ms_step / len(scales),
        "event_ms_per_step": ms_step_events,
        "scales": per_scale,
        "roofline": {
            "kernel": "dense_attn_fwd" if args.dense else "sparstar_bsa_fwd",
            "bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS,
            "traffic": (traffic["bytes_per_launch"] if traffic and traffic.get("workload") == args.workload
                        and len(scales) == 1 and abs(traffic.get("density", -1) - scales[0]["density"]) < 1e-12
                        and not args.dense and not args.uneven else None),
        },
    }
    if not args.dense and not args.fused_select and len(scales) == 1:
        p = per_scale[0]
        rec["scoring_roofline"] = {"kernel": "sparstar_pool_score", "bound": "hbm",
                                   "achieved": p["scoring_gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                   "frac": p["scoring_gbs"] / PEAK_HBM_GBS,
                                   "bytes": scoring_bytes(cfgs[0])}
    if args.calib_copy_mb:
        n = args.calib_copy_mb * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        rec["calib_copy_bytes"] = 2 * n * 4
    if not args.no_cpu_baseline and not args.dense and not args.uneven:
        print("# timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        s = scales[-1]
        rec["cpu_baseline"] = cpu_baseline(s["cfg"], s["density"], s["policy"], s["Q"], s["K"], s["V"],
                                           args.cpu_rows)
        print(f"# oracle sample: {rec['cpu_baseline']['sample']}", file=sys.stderr, flush=True)
    line = json.dumps(rec)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")


if __name__ == "__main__":
    main()
