"""Build libsparstar.so (gfx950) in-tree with hipcc.

    python -m block_sparse_attention_aggregated_amd.build [--jobs N]

Every HIP source is compiled for gfx950 only, with packed-FP32 instruction
selection turned off, then linked into a shared library next to this file.
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsparstar.so")

SOURCES = ["host.cpp", "pool_score.hip", "select.hip", "score_select.hip", "attn_mfma.hip", "attn_simt.hip", "mass.hip",
           "balance.hip", "mfma_probe.hip"]
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          f"-I{INCLUDE}", f"-I{CSRC}"]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Per-source extra flags.  The attention kernel assumes NaN-free scores so that its
# row max is plain v_max3 (IEEE-mode fmax would first quiet every operand).
EXTRA = {"attn_mfma.hip": ["-fno-honor-nans"]}


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    lang = ["-x", "hip"]
    cmd = [hipcc(), *lang, *COMMON, *DEVICE, *EXTRA.get(src, []), "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # hipcc's host pass does not know the packed-fp32 feature and says so; keep other warnings
    for line in (r.stderr or "").splitlines():
        if "packed-fp32-ops" not in line and "warning" in line:
            print(line, file=sys.stderr)
    return obj


def build(jobs: int = 0, verbose: bool = True) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1, 8)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *DEVICE, "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=0)
    build(ap.parse_args().jobs)
