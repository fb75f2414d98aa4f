"""Builds libh3k.so in-tree from the HIP sources in csrc/ with hipcc for gfx950.

Usage: python -m video_diffusion_transformer_03_amd.build   (or build() from Python)
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
OUT = os.path.join(HERE, "libh3k.so")
SOURCES = ["h3k_api.hip", "k_rows.hip", "k_gemm.hip", "k_attn.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fno-gpu-rdc",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wno-unused-result",
]
# Per-source flags. Attention takes row maxima of matrix-core results, which the compiler
# would otherwise quiet (a self-max per value, against signalling NaNs) before each max;
# its inputs are finite and -inf is still honoured.
# The GEMM epilogues are shared by two GEMM kernels whose results must agree bit for bit;
# contraction of a * b + c into one rounding is decided per source expression (not by the
# backend, where the choice can depend on the surrounding kernel).
EXTRA = {"k_attn.hip": ["-fno-honor-nans"], "k_gemm.hip": ["-ffp-contract=on"]}


def _compile(src: str, build_dir: str) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-6000:]}")
    return obj


def build(verbose: bool = True) -> str:
    build_dir = os.path.join(ROOT, "_build")
    os.makedirs(build_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir), SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-4000:]}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}", file=sys.stderr)
    return OUT


if __name__ == "__main__":
    build()
