"""Build libbitlinear.so (gfx950) in-tree with hipcc.

    python -m ternary_weight_lm_amd.build

Compiles every source under csrc/ for --offload-arch=gfx950 and links the
shared library next to this file, where the binding loads it.  No GPU is
needed: hipcc cross-compiles.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libbitlinear.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["pack.hip", "actquant.hip", "gemm.hip", "skinny.hip", "decode.hip", "decode_f32.hip",
           "decode_f16.hip", "decode_bf16.hip", "chain.hip", "gate.hip", "mlgru.hip", "capi.cpp"]

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    # correctly rounded fp32 division / sqrt are relied on; no fused
    # multiply-add contraction anywhere in the quantizers
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    # never emit packed fp32 ALU ops on this hardware
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # scalar kernel arguments arrive preloaded in SGPRs (gfx950 kernel-
    # argument preloading; the code object keeps a fallback that loads them)
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
