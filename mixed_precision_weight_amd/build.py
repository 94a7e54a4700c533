"""Build libowq.so (gfx950) in-tree with hipcc.

Every source is compiled for gfx950 only, with packed-fp32 instructions disabled
(the hardware's packed fp32 forms are avoided on these systems), and the
quantiser translation units without FMA contraction so their fp32 steps are
single IEEE operations. Objects go to ``_build/`` and the shared library to
``mixed_precision_weight_amd/libowq.so``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libowq.so")
BUILD = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = ["-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-Wall",
          "-fno-fast-math", "-fhip-fp32-correctly-rounded-divide-sqrt",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I" + os.path.join(ROOT, "include")]
NO_CONTRACT = {"calib.hip", "pack.hip"}
SOURCES = ["api.cpp", "calib.hip", "topk.hip", "pack.hip", "gemv.hip", "mfv.hip", "gemm.hip"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src + ".o")
    flags = list(COMMON)
    if src in NO_CONTRACT:
        flags.append("-ffp-contract=off")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC] + flags + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(l for l in r.stderr.splitlines()
                     if "packed-fp32-ops" not in l and "not a recognized feature" not in l
                     and l.strip() and "warning generated" not in l and "warnings generated" not in l)
    if warn.strip():
        print(f"[{src}]\n{warn}", file=sys.stderr)
    return obj


def build() -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build())
