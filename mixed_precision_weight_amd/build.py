"""Build libowq.so (gfx950) in-tree with hipcc.

Every source is compiled for gfx950 only, with packed-fp32 instructions disabled
(the hardware's packed fp32 forms are avoided on these systems), and the
quantiser translation units without FMA contraction so their fp32 steps are
single IEEE operations. Objects go to ``_build/`` and the shared library to
``mixed_precision_weight_amd/libowq.so``; the compiler's per-kernel resource
figures (registers, scratch, occupancy) go to ``_build/kernel_resources.json``
and a kernel that uses scratch memory is reported.
"""
from __future__ import annotations

import concurrent.futures as cf
import json
import os
import re
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
NO_CONTRACT = {"calib.hip", "pack.hip", "grouped.hip", "search.hip", "storage.hip", "optq.hip", "backward.hip"}
RESOURCES = os.path.join(BUILD, "kernel_resources.json")
_REMARK = re.compile(r"remark: +(Function Name|TotalSGPRs|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|"
                     r"Occupancy \[waves/SIMD\]|SGPRs Spill|VGPRs Spill|LDS Size \[bytes/block\]): (\S+)")
SOURCES = ["api.cpp", "calib.hip", "topk.hip", "pack.hip", "search.hip", "storage.hip", "backward.hip", "optq.hip",
           "gemv.hip", "mfv.hip", "gemm.hip", "stream.hip", "grouped.hip"]


def _resources(stderr: str) -> dict:
    """Per-kernel register, scratch and occupancy figures from the compiler's
    kernel-resource-usage remarks."""
    out, cur = {}, None
    for line in stderr.splitlines():
        m = _REMARK.search(line)
        if not m:
            continue
        key, val = m.group(1), m.group(2)
        if key == "Function Name":
            cur = out.setdefault(val, {})
        elif cur is not None:
            cur[key.split(" [")[0]] = int(val) if val.isdigit() else val
    return out


def _compile(src: str):
    obj = os.path.join(BUILD, src + ".o")
    flags = list(COMMON)
    if src in NO_CONTRACT:
        flags.append("-ffp-contract=off")
    lang = ["-x", "hip", "-Rpass-analysis=kernel-resource-usage"] if src.endswith(".hip") else []
    cmd = [HIPCC] + flags + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    lines, skip = [], False
    for l in r.stderr.splitlines():
        if "remark:" in l:  # a remark, then the source line and caret it quotes
            skip = True
            continue
        if skip and (l.startswith(" ") or not l.strip()):
            continue
        skip = False
        if ("packed-fp32-ops" not in l and "not a recognized feature" not in l
                and "warning generated" not in l and "warnings generated" not in l):
            lines.append(l)
    if lines:
        print(f"[{src}]\n" + "\n".join(lines), file=sys.stderr)
    return obj, _resources(r.stderr)


def build() -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        done = list(ex.map(_compile, SOURCES))
    objs = [o for o, _ in done]
    res = {k: v for _, r in done for k, v in r.items()}
    with open(RESOURCES, "w") as f:
        json.dump(res, f, indent=1, sort_keys=True)
    for name, r in sorted(res.items()):
        if r.get("ScratchSize", 0) or r.get("VGPRs Spill", 0) or r.get("SGPRs Spill", 0):
            print(f"warning: kernel {name} uses scratch memory ({r.get('ScratchSize')} B/lane, "
                  f"{r.get('VGPRs Spill')} VGPR spills): its loads and stores wait on every load in flight",
                  file=sys.stderr)
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build())
