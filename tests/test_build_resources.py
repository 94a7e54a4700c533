"""The compiler's per-kernel resource figures of the built library.

`build()` records, for every kernel, the registers, scratch memory and occupancy
the compiler reported. A kernel that keeps an array or spilled registers in
scratch memory pays a memory round trip whose wait also covers every load in
flight, which turns the streaming kernels latency-bound; none of them may use
scratch.
"""
import json
import os

import pytest

from mixed_precision_weight_amd import build as B

KERNELS = ("k_gemv", "k_mfv", "k_gemm_dma", "k_gemm", "k_calib_fused", "k_calib_fin", "k_topk", "k_pack",
           "k_search",
           "k_stream_read")


def _load():
    if not os.path.exists(B.RESOURCES):
        pytest.skip("library not built yet (no kernel resource record)")
    with open(B.RESOURCES) as f:
        return json.load(f)


def test_every_kernel_is_recorded():
    res = _load()
    for k in KERNELS:
        assert any(k in name for name in res), k


def test_no_kernel_uses_scratch():
    res = _load()
    bad = {n: r for n, r in res.items()
           if r.get("ScratchSize", 0) or r.get("VGPRs Spill", 0) or r.get("SGPRs Spill", 0)}
    assert not bad, bad


def test_register_budget_allows_resident_waves():
    res = _load()
    for n, r in res.items():
        assert 1 <= r["Occupancy"] <= 8, (n, r)
        assert r["VGPRs"] <= 256 and r["AGPRs"] <= 256, (n, r)


def test_exact_kernels_round_each_step():
    """The kernels whose results must equal the definition bit for bit (the
    calibration's fits and errors, the pack, the step / zero-point search) may not
    contain a mixed-precision FMA with an fp16 result: the compiler forms one from
    an fp32 multiply followed by a conversion to fp16, and it rounds the exact
    product to fp16 once instead of rounding the fp32 product."""
    import re
    import subprocess
    import tempfile
    flags = [f for f in B.COMMON if f != "-fPIC"] + ["-ffp-contract=off", "-x", "hip", "--cuda-device-only", "-S"]
    for src in sorted(B.NO_CONTRACT):
        with tempfile.NamedTemporaryFile(suffix=".s") as out:
            r = subprocess.run([B.HIPCC] + flags + ["-o", out.name, os.path.join(B.CSRC, src)],
                               capture_output=True, text=True)
            assert r.returncode == 0, r.stderr[-2000:]
            asm = open(out.name).read()
        bad = re.findall(r"v_(?:fma|mad)_mix(?:lo|hi)_f16[^\n]*", asm)
        assert not bad, (src, bad[:4])
