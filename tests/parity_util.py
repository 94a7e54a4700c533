"""Shared helpers of the GPU parity tests: host<->device marshalling and the
acceptance rules (bit-exact pack, tie-tolerant weak set, per-output error bound)."""
from __future__ import annotations

import numpy as np

LIN_REL = 2e-3   # |y - y_ref| <= LIN_REL * sum_j |Wdeq_ij x_j| + LIN_ABS
LIN_ABS = 1e-5
TIE_REL = 1e-6   # weak sets may differ only across score ties within this relative gap


def dev(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def host(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def f16_bits(t) -> np.ndarray:
    return host(t).view(np.uint16)


def check_weak_set(gpu_idx: np.ndarray, ref_idx: np.ndarray, ref_score: np.ndarray):
    g = np.asarray(gpu_idx, dtype=np.int64)
    assert (np.diff(g) > 0).all(), "GPU weak indices are not strictly ascending"
    a, b = set(g.tolist()), set(np.asarray(ref_idx).tolist())
    only_g, only_r = sorted(a - b), sorted(b - a)
    assert len(only_g) == len(only_r) and len(g) == len(ref_idx)
    for i in only_g:
        for j in only_r:
            si, sj = ref_score[i], ref_score[j]
            assert abs(si - sj) <= TIE_REL * max(abs(si), abs(sj)), (
                f"weak sets differ beyond ties: gpu-only {i} ({si}), oracle-only {j} ({sj})")


def check_pack(gpu: dict, ref: dict):
    assert np.array_equal(host(gpu["qcodes"]).view(np.uint32), ref["qcodes"]), "qcodes differ"
    assert np.array_equal(f16_bits(gpu["scales"]), ref["scales"]), "scales differ"
    assert np.array_equal(host(gpu["zeros"]), ref["zeros"]), "zeros differ"
    assert np.array_equal(f16_bits(gpu["w_weak"]).reshape(ref["w_weak"].shape), ref["w_weak"]), "w_weak differ"


def check_linear(y_gpu: np.ndarray, y_ref: np.ndarray, bound: np.ndarray, what: str = ""):
    y = y_gpu.astype(np.float64)
    assert np.isfinite(y).all(), f"{what}: non-finite outputs"
    err = np.abs(y - y_ref)
    lim = LIN_REL * bound + LIN_ABS
    bad = err > lim
    if bad.any():
        i = int(np.argmax(err - lim))
        raise AssertionError(f"{what}: {int(bad.sum())} outputs out of tolerance; worst flat index {i}: "
                             f"gpu {y.ravel()[i]!r} ref {y_ref.ravel()[i]!r} bound {bound.ravel()[i]!r}")
    return float(np.max(err / np.maximum(lim, 1e-300)))
