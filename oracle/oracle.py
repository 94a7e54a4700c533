"""ctypes binding of ``liboracle.so`` (see ``owq_oracle.c`` for the arithmetic).

TEST INFRASTRUCTURE: used only by the test-suite, the smoke check and the
benchmark's CPU-baseline leg.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "owq_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32


def build(force: bool = True) -> str:
    """Compile the oracle with gcc: -O2, no FMA contraction, no fast-math."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-fPIC", "-shared", "-Wall", "-Wextra", "-o", _LIB + ".tmp", _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build(force=True)
    lib = ctypes.CDLL(_LIB)
    sig = {
        "owq_oracle_f16_to_f64": (ctypes.c_double, [ctypes.c_uint16]),
        "owq_oracle_f32_to_f16": (ctypes.c_uint16, [ctypes.c_float]),
        "owq_oracle_qparams": (None, [_P, _P, _I64, _P, _P]),
        "owq_oracle_code": (ctypes.c_int, [ctypes.c_uint16, ctypes.c_uint16, ctypes.c_uint8]),
        "owq_oracle_hessian_diag": (None, [_P, _I64, _I64, _P]),
        "owq_oracle_rtn_col_err": (None, [_P, _I64, _I64, _P]),
        "owq_oracle_calibrate_score": (None, [_P, _I64, _I64, _P, _I64, _P, _P]),
        "owq_oracle_select_weak": (None, [_P, _I64, _I32, _P]),
        "owq_oracle_pack": (None, [_P, _I64, _I64, _P, _I32, _P, _P, _P, _P]),
        "owq_oracle_search_qparams": (None, [_P, _P, _I64, _P, ctypes.c_int, ctypes.c_int, _P, _P]),
        "owq_oracle_pack_search": (None, [_P, _I64, _I64, _P, _I32, _P, ctypes.c_int, ctypes.c_int,
                                          _P, _P, _P, _P, ctypes.c_int]),
        "owq_oracle_pack_storage": (None, [_P, _I64, _I64, _P, _I32, _P, _P, _P, _P]),
        "owq_oracle_linear_storage_rows": (None, [_P, _P, _P, _I64, _I64, _P, _P, _I32,
                                                  _P, _I64, _P, _I64, _P, _P, ctypes.c_int]),
        "owq_oracle_linear_backward": (None, [_P, _P, _P, _I64, _I64, _P, _P, _I32, _P, _P, _I64,
                                              _P, _P, _P, _P, ctypes.c_int]),
        "owq_oracle_f64_to_f16": (ctypes.c_uint16, [ctypes.c_double]),
        "owq_oracle_optq_factor": (None, [_P, _I64, _I64, _P, _I32, _P, ctypes.c_int]),
        "owq_oracle_optq_pack": (None, [_P, _I64, _I64, _P, _I32, _P, _P, _P, _P, _P, ctypes.c_int]),
        "owq_oracle_unpack_codes": (None, [_P, _I64, _I64, _P]),
        "owq_oracle_linear_pairs": (None, [_P, _P, _P, _I64, _I64, _P, _P, _I32,
                                           _P, _I64, _P, _P, _I64, _P, _P]),
        "owq_oracle_linear_rows": (None, [_P, _P, _P, _I64, _I64, _P, _P, _I32,
                                          _P, _I64, _P, _I64, _P, _P, ctypes.c_int]),
        "owq_oracle_effective_bits": (ctypes.c_double, [_I64, _I64, ctypes.c_int]),
        "owq_oracle_pack_grouped": (None, [_P, _I64, _I64, _P, _I32, _I64, _P, _P, _P, _P]),
        "owq_oracle_linear_grouped_rows": (None, [_P, _P, _P, _I64, _I64, _I64, _P, _P, _I32,
                                                  _P, _I64, _P, _I64, _P, _P, ctypes.c_int]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def _u16(a) -> np.ndarray:
    """fp16 array (or raw uint16 bits) -> contiguous uint16 bit patterns."""
    a = np.asarray(a)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    assert a.dtype == np.uint16, a.dtype
    return np.ascontiguousarray(a)


def f16_to_f64(h: int) -> float:
    return load().owq_oracle_f16_to_f64(int(h) & 0xFFFF)


def f32_to_f16(f: float) -> int:
    return load().owq_oracle_f32_to_f16(float(np.float32(f)))


def qparams(row, use=None):
    """(s16 bits, z) of one row; ``use`` is an optional boolean column mask."""
    row = _u16(row)
    use_a = None if use is None else np.ascontiguousarray(np.asarray(use, dtype=np.uint8))
    s = np.zeros(1, np.uint16)
    z = np.zeros(1, np.uint8)
    load().owq_oracle_qparams(_ptr(row), _ptr(use_a), row.shape[-1], _ptr(s), _ptr(z))
    return int(s[0]), int(z[0])


def code(w_bits: int, s16: int, z: int) -> int:
    return load().owq_oracle_code(int(w_bits) & 0xFFFF, int(s16) & 0xFFFF, int(z))


def hessian_diag(X) -> np.ndarray:
    X = _u16(X)
    T, K = X.shape
    lam = np.zeros(K, np.float64)
    load().owq_oracle_hessian_diag(_ptr(X), T, K, _ptr(lam))
    return lam


def rtn_col_err(W) -> np.ndarray:
    W = _u16(W)
    N, K = W.shape
    e = np.zeros(K, np.float64)
    load().owq_oracle_rtn_col_err(_ptr(W), N, K, _ptr(e))
    return e


def calibrate_score(W, X):
    W = _u16(W)
    X = _u16(X)
    N, K = W.shape
    T, K2 = X.shape
    assert K == K2
    lam = np.zeros(K, np.float64)
    score = np.zeros(K, np.float64)
    load().owq_oracle_calibrate_score(_ptr(W), N, K, _ptr(X), T, _ptr(lam), _ptr(score))
    return lam, score


def select_weak(score, k: int) -> np.ndarray:
    score = np.ascontiguousarray(np.asarray(score, dtype=np.float64))
    K = score.shape[0]
    assert 0 <= k <= K
    idx = np.zeros(max(k, 1), np.int32)
    load().owq_oracle_select_weak(_ptr(score), K, int(k), _ptr(idx))
    return idx[:k].copy()


def pack(W, weak_idx):
    """Returns dict(qcodes uint32[N][K/32][3], scales uint16[N], zeros uint8[N],
    w_weak uint16[N][k], weak_idx int32[k])."""
    W = _u16(W)
    N, K = W.shape
    assert K % 32 == 0
    idx = np.ascontiguousarray(np.asarray(weak_idx, dtype=np.int32))
    k = idx.shape[0]
    q = np.zeros((N, K // 32, 3), np.uint32)
    s = np.zeros(N, np.uint16)
    z = np.zeros(N, np.uint8)
    ww = np.zeros((N, max(k, 1)), np.uint16)
    load().owq_oracle_pack(_ptr(W), N, K, _ptr(idx) if k else None, k,
                           _ptr(q), _ptr(s), _ptr(z), _ptr(ww))
    return {"qcodes": q, "scales": s, "zeros": z,
            "w_weak": np.ascontiguousarray(ww[:, :k]), "weak_idx": idx}


SEARCH_STEPS = 32  # step factors 1 - a/40, a = 0..31 (1 down to 0.225), of the truncation-aware grid


def search_qparams(row, use=None, lam=None, steps: int = SEARCH_STEPS, zsearch: bool = True):
    """(s16 bits, z) of one row from the truncation-aware grid search."""
    row = _u16(row)
    use_a = None if use is None else np.ascontiguousarray(np.asarray(use, dtype=np.uint8))
    lam_a = None if lam is None else np.ascontiguousarray(np.asarray(lam, dtype=np.float64))
    s = np.zeros(1, np.uint16)
    z = np.zeros(1, np.uint8)
    load().owq_oracle_search_qparams(_ptr(row), _ptr(use_a), row.shape[-1], _ptr(lam_a), int(steps),
                                     1 if zsearch else 0, _ptr(s), _ptr(z))
    return int(s[0]), int(z[0])


def pack_search(W, weak_idx, lam=None, steps: int = SEARCH_STEPS, zsearch: bool = True, threads: int = 0):
    """pack() with each row's step and zero point from the truncation-aware grid
    search (optionally weighted by lam, fp64 [K]); rows over OpenMP threads."""
    W = _u16(W)
    N, K = W.shape
    assert K % 32 == 0
    idx = np.ascontiguousarray(np.asarray(weak_idx, dtype=np.int32))
    k = idx.shape[0]
    lam_a = None if lam is None else np.ascontiguousarray(np.asarray(lam, dtype=np.float64))
    assert lam_a is None or lam_a.shape == (K,)
    q = np.zeros((N, K // 32, 3), np.uint32)
    s = np.zeros(N, np.uint16)
    z = np.zeros(N, np.uint8)
    ww = np.zeros((N, max(k, 1)), np.uint16)
    load().owq_oracle_pack_search(_ptr(W), N, K, _ptr(idx) if k else None, k, _ptr(lam_a), int(steps),
                                  1 if zsearch else 0, _ptr(q), _ptr(s), _ptr(z), _ptr(ww), int(threads))
    return {"qcodes": q, "scales": s, "zeros": z,
            "w_weak": np.ascontiguousarray(ww[:, :k]), "weak_idx": idx}


def pack_storage(W, weak_idx):
    """Storage-favoured form: qcodes uint32 [N][ceil((K-k)/32)][3] of the dense
    columns only, scales, zeros, w_weak, weak_idx (as pack())."""
    W = _u16(W)
    N, K = W.shape
    assert K % 32 == 0
    idx = np.ascontiguousarray(np.asarray(weak_idx, dtype=np.int32))
    k = idx.shape[0]
    Gd = (K - k + 31) // 32
    q = np.zeros((N, max(Gd, 1), 3), np.uint32)
    s = np.zeros(N, np.uint16)
    z = np.zeros(N, np.uint8)
    ww = np.zeros((N, max(k, 1)), np.uint16)
    load().owq_oracle_pack_storage(_ptr(W), N, K, _ptr(idx) if k else None, k, _ptr(q), _ptr(s), _ptr(z), _ptr(ww))
    return {"qcodes": np.ascontiguousarray(q[:, :Gd]), "scales": s, "zeros": z,
            "w_weak": np.ascontiguousarray(ww[:, :k]), "weak_idx": idx, "K": K}


def linear_storage_rows(layer: dict, x, rows=None, threads: int = 0):
    """fp64 y and bound [M][len(rows)] of the storage-favoured product (x: [M][K])."""
    K = int(layer["K"])
    q = np.ascontiguousarray(layer["qcodes"], dtype=np.uint32)
    s = _u16(layer["scales"])
    z = np.ascontiguousarray(layer["zeros"], dtype=np.uint8)
    idx = np.ascontiguousarray(layer["weak_idx"], dtype=np.int32)
    ww = _u16(layer["w_weak"])
    x = _u16(x)
    if x.ndim == 1:
        x = x[None, :]
    M = x.shape[0]
    assert x.shape[1] == K
    N = s.shape[0]
    k = idx.shape[0]
    assert q.shape[1] == (K - k + 31) // 32
    rows = np.arange(N, dtype=np.int64) if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    R = rows.shape[0]
    y = np.zeros((M, R), np.float64)
    b = np.zeros((M, R), np.float64)
    qq = q if q.size else np.zeros((N, 1, 3), np.uint32)
    load().owq_oracle_linear_storage_rows(_ptr(qq), _ptr(s), _ptr(z), N, K, _ptr(idx) if k else None,
                                          _ptr(ww) if k else None, k, _ptr(x), M, _ptr(rows), R, _ptr(y), _ptr(b),
                                          int(threads))
    return y, b


def linear_backward(layer: dict, x, dy, want_dx: bool = True, want_dw: bool = True, threads: int = 0):
    """fp64 (dx [M][K], dx_bound, dw_weak [N][k], dw_bound) of the weak-column-tuning
    backward for upstream gradient dy [M][N] (fp16) and input x [M][K] (fp16)."""
    q = np.ascontiguousarray(layer["qcodes"], dtype=np.uint32)
    s = _u16(layer["scales"])
    z = np.ascontiguousarray(layer["zeros"], dtype=np.uint8)
    idx = np.ascontiguousarray(layer["weak_idx"], dtype=np.int32)
    ww = _u16(layer["w_weak"])
    x = _u16(x)
    dy = _u16(dy)
    if x.ndim == 1:
        x = x[None, :]
    if dy.ndim == 1:
        dy = dy[None, :]
    M, K = x.shape
    N = q.shape[0]
    assert q.shape[1] * 32 == K and dy.shape == (M, N)
    k = idx.shape[0]
    dx = np.zeros((M, K), np.float64) if want_dx else None
    dxb = np.zeros((M, K), np.float64) if want_dx else None
    dw = np.zeros((N, max(k, 1)), np.float64) if want_dw else None
    dwb = np.zeros((N, max(k, 1)), np.float64) if want_dw else None
    load().owq_oracle_linear_backward(_ptr(q), _ptr(s), _ptr(z), N, K, _ptr(idx) if k else None,
                                      _ptr(ww) if k else None, k, _ptr(x), _ptr(dy), M, _ptr(dx), _ptr(dxb),
                                      _ptr(dw), _ptr(dwb), int(threads))
    if want_dw:
        dw, dwb = np.ascontiguousarray(dw[:, :k]), np.ascontiguousarray(dwb[:, :k])
    return dx, dxb, dw, dwb


def f64_to_f16(f: float) -> int:
    return load().owq_oracle_f64_to_f16(float(f))


def optq_factor(X, weak_idx, threads: int = 0) -> np.ndarray:
    """U [K][K] (upper) of the damped Hessian 2 X^T X in dense-then-weak order."""
    X = _u16(X)
    T, K = X.shape
    idx = np.ascontiguousarray(np.asarray(weak_idx, dtype=np.int32))
    U = np.zeros((K, K), np.float64)
    load().owq_oracle_optq_factor(_ptr(X), T, K, _ptr(idx) if idx.size else None, idx.shape[0], _ptr(U), int(threads))
    return U


def optq_pack(W, X, weak_idx, U=None, threads: int = 0) -> dict:
    """Latency-favoured pack of W with OPTQ's sequential quantisation, the weak
    columns last (U from optq_factor(X, weak_idx) unless given)."""
    W = _u16(W)
    N, K = W.shape
    assert K % 32 == 0
    idx = np.ascontiguousarray(np.asarray(weak_idx, dtype=np.int32))
    k = idx.shape[0]
    if U is None:
        U = optq_factor(X, idx, threads)
    U = np.ascontiguousarray(U, dtype=np.float64)
    q = np.zeros((N, K // 32, 3), np.uint32)
    s = np.zeros(N, np.uint16)
    z = np.zeros(N, np.uint8)
    ww = np.zeros((N, max(k, 1)), np.uint16)
    load().owq_oracle_optq_pack(_ptr(W), N, K, _ptr(idx) if k else None, k, _ptr(U), _ptr(q), _ptr(s), _ptr(z),
                                _ptr(ww), int(threads))
    return {"qcodes": q, "scales": s, "zeros": z, "w_weak": np.ascontiguousarray(ww[:, :k]), "weak_idx": idx}


def unpack_codes(qcodes, K: int) -> np.ndarray:
    q = np.ascontiguousarray(np.asarray(qcodes, dtype=np.uint32))
    N = q.shape[0]
    out = np.zeros((N, K), np.uint8)
    load().owq_oracle_unpack_codes(_ptr(q), N, K, _ptr(out))
    return out


def linear_pairs(layer: dict, x, pm, pi):
    """fp64 y and error bound for the (token pm[p], row pi[p]) pairs."""
    q = np.ascontiguousarray(layer["qcodes"], dtype=np.uint32)
    s = _u16(layer["scales"])
    z = np.ascontiguousarray(layer["zeros"], dtype=np.uint8)
    idx = np.ascontiguousarray(layer["weak_idx"], dtype=np.int32)
    ww = _u16(layer["w_weak"])
    x = _u16(x)
    if x.ndim == 1:
        x = x[None, :]
    M, K = x.shape
    N = q.shape[0]
    assert q.shape[1] * 32 == K
    k = idx.shape[0]
    pm = np.ascontiguousarray(np.asarray(pm, dtype=np.int64))
    pi = np.ascontiguousarray(np.asarray(pi, dtype=np.int64))
    assert pm.shape == pi.shape
    assert (pm >= 0).all() and (pm < M).all() and (pi >= 0).all() and (pi < N).all()
    P = pm.shape[0]
    y = np.zeros(P, np.float64)
    b = np.zeros(P, np.float64)
    load().owq_oracle_linear_pairs(_ptr(q), _ptr(s), _ptr(z), N, K,
                                   _ptr(idx) if k else None, _ptr(ww) if k else None, k,
                                   _ptr(x), M, _ptr(pm), _ptr(pi), P, _ptr(y), _ptr(b))
    return y, b


def linear_full(layer: dict, x):
    """All M x N outputs (small cases): y[M][N] and bound[M][N] in fp64."""
    x = _u16(x)
    if x.ndim == 1:
        x = x[None, :]
    M = x.shape[0]
    N = layer["qcodes"].shape[0]
    mm, ii = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    y, b = linear_pairs(layer, x, mm.ravel(), ii.ravel())
    return y.reshape(M, N), b.reshape(M, N)


def linear_rows(layer: dict, x, rows=None, threads: int = 0):
    """fp64 y and bound [M][len(rows)] for every token of the listed rows (all
    rows if None), rows spread over OpenMP threads (0: all). Bit-identical to
    linear_pairs on the same (token, row)."""
    q = np.ascontiguousarray(layer["qcodes"], dtype=np.uint32)
    s = _u16(layer["scales"])
    z = np.ascontiguousarray(layer["zeros"], dtype=np.uint8)
    idx = np.ascontiguousarray(layer["weak_idx"], dtype=np.int32)
    ww = _u16(layer["w_weak"])
    x = _u16(x)
    if x.ndim == 1:
        x = x[None, :]
    M, K = x.shape
    N = q.shape[0]
    assert q.shape[1] * 32 == K
    k = idx.shape[0]
    rows = np.arange(N, dtype=np.int64) if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    assert rows.ndim == 1 and (rows >= 0).all() and (rows < N).all()
    R = rows.shape[0]
    y = np.zeros((M, R), np.float64)
    b = np.zeros((M, R), np.float64)
    load().owq_oracle_linear_rows(_ptr(q), _ptr(s), _ptr(z), N, K,
                                  _ptr(idx) if k else None, _ptr(ww) if k else None, k,
                                  _ptr(x), M, _ptr(rows), R, _ptr(y), _ptr(b), int(threads))
    return y, b


def effective_bits(K: int, k: int, latency_favored: bool) -> float:
    return load().owq_oracle_effective_bits(int(K), int(k), 1 if latency_favored else 0)


def pack_grouped(W, weak_idx, G: int):
    """Group-wise form: dict(qcodes uint32[N][K/32][3], scales uint16[N][K/G],
    zeros uint8[N][K/G], w_weak uint16[N][k], weak_idx int32[k], group G)."""
    W = _u16(W)
    N, K = W.shape
    assert K % 32 == 0 and G % 32 == 0 and G > 0 and K % G == 0
    idx = np.ascontiguousarray(np.asarray(weak_idx, dtype=np.int32))
    k = idx.shape[0]
    q = np.zeros((N, K // 32, 3), np.uint32)
    s = np.zeros((N, K // G), np.uint16)
    z = np.zeros((N, K // G), np.uint8)
    ww = np.zeros((N, max(k, 1)), np.uint16)
    load().owq_oracle_pack_grouped(_ptr(W), N, K, _ptr(idx) if k else None, k, int(G),
                                   _ptr(q), _ptr(s), _ptr(z), _ptr(ww))
    return {"qcodes": q, "scales": s, "zeros": z,
            "w_weak": np.ascontiguousarray(ww[:, :k]), "weak_idx": idx, "group": int(G)}


def linear_grouped_rows(layer: dict, x, rows=None, threads: int = 0):
    """fp64 y and bound [M][len(rows)] of the group-wise form (all rows if None)."""
    q = np.ascontiguousarray(layer["qcodes"], dtype=np.uint32)
    s = _u16(layer["scales"])
    z = np.ascontiguousarray(layer["zeros"], dtype=np.uint8)
    idx = np.ascontiguousarray(layer["weak_idx"], dtype=np.int32)
    ww = _u16(layer["w_weak"])
    G = int(layer["group"])
    x = _u16(x)
    if x.ndim == 1:
        x = x[None, :]
    M, K = x.shape
    N = q.shape[0]
    assert q.shape[1] * 32 == K and s.shape == (N, K // G) and z.shape == (N, K // G)
    k = idx.shape[0]
    rows = np.arange(N, dtype=np.int64) if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    assert rows.ndim == 1 and (rows >= 0).all() and (rows < N).all()
    R = rows.shape[0]
    y = np.zeros((M, R), np.float64)
    b = np.zeros((M, R), np.float64)
    load().owq_oracle_linear_grouped_rows(_ptr(q), _ptr(s), _ptr(z), N, K, G,
                                          _ptr(idx) if k else None, _ptr(ww) if k else None, k,
                                          _ptr(x), M, _ptr(rows), R, _ptr(y), _ptr(b), int(threads))
    return y, b
