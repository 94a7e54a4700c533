"""ctypes binding of libowq.so (the C ABI in include/owq.h).

Argument marshalling only: every step runs in the library's HIP kernels. Torch
provides device memory and the current stream. fp16 tensors are handed over as
their IEEE binary16 bit patterns. A missing library is an error: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libowq.so")

OWQ_OK = 0
STATUS = {0: "OWQ_OK", 1: "OWQ_ERR_NULL", 2: "OWQ_ERR_SHAPE", 3: "OWQ_ERR_RANGE", 4: "OWQ_ERR_ALIGN",
          5: "OWQ_ERR_UNSUPPORTED", 6: "OWQ_ERR_WORKSPACE", 7: "OWQ_ERR_HIP"}

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32


class OwqLayer(ctypes.Structure):
    """Mirror of ``owq_layer`` (host struct, device pointers)."""
    _fields_ = [("N", ctypes.c_int64), ("K", ctypes.c_int64), ("k", ctypes.c_int32),
                ("bits", ctypes.c_int32), ("qcodes", _P), ("scales", _P), ("zeros", _P),
                ("weak_idx", _P), ("w_weak", _P)]


EXPORTS = {
    "owq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "owq_last_error": (ctypes.c_char_p, []),
    "owq_calibrate_workspace_bytes": (ctypes.c_size_t, [_I64, _I64, _I64]),
    "owq_calibrate_score": (ctypes.c_int, [_P, _I64, _I64, _P, _I64, _P, _P, _P, ctypes.c_size_t, _P]),
    "owq_select_weak": (ctypes.c_int, [_P, _I64, _I32, _P, _P]),
    "owq_pack": (ctypes.c_int, [_P, _I64, _I64, _P, _I32, _P, _P, _P, _P, _P]),
    "owq_linear": (ctypes.c_int, [ctypes.POINTER(OwqLayer), _P, _I64, _P, _P]),
    "owq_linear_batched": (ctypes.c_int, [ctypes.POINTER(OwqLayer), ctypes.POINTER(_P),
                                          ctypes.POINTER(_P), _I32, _I64, _P]),
    "owq_stream_read_sink_words": (_I64, [_I64]),
    "owq_stream_read": (ctypes.c_int, [_P, _I64, _P, _I64, _P]),
}

_lib = None


class OwqError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: {STATUS.get(status, status)}: {detail}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Open libowq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise FileNotFoundError(
                f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def _check(status: int, where: str):
    if status != OWQ_OK:
        raise OwqError(status, where, lib().owq_last_error().decode())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t: torch.Tensor, dtype, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


# ------------------------------------------------------------------ calibration


def calibrate_workspace_bytes(N: int, K: int, T: int) -> int:
    return int(lib().owq_calibrate_workspace_bytes(N, K, T))


def calibrate(W: torch.Tensor, X: torch.Tensor, workspace: torch.Tensor | None = None, stream=None):
    """lambda (fp64 [K]) and score (fp64 [K]) of fp16 W [N][K] and X [T][K]."""
    _dev(W, torch.float16, "W")
    _dev(X, torch.float16, "X")
    N, K = W.shape
    T = X.shape[0]
    nbytes = calibrate_workspace_bytes(N, K, T)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=W.device)
    lam = torch.empty(K, dtype=torch.float64, device=W.device)
    score = torch.empty(K, dtype=torch.float64, device=W.device)
    _check(lib().owq_calibrate_score(_ptr(W), N, K, _ptr(X), T, _ptr(lam), _ptr(score), _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), _stream(stream)),
           "owq_calibrate_score")
    return lam, score


def select_weak(score: torch.Tensor, k: int, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Indices of the k largest scores, ascending (int32 [k]); written to out if given."""
    _dev(score, torch.float64, "score")
    if out is None:
        out = torch.empty(max(k, 1), dtype=torch.int32, device=score.device)
    else:
        _dev(out, torch.int32, "out")
        if out.numel() < k:
            raise ValueError(f"out holds {out.numel()} indices, k = {k}")
    _check(lib().owq_select_weak(_ptr(score), score.numel(), int(k), _ptr(out) if k else None,
                                 _stream(stream)), "owq_select_weak")
    return out[:k]


# ------------------------------------------------------------------------ pack


def pack(W: torch.Tensor, weak_idx: torch.Tensor, out: dict | None = None, stream=None) -> dict:
    """Latency-favoured packed layer: dict of device tensors
    qcodes int32 [N][K/32][3] (uint32 bits), scales fp16 [N], zeros uint8 [N],
    w_weak fp16 [N][k], weak_idx int32 [k]."""
    _dev(W, torch.float16, "W")
    _dev(weak_idx, torch.int32, "weak_idx")
    N, K = W.shape
    k = weak_idx.numel()
    dev = W.device
    if out is None:
        out = {"qcodes": torch.empty((N, K // 32, 3), dtype=torch.int32, device=dev),
               "scales": torch.empty(N, dtype=torch.float16, device=dev),
               "zeros": torch.empty(N, dtype=torch.uint8, device=dev),
               "w_weak": torch.empty((N, k), dtype=torch.float16, device=dev)}
    out["weak_idx"] = weak_idx
    _check(lib().owq_pack(_ptr(W), N, K, _ptr(weak_idx) if k else None, k, _ptr(out["qcodes"]),
                          _ptr(out["scales"]), _ptr(out["zeros"]), _ptr(out["w_weak"]) if k else None,
                          _stream(stream)), "owq_pack")
    return out


# ---------------------------------------------------------------------- linear


def layer_struct(layer: dict) -> OwqLayer:
    q = layer["qcodes"]
    N, G = q.shape[0], q.shape[1]
    k = layer["weak_idx"].numel()
    return OwqLayer(N, G * 32, k, 3, q.data_ptr(), layer["scales"].data_ptr(), layer["zeros"].data_ptr(),
                    layer["weak_idx"].data_ptr() if k else None, layer["w_weak"].data_ptr() if k else None)


def linear(layer: dict, x: torch.Tensor, y: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """y = x W^T (fp16 [M][N]) for fp16 x [M][K] and a packed layer."""
    _dev(x, torch.float16, "x")
    L = layer_struct(layer)
    M = x.shape[0] if x.dim() == 2 else 1
    if y is None:
        y = torch.empty((M, L.N), dtype=torch.float16, device=x.device)
    _check(lib().owq_linear(ctypes.byref(L), _ptr(x), M, _ptr(y), _stream(stream)), "owq_linear")
    return y


def linear_batched(layers: list, xs: list, ys: list | None = None, stream=None) -> list:
    """Several independent decode linears (same 1 <= M <= 16) in one launch."""
    n = len(layers)
    Ls = (OwqLayer * n)(*[layer_struct(l) for l in layers])
    M = xs[0].shape[0]
    if ys is None:
        ys = [torch.empty((M, Ls[i].N), dtype=torch.float16, device=xs[i].device) for i in range(n)]
    xp = (_P * n)(*[x.data_ptr() for x in xs])
    yp = (_P * n)(*[y.data_ptr() for y in ys])
    _check(lib().owq_linear_batched(Ls, xp, yp, n, M, _stream(stream)), "owq_linear_batched")
    return ys


class PreparedBatched:
    """One owq_linear_batched call with its argument arrays built once.

    For decode loops that launch the same layers on the same buffers again and
    again: each call then only crosses into the library (which still checks the
    arguments) instead of rebuilding the layer structs and pointer arrays. The
    tensors must stay alive, at the same addresses, while the object is used.
    """

    def __init__(self, layers: list, xs: list, ys: list, stream=None):
        n = len(layers)
        for x in xs:
            _dev(x, torch.float16, "x")
        for y in ys:
            _dev(y, torch.float16, "y")
        self._keep = (list(layers), list(xs), list(ys))
        self.Ls = (OwqLayer * n)(*[layer_struct(l) for l in layers])
        self.xp = (_P * n)(*[x.data_ptr() for x in xs])
        self.yp = (_P * n)(*[y.data_ptr() for y in ys])
        self.n = n
        self.M = xs[0].shape[0]
        self.stream = _stream(stream)
        self.fn = lib().owq_linear_batched

    def __call__(self):
        _check(self.fn(self.Ls, self.xp, self.yp, self.n, self.M, self.stream), "owq_linear_batched")


# ----------------------------------------------------------- measurement aid


def stream_read(buf: torch.Tensor, sink: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Read-only HBM stream over `buf` (any dtype, contiguous, size a multiple of
    12 bytes) with the M = 1 decode kernel's geometry; not a step of the method.
    Returns the int32 sink: word w is the XOR of the 32-bit words of bytes
    [4608 w, 4608 (w + 1)) of the buffer."""
    if not isinstance(buf, torch.Tensor) or not buf.is_cuda or not buf.is_contiguous():
        raise TypeError("buf must be a contiguous CUDA (HIP) tensor")
    nbytes = buf.numel() * buf.element_size()
    words = lib().owq_stream_read_sink_words(nbytes)
    if sink is None:
        sink = torch.empty(max(words, 1), dtype=torch.int32, device=buf.device)
    _dev(sink, torch.int32, "sink")
    _check(lib().owq_stream_read(_ptr(buf), nbytes, _ptr(sink), sink.numel(), _stream(stream)), "owq_stream_read")
    return sink
