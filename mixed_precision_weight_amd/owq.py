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


class OwqCalibItem(ctypes.Structure):
    """Mirror of ``owq_calib_item`` (host struct, device pointers)."""
    _fields_ = [("W", _P), ("N", _I64), ("K", _I64), ("X", _P), ("T", _I64), ("lam", _P), ("score", _P)]


class OwqPackItem(ctypes.Structure):
    """Mirror of ``owq_pack_item`` (host struct, device pointers)."""
    _fields_ = [("W", _P), ("N", _I64), ("K", _I64), ("weak_idx", _P), ("k", _I32), ("qcodes", _P),
                ("scales", _P), ("zeros", _P), ("w_weak", _P)]


class OwqLayer(ctypes.Structure):
    """Mirror of ``owq_layer`` (host struct, device pointers)."""
    _fields_ = [("N", ctypes.c_int64), ("K", ctypes.c_int64), ("k", ctypes.c_int32),
                ("bits", ctypes.c_int32), ("qcodes", _P), ("scales", _P), ("zeros", _P),
                ("weak_idx", _P), ("w_weak", _P)]


class OwqGroupedLayer(ctypes.Structure):
    """Mirror of ``owq_grouped_layer`` (host struct, device pointers)."""
    _fields_ = [("N", ctypes.c_int64), ("K", ctypes.c_int64), ("G", ctypes.c_int64), ("k", ctypes.c_int32),
                ("bits", ctypes.c_int32), ("qcodes", _P), ("scales", _P), ("zeros", _P),
                ("weak_idx", _P), ("w_weak", _P)]


EXPORTS = {
    "owq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "owq_last_error": (ctypes.c_char_p, []),
    "owq_calibrate_workspace_bytes": (ctypes.c_size_t, [_I64, _I64, _I64]),
    "owq_calibrate_score": (ctypes.c_int, [_P, _I64, _I64, _P, _I64, _P, _P, _P, ctypes.c_size_t, _P]),
    "owq_calibrate_score_noalloc": (ctypes.c_int, [_P, _I64, _I64, _P, _I64, _P, _P, _P]),
    "owq_calibrate_noalloc_max_workspace": (ctypes.c_size_t, []),
    "owq_calibrate_batched_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(OwqCalibItem), _I32]),
    "owq_calibrate_score_batched": (ctypes.c_int, [ctypes.POINTER(OwqCalibItem), _I32, _P, ctypes.c_size_t, _P]),
    "owq_select_weak": (ctypes.c_int, [_P, _I64, _I32, _P, _P]),
    "owq_select_weak_batched": (ctypes.c_int, [ctypes.POINTER(_P), ctypes.POINTER(_I64), ctypes.POINTER(_I32),
                                               ctypes.POINTER(_P), _I32, _P]),
    "owq_pack": (ctypes.c_int, [_P, _I64, _I64, _P, _I32, _P, _P, _P, _P, _P]),
    "owq_pack_batched": (ctypes.c_int, [ctypes.POINTER(OwqPackItem), _I32, _P]),
    "owq_pack_search": (ctypes.c_int, [_P, _I64, _I64, _P, _I32, _P, _P, _P, _P, _P, _P]),
    "owq_pack_storage": (ctypes.c_int, [_P, _I64, _I64, _P, _I32, _P, _P, _P, _P, _P]),
    "owq_linear_storage_workspace_bytes": (ctypes.c_size_t, [_I64, _I32, _I64]),
    "owq_linear_storage": (ctypes.c_int, [ctypes.POINTER(OwqLayer), _P, _I64, _P, _P, ctypes.c_size_t, _P]),
    "owq_linear_storage_batched_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(OwqLayer), _I32, _I64]),
    "owq_linear_storage_batched": (ctypes.c_int, [ctypes.POINTER(OwqLayer), ctypes.POINTER(_P), ctypes.POINTER(_P),
                                                  _I32, _I64, _P, ctypes.c_size_t, _P]),
    "owq_linear_backward_workspace_bytes": (ctypes.c_size_t, [_I64, _I64, _I32]),
    "owq_linear_backward": (ctypes.c_int, [ctypes.POINTER(OwqLayer), _P, _P, _I64, _P, _P, _P, ctypes.c_size_t,
                                           _P]),
    "owq_linear_backward_batched_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(OwqLayer), _I32]),
    "owq_linear_backward_batched": (ctypes.c_int, [ctypes.POINTER(OwqLayer), ctypes.POINTER(_P), ctypes.POINTER(_P),
                                                   _I32, _I64, ctypes.POINTER(_P), ctypes.POINTER(_P), _P,
                                                   ctypes.c_size_t, _P]),
    "owq_pack_optq_workspace_bytes": (ctypes.c_size_t, [_I64, _I64, _I32]),
    "owq_pack_optq": (ctypes.c_int, [_P, _I64, _I64, _P, _I64, _P, _I32, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "owq_linear": (ctypes.c_int, [ctypes.POINTER(OwqLayer), _P, _I64, _P, _P]),
    "owq_linear_batched": (ctypes.c_int, [ctypes.POINTER(OwqLayer), ctypes.POINTER(_P),
                                          ctypes.POINTER(_P), _I32, _I64, _P]),
    "owq_pack_grouped": (ctypes.c_int, [_P, _I64, _I64, _P, _I32, _I64, _P, _P, _P, _P, _P]),
    "owq_linear_grouped": (ctypes.c_int, [ctypes.POINTER(OwqGroupedLayer), _P, _I64, _P, _P]),
    "owq_linear_grouped_batched": (ctypes.c_int, [ctypes.POINTER(OwqGroupedLayer), ctypes.POINTER(_P),
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


def _meta(t, dtype, name: str, shape=None) -> torch.Tensor:
    """Type, dtype, shape and contiguity of one argument. Runs before any device
    check, so a caller's shape mistake is reported as such on any device."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _on_device(*named):
    """Every (name, tensor) is a HIP tensor, all on one device."""
    devs = set()
    for name, t in named:
        if t is None:
            continue
        if not t.is_cuda:
            raise TypeError(f"{name} must be a CUDA (HIP) tensor")
        devs.add(t.device)
    if len(devs) > 1:
        raise ValueError(f"arguments are on different devices: {sorted(str(d) for d in devs)}")


def _dev(t: torch.Tensor, dtype, name: str, shape=None) -> torch.Tensor:
    _meta(t, dtype, name, shape)
    _on_device((name, t))
    return t


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


# ------------------------------------------------------------------ calibration


def calibrate_workspace_bytes(N: int, K: int, T: int) -> int:
    return int(lib().owq_calibrate_workspace_bytes(N, K, T))


def _calib_shapes(W, X):
    _meta(W, torch.float16, "W")
    _meta(X, torch.float16, "X")
    if W.dim() != 2 or X.dim() != 2:
        raise ValueError(f"W and X must be 2-D, got {tuple(W.shape)} and {tuple(X.shape)}")
    N, K = W.shape
    T = X.shape[0]
    if X.shape[1] != K:
        raise ValueError(f"X has {X.shape[1]} columns, W has {K}: both are [*, K]")
    return N, K, T


def calibrate(W: torch.Tensor, X: torch.Tensor, workspace: torch.Tensor | None = None, stream=None):
    """lambda (fp64 [K]) and score (fp64 [K]) of fp16 W [N][K] and X [T][K]."""
    N, K, T = _calib_shapes(W, X)
    if workspace is not None:
        _meta(workspace, torch.uint8, "workspace")
    _on_device(("W", W), ("X", X), ("workspace", workspace))
    nbytes = calibrate_workspace_bytes(N, K, T)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=W.device)
    lam = torch.empty(K, dtype=torch.float64, device=W.device)
    score = torch.empty(K, dtype=torch.float64, device=W.device)
    _check(lib().owq_calibrate_score(_ptr(W), N, K, _ptr(X), T, _ptr(lam), _ptr(score), _ptr(workspace),
                                     _nbytes(workspace), _stream(stream)),
           "owq_calibrate_score")
    return lam, score


def calibrate_noalloc(W: torch.Tensor, X: torch.Tensor, lam: torch.Tensor | None = None,
                      score: torch.Tensor | None = None, stream=None):
    """As calibrate(), with the library's own workspace (owq_calibrate_score_noalloc:
    no device allocation in the library). lam / score: optional fp64 [K] outputs,
    so that a caller that cannot allocate passes its own."""
    N, K, T = _calib_shapes(W, X)
    for name, t in (("lam", lam), ("score", score)):
        if t is not None:
            _meta(t, torch.float64, name, (K,))
    _on_device(("W", W), ("X", X), ("lam", lam), ("score", score))
    if lam is None:
        lam = torch.empty(K, dtype=torch.float64, device=W.device)
    if score is None:
        score = torch.empty(K, dtype=torch.float64, device=W.device)
    _check(lib().owq_calibrate_score_noalloc(_ptr(W), N, K, _ptr(X), T, _ptr(lam), _ptr(score), _stream(stream)),
           "owq_calibrate_score_noalloc")
    return lam, score


def _calib_items(Ws: list, Xs: list, outs=None):
    n = len(Ws)
    if n < 1 or len(Xs) != n:
        raise ValueError(f"need one X per W: {n} W, {len(Xs)} X")
    items = (OwqCalibItem * n)()
    res = []
    shapes = []
    for i, (W, X) in enumerate(zip(Ws, Xs)):
        try:
            shapes.append(_calib_shapes(W, X))
        except (TypeError, ValueError) as e:
            raise type(e)(f"[{i}] {e}") from None
    _on_device(*[(f"[{i}] W", W) for i, W in enumerate(Ws)], *[(f"[{i}] X", X) for i, X in enumerate(Xs)])
    for i, (W, X) in enumerate(zip(Ws, Xs)):
        N, K, T = shapes[i]
        if outs is None:
            lam = torch.empty(K, dtype=torch.float64, device=W.device)
            score = torch.empty(K, dtype=torch.float64, device=W.device)
        else:
            lam, score = outs[i]
        items[i] = OwqCalibItem(W.data_ptr(), N, K, X.data_ptr(), T, lam.data_ptr(), score.data_ptr())
        res.append((lam, score))
    return items, res


def calibrate_batched_workspace_bytes(shapes: list) -> int:
    """Workspace of calibrate_batched for (N, K, T) per linear."""
    n = len(shapes)
    items = (OwqCalibItem * max(n, 1))()
    for i, (N, K, T) in enumerate(shapes):
        items[i] = OwqCalibItem(None, N, K, None, T, None, None)
    return int(lib().owq_calibrate_batched_workspace_bytes(items, n))


def calibrate_batched(Ws: list, Xs: list, workspace: torch.Tensor | None = None, stream=None) -> list:
    """calibrate() of several linears in one pipelined sequence of launches
    (owq_calibrate_score_batched); returns one (lambda, score) pair per linear."""
    items, res = _calib_items(Ws, Xs)
    n = len(Ws)
    nbytes = int(lib().owq_calibrate_batched_workspace_bytes(items, n))
    if workspace is None:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=Ws[0].device)
    else:
        _meta(workspace, torch.uint8, "workspace")
        _on_device(("workspace", workspace))
    _check(lib().owq_calibrate_score_batched(items, n, _ptr(workspace), _nbytes(workspace), _stream(stream)),
           "owq_calibrate_score_batched")
    return res


def calibrate_noalloc_max_workspace() -> int:
    return int(lib().owq_calibrate_noalloc_max_workspace())


def select_weak(score: torch.Tensor, k: int, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Indices of the k largest scores, ascending (int32 [k]); written to out if given."""
    _meta(score, torch.float64, "score")
    if score.dim() != 1:
        raise ValueError(f"score must be 1-D, got shape {tuple(score.shape)}")
    k = int(k)
    if not 0 <= k <= score.numel():
        raise ValueError(f"k = {k} outside [0, K = {score.numel()}]")
    if out is not None:
        _meta(out, torch.int32, "out")
        if out.dim() != 1 or out.numel() < k:
            raise ValueError(f"out must be 1-D with at least k = {k} entries, got shape {tuple(out.shape)}")
    _on_device(("score", score), ("out", out))
    if out is None:
        out = torch.empty(max(k, 1), dtype=torch.int32, device=score.device)
    _check(lib().owq_select_weak(_ptr(score), score.numel(), k, _ptr(out) if k else None,
                                 _stream(stream)), "owq_select_weak")
    return out[:k]


def select_weak_batched(scores: list, ks: list, outs: list | None = None, stream=None) -> list:
    """owq_select_weak for several score vectors in one launch;
    returns one int32 [k] index tensor per score (written to outs[i] if given)."""
    n = len(scores)
    if n < 1 or len(ks) != n or (outs is not None and len(outs) != n):
        raise ValueError(f"need one k (and out) per score: {n} scores, {len(ks)} k"
                         + ("" if outs is None else f", {len(outs)} out"))
    for i, (sc, k) in enumerate(zip(scores, ks)):
        _meta(sc, torch.float64, f"[{i}] score")
        if sc.dim() != 1:
            raise ValueError(f"[{i}] score must be 1-D, got shape {tuple(sc.shape)}")
        if not 0 <= int(k) <= sc.numel():
            raise ValueError(f"[{i}] k = {k} outside [0, K = {sc.numel()}]")
        if outs is not None:
            _meta(outs[i], torch.int32, f"[{i}] out")
            if outs[i].dim() != 1 or outs[i].numel() < int(k):
                raise ValueError(f"[{i}] out must be 1-D with at least k = {k} entries, "
                                 f"got shape {tuple(outs[i].shape)}")
    _on_device(*[(f"[{i}] score", sc) for i, sc in enumerate(scores)],
               *([] if outs is None else [(f"[{i}] out", o) for i, o in enumerate(outs)]))
    if outs is None:
        outs = [torch.empty(max(int(k), 1), dtype=torch.int32, device=sc.device) for sc, k in zip(scores, ks)]
    sp = (_P * n)(*[sc.data_ptr() for sc in scores])
    Kp = (_I64 * n)(*[sc.numel() for sc in scores])
    kp = (_I32 * n)(*[int(k) for k in ks])
    op = (_P * n)(*[o.data_ptr() for o in outs])
    _check(lib().owq_select_weak_batched(sp, Kp, kp, op, n, _stream(stream)), "owq_select_weak_batched")
    return [o[:int(k)] for o, k in zip(outs, ks)]


# ------------------------------------------------------------------------ pack

_PACK_OUT = ("qcodes", "scales", "zeros", "w_weak")


def _pack_out_shapes(N: int, K: int, k: int) -> dict:
    return {"qcodes": ((N, K // 32, 3), torch.int32), "scales": ((N,), torch.float16),
            "zeros": ((N,), torch.uint8), "w_weak": ((N, k), torch.float16)}


def _pack_args(W, weak_idx, out, where="", device_check=True):
    """Checked shapes (N, K, k) of one pack, and its out dict (allocated if None;
    device_check=False: the caller checks the devices of every pack first)."""
    _meta(W, torch.float16, f"{where}W")
    _meta(weak_idx, torch.int32, f"{where}weak_idx")
    if W.dim() != 2 or weak_idx.dim() != 1:
        raise ValueError(f"{where}W must be 2-D and weak_idx 1-D, got {tuple(W.shape)} and {tuple(weak_idx.shape)}")
    N, K = W.shape
    k = weak_idx.numel()
    if K % 32 or k > K:
        raise ValueError(f"{where}K = {K} must be a multiple of 32 and k = {k} at most K")
    want = _pack_out_shapes(N, K, k)
    if out is not None:
        for name in _PACK_OUT:
            if name not in out:
                raise ValueError(f"{where}out lacks {name!r}")
            _meta(out[name], want[name][1], f"{where}out[{name!r}]", want[name][0])
    if device_check:
        _on_device((f"{where}W", W), (f"{where}weak_idx", weak_idx),
                   *[(f"{where}out[{n!r}]", out[n]) for n in (_PACK_OUT if out else ())])
    if out is None:
        out = {name: torch.empty(shape, dtype=dt, device=W.device) for name, (shape, dt) in want.items()}
    out["weak_idx"] = weak_idx
    return N, K, k, out


def pack(W: torch.Tensor, weak_idx: torch.Tensor, out: dict | None = None, stream=None) -> dict:
    """Latency-favoured packed layer: dict of device tensors
    qcodes int32 [N][K/32][3] (uint32 bits), scales fp16 [N], zeros uint8 [N],
    w_weak fp16 [N][k], weak_idx int32 [k]."""
    N, K, k, out = _pack_args(W, weak_idx, out)
    _check(lib().owq_pack(_ptr(W), N, K, _ptr(weak_idx) if k else None, k, _ptr(out["qcodes"]),
                          _ptr(out["scales"]), _ptr(out["zeros"]), _ptr(out["w_weak"]) if k else None,
                          _stream(stream)), "owq_pack")
    return out


def pack_batched(Ws: list, weak_idxs: list, outs: list | None = None, stream=None) -> list:
    """pack() of several linears (owq_pack_batched: the linears of one kernel
    form in one launch); returns one packed dict per linear (outs[i] if given)."""
    n = len(Ws)
    if n < 1 or len(weak_idxs) != n or (outs is not None and len(outs) != n):
        raise ValueError(f"need one weak_idx (and out) per W: {n} W, {len(weak_idxs)} weak_idx"
                         + ("" if outs is None else f", {len(outs)} out"))
    named = []
    for i, (W, ix) in enumerate(zip(Ws, weak_idxs)):  # every shape first, then every device
        _pack_args(W, ix, None if outs is None else outs[i], f"[{i}] ", device_check=False)
        named += [(f"[{i}] W", W), (f"[{i}] weak_idx", ix)]
        if outs is not None:
            named += [(f"[{i}] out[{n!r}]", outs[i][n]) for n in _PACK_OUT]
    _on_device(*named)
    args = [_pack_args(W, ix, None if outs is None else outs[i], f"[{i}] ", device_check=False)
            for i, (W, ix) in enumerate(zip(Ws, weak_idxs))]
    items = (OwqPackItem * n)()
    for i, (W, (N, K, k, out)) in enumerate(zip(Ws, args)):
        items[i] = OwqPackItem(W.data_ptr(), N, K, out["weak_idx"].data_ptr() if k else None, k,
                               out["qcodes"].data_ptr(), out["scales"].data_ptr(), out["zeros"].data_ptr(),
                               out["w_weak"].data_ptr() if k else None)
    _check(lib().owq_pack_batched(items, n, _stream(stream)), "owq_pack_batched")
    return [a[3] for a in args]


def pack_search(W: torch.Tensor, weak_idx: torch.Tensor, lam: torch.Tensor | None = None,
                out: dict | None = None, stream=None) -> dict:
    """pack() with each row's step and zero point from the truncation-aware grid
    search (owq_pack_search); lam: optional fp64 [K] column weights (the Hessian
    diagonal from calibrate())."""
    _meta(W, torch.float16, "W")
    _meta(weak_idx, torch.int32, "weak_idx")
    if W.dim() != 2 or weak_idx.dim() != 1:
        raise ValueError(f"W must be 2-D and weak_idx 1-D, got {tuple(W.shape)} and {tuple(weak_idx.shape)}")
    N, K = W.shape
    k = weak_idx.numel()
    if K % 32 or k > K:
        raise ValueError(f"K = {K} must be a multiple of 32 and k = {k} at most K")
    if lam is not None:
        _meta(lam, torch.float64, "lam", (K,))
    want = _pack_out_shapes(N, K, k)
    if out is not None:
        for name in _PACK_OUT:
            if name not in out:
                raise ValueError(f"out lacks {name!r}")
            _meta(out[name], want[name][1], f"out[{name!r}]", want[name][0])
    _on_device(("W", W), ("weak_idx", weak_idx), ("lam", lam),
               *[(f"out[{n!r}]", out[n]) for n in (_PACK_OUT if out else ())])
    if out is None:
        out = {name: torch.empty(shape, dtype=dt, device=W.device) for name, (shape, dt) in want.items()}
    out["weak_idx"] = weak_idx
    _check(lib().owq_pack_search(_ptr(W), N, K, _ptr(weak_idx) if k else None, k, _ptr(lam), _ptr(out["qcodes"]),
                                 _ptr(out["scales"]), _ptr(out["zeros"]), _ptr(out["w_weak"]) if k else None,
                                 _stream(stream)), "owq_pack_search")
    return out


def pack_optq_workspace_bytes(N: int, K: int, k: int) -> int:
    return int(lib().owq_pack_optq_workspace_bytes(N, K, k))


def pack_optq(W: torch.Tensor, X: torch.Tensor, weak_idx: torch.Tensor, out: dict | None = None,
              workspace: torch.Tensor | None = None, stream=None) -> dict:
    """Latency-favoured pack with OPTQ's sequential quantisation and the weak
    columns last (owq_pack_optq) on calibration input X [T][K]."""
    N, K, T = _calib_shapes(W, X)
    _meta(weak_idx, torch.int32, "weak_idx")
    if weak_idx.dim() != 1:
        raise ValueError(f"weak_idx must be 1-D, got {tuple(weak_idx.shape)}")
    k = weak_idx.numel()
    if K % 32 or k > K:
        raise ValueError(f"K = {K} must be a multiple of 32 and k = {k} at most K")
    want = _pack_out_shapes(N, K, k)
    if out is not None:
        for name in _PACK_OUT:
            if name not in out:
                raise ValueError(f"out lacks {name!r}")
            _meta(out[name], want[name][1], f"out[{name!r}]", want[name][0])
    if workspace is not None:
        _meta(workspace, torch.uint8, "workspace")
    _on_device(("W", W), ("X", X), ("weak_idx", weak_idx), ("workspace", workspace),
               *[(f"out[{n!r}]", out[n]) for n in (_PACK_OUT if out else ())])
    if out is None:
        out = {name: torch.empty(shape, dtype=dt, device=W.device) for name, (shape, dt) in want.items()}
    out["weak_idx"] = weak_idx
    if workspace is None:
        workspace = torch.empty(pack_optq_workspace_bytes(N, K, k), dtype=torch.uint8, device=W.device)
    _check(lib().owq_pack_optq(_ptr(W), N, K, _ptr(X), T, _ptr(weak_idx) if k else None, k, _ptr(out["qcodes"]),
                               _ptr(out["scales"]), _ptr(out["zeros"]), _ptr(out["w_weak"]) if k else None,
                               _ptr(workspace), _nbytes(workspace), _stream(stream)), "owq_pack_optq")
    return out


# ------------------------------------------------------- storage-favoured form


def pack_storage(W: torch.Tensor, weak_idx: torch.Tensor, out: dict | None = None, stream=None) -> dict:
    """Storage-favoured packed layer (owq_pack_storage): qcodes int32
    [N][ceil((K-k)/32)][3] of the dense columns only, scales, zeros, w_weak,
    weak_idx, and "K" (the full column count)."""
    _meta(W, torch.float16, "W")
    _meta(weak_idx, torch.int32, "weak_idx")
    if W.dim() != 2 or weak_idx.dim() != 1:
        raise ValueError(f"W must be 2-D and weak_idx 1-D, got {tuple(W.shape)} and {tuple(weak_idx.shape)}")
    N, K = W.shape
    k = weak_idx.numel()
    if K % 32 or k > K:
        raise ValueError(f"K = {K} must be a multiple of 32 and k = {k} at most K")
    want = _pack_out_shapes(N, K, k)
    want["qcodes"] = ((N, (K - k + 31) // 32, 3), torch.int32)
    if out is not None:
        for name in _PACK_OUT:
            if name not in out:
                raise ValueError(f"out lacks {name!r}")
            _meta(out[name], want[name][1], f"out[{name!r}]", want[name][0])
    _on_device(("W", W), ("weak_idx", weak_idx), *[(f"out[{n!r}]", out[n]) for n in (_PACK_OUT if out else ())])
    if out is None:
        out = {name: torch.empty(shape, dtype=dt, device=W.device) for name, (shape, dt) in want.items()}
    out["weak_idx"] = weak_idx
    out["K"] = K
    q = out["qcodes"]
    _check(lib().owq_pack_storage(_ptr(W), N, K, _ptr(weak_idx) if k else None, k, _ptr(q) if q.numel() else None,
                                  _ptr(out["scales"]), _ptr(out["zeros"]), _ptr(out["w_weak"]) if k else None,
                                  _stream(stream)), "owq_pack_storage")
    return out


def linear_storage_workspace_bytes(K: int, k: int, M: int) -> int:
    return int(lib().owq_linear_storage_workspace_bytes(K, k, M))


def _storage_args(layer: dict, x: torch.Tensor, y, where: str = ""):
    """Checked shapes of one storage-form product: (OwqLayer, N, K, k, M)."""
    if "K" not in layer:
        raise ValueError(f"{where}layer lacks 'K' (the full column count of the storage-favoured form)")
    K = int(layer["K"])
    q = _meta(layer["qcodes"], torch.int32, f"{where}qcodes")
    idx = _meta(layer["weak_idx"], torch.int32, f"{where}weak_idx")
    N, k = q.shape[0], idx.numel()
    if q.dim() != 3 or tuple(q.shape[1:]) != ((K - k + 31) // 32, 3) or idx.dim() != 1:
        raise ValueError(f"{where}qcodes {tuple(q.shape)} / weak_idx {tuple(idx.shape)} do not fit K = {K}")
    for name, (shape, dt) in _pack_out_shapes(N, K, k).items():
        if name != "qcodes":
            _meta(layer[name], dt, f"{where}{name}", shape)
    M = _xy_shapes(N, K, x, y, tag=where)
    L = OwqLayer(N, K, k, 3, q.data_ptr() if q.numel() else None, layer["scales"].data_ptr(),
                 layer["zeros"].data_ptr(), idx.data_ptr() if k else None, layer["w_weak"].data_ptr() if k else None)
    return L, N, K, k, M


def linear_storage(layer: dict, x: torch.Tensor, y: torch.Tensor | None = None,
                   workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """y = x W^T for a layer in the storage-favoured form (owq_linear_storage)."""
    L, N, K, k, M = _storage_args(layer, x, y)
    if workspace is not None:
        _meta(workspace, torch.uint8, "workspace")
    _on_device(("x", x), ("y", y), ("workspace", workspace), *_layer_named(layer))
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=x.device)
    if workspace is None:
        workspace = torch.empty(linear_storage_workspace_bytes(K, k, M), dtype=torch.uint8, device=x.device)
    _check(lib().owq_linear_storage(ctypes.byref(L), _ptr(x), M, _ptr(y), _ptr(workspace), _nbytes(workspace),
                                    _stream(stream)), "owq_linear_storage")
    return y


def linear_storage_batched_workspace_bytes(layers: list, M: int) -> int:
    """Workspace of linear_storage_batched for these storage-form layers at M tokens."""
    n = len(layers)
    Ls = (OwqLayer * max(n, 1))()
    for i, l in enumerate(layers):
        q, idx = l["qcodes"], l["weak_idx"]
        Ls[i] = OwqLayer(q.shape[0], int(l["K"]), idx.numel(), 3, None, None, None, None, None)
    return int(lib().owq_linear_storage_batched_workspace_bytes(Ls, n, M))


def linear_storage_batched(layers: list, xs: list, ys: list | None = None, workspace: torch.Tensor | None = None,
                           stream=None) -> list:
    """linear_storage() of several layers at one M (owq_linear_storage_batched:
    three launches for all of them); returns one y per layer (ys[i] if given)."""
    n = len(layers)
    if n < 1 or len(xs) != n or (ys is not None and len(ys) != n):
        raise ValueError(f"need one x (and y) per layer: {n} layers, {len(xs)} x"
                         + ("" if ys is None else f", {len(ys)} y"))
    args = [_storage_args(l, x, None if ys is None else ys[i], f"[{i}] ")
            for i, (l, x) in enumerate(zip(layers, xs))]
    Ms = {a[4] for a in args}
    if len(Ms) != 1:
        raise ValueError(f"every x must have the same M, got {sorted(Ms)}")
    M = Ms.pop()
    if workspace is not None:
        _meta(workspace, torch.uint8, "workspace")
    named = [("workspace", workspace)]
    for i, (l, x) in enumerate(zip(layers, xs)):
        named += [(f"[{i}] x", x), (f"[{i}] y", None if ys is None else ys[i])]
        named += [(f"[{i}] {nm}", t) for nm, t in _layer_named(l)]
    _on_device(*named)
    if ys is None:
        ys = [torch.empty((M, a[1]), dtype=torch.float16, device=xs[0].device) for a in args]
    Ls = (OwqLayer * n)(*[a[0] for a in args])
    nbytes = int(lib().owq_linear_storage_batched_workspace_bytes(Ls, n, M))
    if workspace is None:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=xs[0].device)
    xp = (_P * n)(*[x.data_ptr() for x in xs])
    yp = (_P * n)(*[y.data_ptr() for y in ys])
    _check(lib().owq_linear_storage_batched(Ls, xp, yp, n, M, _ptr(workspace), _nbytes(workspace), _stream(stream)),
           "owq_linear_storage_batched")
    return ys


# ---------------------------------------------------------------------- linear


def layer_shapes(layer: dict):
    """(N, K, k) of a packed layer dict, after checking that its five tensors
    agree with one another."""
    for name in _PACK_OUT + ("weak_idx",):
        if name not in layer:
            raise ValueError(f"layer lacks {name!r}")
    q = layer["qcodes"]
    _meta(q, torch.int32, "qcodes")
    if q.dim() != 3 or q.shape[2] != 3:
        raise ValueError(f"qcodes must be [N][K/32][3], got {tuple(q.shape)}")
    N, K = q.shape[0], q.shape[1] * 32
    idx = _meta(layer["weak_idx"], torch.int32, "weak_idx")
    if idx.dim() != 1:
        raise ValueError(f"weak_idx must be 1-D, got {tuple(idx.shape)}")
    k = idx.numel()
    for name, (shape, dt) in _pack_out_shapes(N, K, k).items():
        _meta(layer[name], dt, name, shape)
    return N, K, k


def _layer_named(layer: dict, tag: str = ""):
    return [(tag + n, layer[n]) for n in _PACK_OUT + ("weak_idx",)]


def layer_struct(layer: dict) -> OwqLayer:
    N, K, k = layer_shapes(layer)
    return OwqLayer(N, K, k, 3, layer["qcodes"].data_ptr(), layer["scales"].data_ptr(), layer["zeros"].data_ptr(),
                    layer["weak_idx"].data_ptr() if k else None, layer["w_weak"].data_ptr() if k else None)


def _xy_shapes(N: int, K: int, x, y, tag: str = "", M: int | None = None):
    """x fp16 [M][K] (or [K] for M = 1); y fp16 [M][N] if given. Returns M."""
    _meta(x, torch.float16, tag + "x")
    if x.dim() == 1:
        xs = (1, x.shape[0])
    elif x.dim() == 2:
        xs = tuple(x.shape)
    else:
        raise ValueError(f"{tag}x must be [M][K] or [K], got {tuple(x.shape)}")
    if xs[1] != K:
        raise ValueError(f"{tag}x has {xs[1]} columns, the layer has K = {K}")
    if xs[0] < 1:
        raise ValueError(f"{tag}x has no rows")
    if M is not None and xs[0] != M:
        raise ValueError(f"{tag}x has {xs[0]} rows, the batch has M = {M}")
    if y is not None:
        _meta(y, torch.float16, tag + "y")
        if y.numel() != xs[0] * N or (y.dim() == 2 and tuple(y.shape) != (xs[0], N)) or y.dim() > 2:
            raise ValueError(f"{tag}y has shape {tuple(y.shape)}, expected ({xs[0]}, {N})")
    return xs[0]


def linear(layer: dict, x: torch.Tensor, y: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """y = x W^T (fp16 [M][N]) for fp16 x [M][K] and a packed layer."""
    N, K, k = layer_shapes(layer)
    M = _xy_shapes(N, K, x, y)
    _on_device(("x", x), ("y", y), *_layer_named(layer))
    L = layer_struct(layer)
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=x.device)
    _check(lib().owq_linear(ctypes.byref(L), _ptr(x), M, _ptr(y), _stream(stream)), "owq_linear")
    return y


def pack_grouped(W: torch.Tensor, weak_idx: torch.Tensor, G: int, out: dict | None = None, stream=None) -> dict:
    """Group-wise packed layer (owq_pack_grouped): qcodes int32 [N][K/32][3],
    scales fp16 [N][K/G], zeros uint8 [N][K/G], w_weak fp16 [N][k], weak_idx,
    and the group size under "group"."""
    _meta(W, torch.float16, "W")
    _meta(weak_idx, torch.int32, "weak_idx")
    if W.dim() != 2 or weak_idx.dim() != 1:
        raise ValueError(f"W must be 2-D and weak_idx 1-D, got {tuple(W.shape)} and {tuple(weak_idx.shape)}")
    N, K = W.shape
    k = weak_idx.numel()
    G = int(G)
    if K % 32 or k > K:
        raise ValueError(f"K = {K} must be a multiple of 32 and k = {k} at most K")
    if G < 32 or G > 2048 or G & (G - 1) or K % G:
        raise ValueError(f"G = {G}: need a power of two in [32, 2048] dividing K = {K}")
    want = {"qcodes": ((N, K // 32, 3), torch.int32), "scales": ((N, K // G), torch.float16),
            "zeros": ((N, K // G), torch.uint8), "w_weak": ((N, k), torch.float16)}
    if out is not None:
        for name, (shape, dt) in want.items():
            if name not in out:
                raise ValueError(f"out lacks {name!r}")
            _meta(out[name], dt, f"out[{name!r}]", shape)
    _on_device(("W", W), ("weak_idx", weak_idx), *[(f"out[{n!r}]", out[n]) for n in (want if out else ())])
    if out is None:
        out = {name: torch.empty(shape, dtype=dt, device=W.device) for name, (shape, dt) in want.items()}
    out["weak_idx"] = weak_idx
    out["group"] = G
    _check(lib().owq_pack_grouped(_ptr(W), N, K, _ptr(weak_idx) if k else None, k, G, _ptr(out["qcodes"]),
                                  _ptr(out["scales"]), _ptr(out["zeros"]), _ptr(out["w_weak"]) if k else None,
                                  _stream(stream)), "owq_pack_grouped")
    return out


def grouped_layer_struct(layer: dict) -> OwqGroupedLayer:
    """Checked host struct of a group-wise layer dict."""
    if "group" not in layer:
        raise ValueError("layer lacks 'group'")
    G = int(layer["group"])
    q = _meta(layer["qcodes"], torch.int32, "qcodes")
    if q.dim() != 3 or q.shape[2] != 3:
        raise ValueError(f"qcodes must be [N][K/32][3], got {tuple(q.shape)}")
    N, K = q.shape[0], q.shape[1] * 32
    if G < 32 or K % G:
        raise ValueError(f"G = {G} does not divide K = {K}")
    idx = _meta(layer["weak_idx"], torch.int32, "weak_idx")
    if idx.dim() != 1:
        raise ValueError(f"weak_idx must be 1-D, got {tuple(idx.shape)}")
    k = idx.numel()
    _meta(layer["scales"], torch.float16, "scales", (N, K // G))
    _meta(layer["zeros"], torch.uint8, "zeros", (N, K // G))
    _meta(layer["w_weak"], torch.float16, "w_weak", (N, k))
    return OwqGroupedLayer(N, K, G, k, 3, q.data_ptr(), layer["scales"].data_ptr(), layer["zeros"].data_ptr(),
                           idx.data_ptr() if k else None, layer["w_weak"].data_ptr() if k else None)


def linear_grouped(layer: dict, x: torch.Tensor, y: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """y = x W^T (fp16 [M][N]) for a group-wise packed layer (owq_linear_grouped)."""
    L = grouped_layer_struct(layer)
    M = _xy_shapes(L.N, L.K, x, y)
    _on_device(("x", x), ("y", y), *_layer_named(layer))
    if y is None:
        y = torch.empty((M, L.N), dtype=torch.float16, device=x.device)
    _check(lib().owq_linear_grouped(ctypes.byref(L), _ptr(x), M, _ptr(y), _stream(stream)), "owq_linear_grouped")
    return y


def linear_grouped_batched(layers: list, xs: list, ys: list | None = None, stream=None) -> list:
    """owq_linear_grouped for several group-wise layers at the same M in one
    launch (M <= 4)."""
    if not layers or len(xs) != len(layers) or (ys is not None and len(ys) != len(layers)):
        raise ValueError("layers, xs (and ys) must be non-empty lists of one length")
    Ls = (OwqGroupedLayer * len(layers))()
    M = None
    out = []
    for i, lay in enumerate(layers):
        Ls[i] = grouped_layer_struct(lay)
        y = None if ys is None else ys[i]
        M = _xy_shapes(Ls[i].N, Ls[i].K, xs[i], y, f"layer {i}: ", M)
        _on_device((f"layer {i}: x", xs[i]), (f"layer {i}: y", y), *_layer_named(lay, f"layer {i}: "))
        out.append(y if y is not None else torch.empty((M, Ls[i].N), dtype=torch.float16, device=xs[i].device))
    xp = (_P * len(layers))(*[x.data_ptr() for x in xs])
    yp = (_P * len(layers))(*[y.data_ptr() for y in out])
    _check(lib().owq_linear_grouped_batched(Ls, xp, yp, len(layers), M, _stream(stream)),
           "owq_linear_grouped_batched")
    return out


def linear_backward_workspace_bytes(N: int, K: int, k: int) -> int:
    return int(lib().owq_linear_backward_workspace_bytes(N, K, k))


def linear_backward(layer: dict, x: torch.Tensor | None, dy: torch.Tensor, want_dx: bool = True,
                    want_dw: bool = True, workspace: torch.Tensor | None = None, stream=None):
    """Weak-column-tuning backward (owq_linear_backward): (dx fp16 [M][K] or None,
    dw_weak fp32 [N][k] or None) for the upstream gradient dy fp16 [M][N]."""
    N, K, k = layer_shapes(layer)
    _meta(dy, torch.float16, "dy")
    if dy.dim() != 2 or dy.shape[1] != N:
        raise ValueError(f"dy has shape {tuple(dy.shape)}, expected (M, {N})")
    M = dy.shape[0]
    if want_dw and k > 0:
        if x is None:
            raise ValueError("x is needed for dw_weak")
        _xy_shapes(N, K, x, None, M=M)
    elif x is not None:
        _xy_shapes(N, K, x, None, M=M)
    if workspace is not None:
        _meta(workspace, torch.uint8, "workspace")
    _on_device(("x", x), ("dy", dy), ("workspace", workspace), *_layer_named(layer))
    dx = torch.empty((M, K), dtype=torch.float16, device=dy.device) if want_dx else None
    dw = torch.empty((N, k), dtype=torch.float32, device=dy.device) if want_dw else None
    if want_dx and workspace is None:
        workspace = torch.empty(linear_backward_workspace_bytes(N, K, k), dtype=torch.uint8, device=dy.device)
    L = layer_struct(layer)
    _check(lib().owq_linear_backward(ctypes.byref(L), _ptr(x), _ptr(dy), M, _ptr(dx),
                                     _ptr(dw) if (want_dw and k) else None, _ptr(workspace) if want_dx else None,
                                     _nbytes(workspace) if want_dx else 0, _stream(stream)), "owq_linear_backward")
    return dx, dw


def linear_backward_batched_workspace_bytes(layers: list) -> int:
    Ls = (OwqLayer * len(layers))(*[layer_struct(l) for l in layers])
    return int(lib().owq_linear_backward_batched_workspace_bytes(Ls, len(layers)))


def linear_backward_batched(layers: list, xs: list | None, dys: list, want_dx: bool = True, want_dw: bool = True,
                            workspace: torch.Tensor | None = None, stream=None):
    """owq_linear_backward_batched: the backward of several layers (same M) in one
    launch per 4 tokens. Returns (dxs, dws), lists of fp16 [M][K] / fp32 [N][k]
    tensors (None where not wanted)."""
    n = len(layers)
    if n < 1 or len(dys) != n or (xs is not None and len(xs) != n):
        raise ValueError(f"need as many dy (and x) as layers: {n} layers, {len(dys)} dy"
                         + ("" if xs is None else f", {len(xs)} x"))
    M = None
    named = []
    shapes = []
    for i, layer in enumerate(layers):
        N, K, k = layer_shapes(layer)
        shapes.append((N, K, k))
        dy = dys[i]
        _meta(dy, torch.float16, f"[{i}] dy")
        if dy.dim() != 2 or dy.shape[1] != N:
            raise ValueError(f"[{i}] dy has shape {tuple(dy.shape)}, expected (M, {N})")
        if M is None:
            M = dy.shape[0]
        elif dy.shape[0] != M:
            raise ValueError(f"[{i}] dy has {dy.shape[0]} tokens, the first layer's has {M}")
        x = None if xs is None else xs[i]
        if want_dw and k > 0 and x is None:
            raise ValueError(f"[{i}] x is needed for dw_weak")
        if x is not None:
            _xy_shapes(N, K, x, None, f"[{i}] ", M=M)
        named += [(f"[{i}] dy", dy), (f"[{i}] x", x)] + _layer_named(layer, f"[{i}] ")
    if workspace is not None:
        _meta(workspace, torch.uint8, "workspace")
        named.append(("workspace", workspace))
    _on_device(*named)
    dev = dys[0].device
    dxs = [torch.empty((M, K), dtype=torch.float16, device=dev) if want_dx else None for (N, K, k) in shapes]
    dws = [torch.empty((N, k), dtype=torch.float32, device=dev) if want_dw else None for (N, K, k) in shapes]
    Ls = (OwqLayer * n)(*[layer_struct(l) for l in layers])
    if want_dx and workspace is None:
        workspace = torch.empty(int(lib().owq_linear_backward_batched_workspace_bytes(Ls, n)), dtype=torch.uint8,
                                device=dev)
    xp = None if xs is None else (_P * n)(*[None if x is None else x.data_ptr() for x in xs])
    dyp = (_P * n)(*[dy.data_ptr() for dy in dys])
    dxp = (_P * n)(*[dx.data_ptr() for dx in dxs]) if want_dx else None
    dwp = (_P * n)(*[dw.data_ptr() if (dw is not None and dw.numel()) else None for dw in dws]) if want_dw else None
    _check(lib().owq_linear_backward_batched(Ls, xp, dyp, n, M, dxp, dwp, _ptr(workspace) if want_dx else None,
                                             _nbytes(workspace) if want_dx else 0, _stream(stream)),
           "owq_linear_backward_batched")
    return dxs, dws


def _batched_args(layers: list, xs: list, ys: list | None):
    n = len(layers)
    if n < 1 or len(xs) != n or (ys is not None and len(ys) != n):
        raise ValueError(f"need as many x (and y) as layers: {n} layers, {len(xs)} x"
                         + ("" if ys is None else f", {len(ys)} y"))
    M = None
    named = []
    for i, layer in enumerate(layers):
        N, K, _ = layer_shapes(layer)
        M = _xy_shapes(N, K, xs[i], None if ys is None else ys[i], f"[{i}] ", M)
        named += [(f"[{i}] x", xs[i])] + ([] if ys is None else [(f"[{i}] y", ys[i])])
        named += _layer_named(layer, f"[{i}] ")
    _on_device(*named)
    return n, M


def linear_batched(layers: list, xs: list, ys: list | None = None, stream=None) -> list:
    """Several independent decode linears (same 1 <= M <= 16) in one launch."""
    n, M = _batched_args(layers, xs, ys)
    Ls = (OwqLayer * n)(*[layer_struct(l) for l in layers])
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
    With stream=None each call enqueues on torch's current stream at that call
    (so calls made under HIP graph capture are captured); a given stream is
    used for every call.
    """

    def __init__(self, layers: list, xs: list, ys: list, stream=None):
        n, M = _batched_args(layers, xs, ys)
        self._keep = (list(layers), list(xs), list(ys))
        self.Ls = (OwqLayer * n)(*[layer_struct(l) for l in layers])
        self.xp = (_P * n)(*[x.data_ptr() for x in xs])
        self.yp = (_P * n)(*[y.data_ptr() for y in ys])
        self.n = n
        self.M = M
        self.stream = None if stream is None else _stream(stream)
        self.fn = lib().owq_linear_batched

    def __call__(self):
        st = self.stream if self.stream is not None else _stream()
        _check(self.fn(self.Ls, self.xp, self.yp, self.n, self.M, st), "owq_linear_batched")


class PreparedCalibrate:
    """One owq_calibrate_score_batched call with its item array, outputs and
    workspace built once (outputs: `results`, one (lambda, score) pair per
    linear, rewritten by every call). The W and X tensors must stay alive, at
    the same addresses, while the object is used. With stream=None each call
    enqueues on torch's current stream at that call."""

    def __init__(self, Ws: list, Xs: list, workspace: torch.Tensor | None = None, stream=None):
        self.items, self.results = _calib_items(Ws, Xs)
        self.n = len(Ws)
        nbytes = int(lib().owq_calibrate_batched_workspace_bytes(self.items, self.n))
        if workspace is None:
            workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=Ws[0].device)
        else:
            _meta(workspace, torch.uint8, "workspace")
            _on_device(("workspace", workspace))
        self._keep = (list(Ws), list(Xs), workspace)
        self.ws = _ptr(workspace)
        self.ws_bytes = _nbytes(workspace)
        self.stream = None if stream is None else _stream(stream)
        self.fn = lib().owq_calibrate_score_batched

    def __call__(self) -> list:
        st = self.stream if self.stream is not None else _stream()
        _check(self.fn(self.items, self.n, self.ws, self.ws_bytes, st), "owq_calibrate_score_batched")
        return self.results


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
