"""CPU tests of the C ABI: libowq.so loads, exports every function include/owq.h
declares, and rejects invalid arguments synchronously (before any HIP call, so
these run without a GPU). No compute call is made here."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "owq.h")

FAKE = 0x100000  # non-NULL, 256-byte aligned host address; never dereferenced on error paths


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(owq_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from mixed_precision_weight_amd import owq
    return owq.lib()


def test_library_exports_every_declared_symbol(lib):
    names = _declared()
    assert len(names) >= 8
    out = subprocess.run(["nm", "-D", "--defined-only", os.path.join(ROOT, "mixed_precision_weight_amd", "libowq.so")],
                         capture_output=True, text=True, check=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if l.strip())
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        getattr(lib, n)


def test_binding_covers_header():
    from mixed_precision_weight_amd import owq
    assert set(_declared()) == set(owq.EXPORTS)


def test_status_strings(lib):
    for s in range(8):
        txt = lib.owq_status_string(s).decode()
        assert txt.startswith("OWQ_")
    assert lib.owq_status_string(99) is not None


def test_workspace_bytes(lib):
    assert lib.owq_calibrate_workspace_bytes(4096, 4096, 2048) > 0
    assert lib.owq_calibrate_workspace_bytes(4096, 4100, 2048) == 0
    assert lib.owq_calibrate_workspace_bytes(0, 4096, 2048) == 0
    assert lib.owq_calibrate_workspace_bytes(4096, 4096, 0) == 0
    assert lib.owq_calibrate_workspace_bytes(4096, 65536 + 32, 16) == 0
    # monotone in each size
    a = lib.owq_calibrate_workspace_bytes(1024, 4096, 2048)
    b = lib.owq_calibrate_workspace_bytes(8192, 4096, 2048)
    assert b >= a


def _err(lib):
    return lib.owq_last_error().decode()


def test_calibrate_validation(lib):
    f = lib.owq_calibrate_score
    ws = lib.owq_calibrate_workspace_bytes(64, 64, 64)
    assert f(None, 64, 64, FAKE, 64, FAKE, FAKE, FAKE, ws, None) == 1
    assert "non-NULL" in _err(lib)
    assert f(FAKE, 0, 64, FAKE, 64, FAKE, FAKE, FAKE, ws, None) == 2
    assert f(FAKE, 64, 48, FAKE, 64, FAKE, FAKE, FAKE, ws, None) == 2
    assert f(FAKE, 64, 64, FAKE, 0, FAKE, FAKE, FAKE, ws, None) == 2
    assert f(FAKE + 2, 64, 64, FAKE, 64, FAKE, FAKE, FAKE, ws, None) == 4
    assert f(FAKE, 64, 64, FAKE, 64, FAKE, FAKE, FAKE + 16, ws, None) == 4
    assert f(FAKE, 64, 64, FAKE, 64, FAKE, FAKE, FAKE, ws - 1, None) == 6
    assert "workspace" in _err(lib)


def test_calibrate_batched_validation(lib):
    from mixed_precision_weight_amd import owq
    It = owq.OwqCalibItem
    a, b = It(FAKE, 64, 64, FAKE, 32, FAKE, FAKE), It(FAKE, 128, 96, FAKE, 48, FAKE, FAKE)
    two = (It * 2)(a, b)
    per = [lib.owq_calibrate_workspace_bytes(64, 64, 32), lib.owq_calibrate_workspace_bytes(128, 96, 48)]
    ws = lib.owq_calibrate_batched_workspace_bytes(two, 2)
    assert ws == sum((x + 255) // 256 * 256 for x in per)
    assert lib.owq_calibrate_batched_workspace_bytes(two, 0) == 0
    assert lib.owq_calibrate_batched_workspace_bytes(None, 2) == 0
    assert lib.owq_calibrate_batched_workspace_bytes((It * 2)(a, It(FAKE, 64, 48, FAKE, 32, FAKE, FAKE)), 2) == 0
    f = lib.owq_calibrate_score_batched
    assert f(None, 2, FAKE, ws, None) == 1
    assert f(two, 2, None, ws, None) == 1
    assert f(two, 0, FAKE, ws, None) == 5
    assert f(two, 65, FAKE, ws, None) == 5
    assert f(two, 2, FAKE + 16, ws, None) == 4
    assert f(two, 2, FAKE, ws - 1, None) == 6
    assert "workspace" in _err(lib)
    assert f((It * 2)(a, It(FAKE, 128, 96, FAKE, 48, None, FAKE)), 2, FAKE, ws, None) == 1
    assert "item 1" in _err(lib)
    assert f((It * 2)(a, It(FAKE, 128, 40, FAKE, 48, FAKE, FAKE)), 2, FAKE, ws, None) == 2
    assert f((It * 2)(a, It(FAKE, 128, 96, FAKE, 0, FAKE, FAKE)), 2, FAKE, ws, None) == 2
    assert f((It * 2)(It(FAKE + 2, 64, 64, FAKE, 32, FAKE, FAKE), b), 2, FAKE, ws, None) == 4
    assert "item 0" in _err(lib)


def test_select_validation(lib):
    f = lib.owq_select_weak
    assert f(None, 64, 4, FAKE, None) == 1
    assert f(FAKE, 0, 0, FAKE, None) == 2
    assert f(FAKE, 64, 65, FAKE, None) == 3
    assert f(FAKE, 64, -1, FAKE, None) == 3
    assert f(FAKE, 64, 4, None, None) == 1
    assert f(FAKE + 4, 64, 4, FAKE, None) == 4
    assert f(FAKE, 64, 0, None, None) == 0       # k == 0: nothing to do, nothing enqueued


def test_pack_validation(lib):
    f = lib.owq_pack
    assert f(None, 8, 64, FAKE, 2, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert f(FAKE, 8, 64, None, 2, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert f(FAKE, 8, 64, FAKE, 2, FAKE, FAKE, FAKE, None, None) == 1
    assert f(FAKE, 8, 65, FAKE, 2, FAKE, FAKE, FAKE, FAKE, None) == 2
    assert f(FAKE, 8, 16, FAKE, 2, FAKE, FAKE, FAKE, FAKE, None) == 2
    assert f(FAKE, 8, 65536 + 32, FAKE, 2, FAKE, FAKE, FAKE, FAKE, None) == 2
    assert f(FAKE, 0, 64, FAKE, 2, FAKE, FAKE, FAKE, FAKE, None) == 2
    assert f(FAKE, 8, 64, FAKE, 65, FAKE, FAKE, FAKE, FAKE, None) == 3
    assert f(FAKE, 8, 64, FAKE, -2, FAKE, FAKE, FAKE, FAKE, None) == 3
    assert f(FAKE + 8, 8, 64, FAKE, 2, FAKE, FAKE, FAKE, FAKE, None) == 4
    assert f(FAKE, 8, 64, FAKE, 2, FAKE + 1, FAKE, FAKE, FAKE, None) == 4


def test_pack_batched_validation(lib):
    from mixed_precision_weight_amd import owq
    It = owq.OwqPackItem
    a = It(FAKE, 8, 64, FAKE, 2, FAKE, FAKE, FAKE, FAKE)
    f = lib.owq_pack_batched
    two = lambda x, y: (It * 2)(x, y)
    assert f(None, 2, None) == 1
    assert f(two(a, a), 0, None) == 5
    assert f(two(a, a), 65, None) == 5
    assert f(two(a, It(None, 8, 64, FAKE, 2, FAKE, FAKE, FAKE, FAKE)), 2, None) == 1
    assert "item 1" in _err(lib)
    assert f(two(a, It(FAKE, 8, 65, FAKE, 2, FAKE, FAKE, FAKE, FAKE)), 2, None) == 2
    assert f(two(a, It(FAKE, 0, 64, FAKE, 2, FAKE, FAKE, FAKE, FAKE)), 2, None) == 2
    assert f(two(a, It(FAKE, 8, 64, FAKE, 65, FAKE, FAKE, FAKE, FAKE)), 2, None) == 3
    assert f(two(It(FAKE, 8, 64, None, 2, FAKE, FAKE, FAKE, FAKE), a), 2, None) == 1
    assert "item 0" in _err(lib)
    assert f(two(a, It(FAKE + 8, 8, 64, FAKE, 2, FAKE, FAKE, FAKE, FAKE)), 2, None) == 4
    assert f(two(a, It(FAKE, 8, 64, FAKE, 2, FAKE, FAKE + 1, FAKE, FAKE)), 2, None) == 4


def test_pack_search_validation(lib):
    f = lib.owq_pack_search
    assert f(None, 8, 64, FAKE, 2, None, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert f(FAKE, 8, 64, None, 2, None, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert f(FAKE, 8, 64, FAKE, 2, None, FAKE, FAKE, FAKE, None, None) == 1
    assert f(FAKE, 8, 65, FAKE, 2, None, FAKE, FAKE, FAKE, FAKE, None) == 2
    assert f(FAKE, 0, 64, FAKE, 2, None, FAKE, FAKE, FAKE, FAKE, None) == 2
    assert f(FAKE, 8, 64, FAKE, 65, None, FAKE, FAKE, FAKE, FAKE, None) == 3
    assert f(FAKE + 8, 8, 64, FAKE, 2, None, FAKE, FAKE, FAKE, FAKE, None) == 4
    assert f(FAKE, 8, 64, FAKE, 2, FAKE + 4, FAKE, FAKE, FAKE, FAKE, None) == 4  # lambda: 8 bytes
    assert f(FAKE, 8, 64, FAKE, 2, None, FAKE + 2, FAKE, FAKE, FAKE, None) == 4


def test_pack_storage_validation(lib):
    f = lib.owq_pack_storage
    assert f(None, 8, 64, FAKE, 2, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert f(FAKE, 8, 64, FAKE, 2, None, FAKE, FAKE, FAKE, None) == 1   # codes needed unless k == K
    assert f(FAKE, 8, 65, FAKE, 2, FAKE, FAKE, FAKE, FAKE, None) == 2
    assert f(FAKE, 8, 64, FAKE, 65, FAKE, FAKE, FAKE, FAKE, None) == 3
    assert f(FAKE + 8, 8, 64, FAKE, 2, FAKE, FAKE, FAKE, FAKE, None) == 4


def test_linear_storage_validation(lib):
    from mixed_precision_weight_amd import owq
    assert lib.owq_linear_storage_workspace_bytes(4096, 32, 1) >= 2 * (4096 - 32)
    assert lib.owq_linear_storage_workspace_bytes(4096, 4097, 1) == 0
    assert lib.owq_linear_storage_workspace_bytes(4100, 32, 1) == 0
    f = lib.owq_linear_storage
    ws = lib.owq_linear_storage_workspace_bytes(64, 2, 3)
    L = _layer(owq)
    assert f(None, FAKE, 3, FAKE, FAKE, ws, None) == 1
    assert f(L, FAKE, 3, FAKE, None, ws, None) == 1
    assert f(L, FAKE, 3, FAKE, FAKE, ws - 1, None) == 6
    assert f(L, FAKE, 3, FAKE, FAKE + 16, ws, None) == 4
    assert f(_layer(owq, K=48), FAKE, 3, FAKE, FAKE, ws, None) == 2


def test_linear_storage_batched_validation(lib):
    from mixed_precision_weight_amd import owq
    P = ctypes.c_void_p
    Ls = (owq.OwqLayer * 2)(_layer(owq), _layer(owq, N=16))
    per = [lib.owq_linear_storage_workspace_bytes(64, 2, 3)] * 2
    ws = lib.owq_linear_storage_batched_workspace_bytes(Ls, 2, 3)
    assert ws == sum((b + 255) // 256 * 256 for b in per)
    assert lib.owq_linear_storage_batched_workspace_bytes(Ls, 0, 3) == 0
    assert lib.owq_linear_storage_batched_workspace_bytes(None, 2, 3) == 0
    f = lib.owq_linear_storage_batched
    two = lambda a, b: (P * 2)(a, b)
    xs, ys = two(FAKE, FAKE), two(FAKE, FAKE)
    assert f(None, xs, ys, 2, 3, FAKE, ws, None) == 1
    assert f(Ls, None, ys, 2, 3, FAKE, ws, None) == 1
    assert f(Ls, xs, ys, 0, 3, FAKE, ws, None) == 5
    assert f(Ls, xs, ys, 65, 3, FAKE, ws, None) == 5
    assert f(Ls, xs, ys, 2, 3, None, ws, None) == 1
    assert f(Ls, xs, ys, 2, 3, FAKE + 16, ws, None) == 4
    assert f(Ls, xs, ys, 2, 3, FAKE, ws - 1, None) == 6
    assert f(Ls, two(FAKE, None), ys, 2, 3, FAKE, ws, None) == 1
    assert "layer 1" in _err(lib)
    assert f((owq.OwqLayer * 2)(_layer(owq), _layer(owq, K=48)), xs, ys, 2, 3, FAKE, ws, None) == 2


def test_pack_optq_validation(lib):
    f = lib.owq_pack_optq
    ws = lib.owq_pack_optq_workspace_bytes(8, 64, 2)
    assert ws >= 2 * 64 * 64 * 8 + 8 * 64 * 8  # H (factored in place into L), L^-1, W in fp64
    assert lib.owq_pack_optq_workspace_bytes(8, 65, 2) == 0
    assert f(None, 8, 64, FAKE, 16, FAKE, 2, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None) == 1
    assert f(FAKE, 8, 64, None, 16, FAKE, 2, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None) == 1
    assert f(FAKE, 8, 64, FAKE, 0, FAKE, 2, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None) == 2
    assert f(FAKE, 8, 64, FAKE, 16, FAKE, 65, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None) == 3
    assert f(FAKE, 8, 64, FAKE, 16, FAKE, 2, FAKE, FAKE, FAKE, FAKE, FAKE + 16, ws, None) == 4
    assert f(FAKE, 8, 64, FAKE, 16, FAKE, 2, FAKE, FAKE, FAKE, FAKE, FAKE, ws - 1, None) == 6


def test_linear_backward_validation(lib):
    from mixed_precision_weight_amd import owq
    assert lib.owq_linear_backward_workspace_bytes(4096, 4096, 32) > 0
    assert lib.owq_linear_backward_workspace_bytes(4096, 4100, 32) == 0
    assert lib.owq_linear_backward_workspace_bytes(0, 4096, 32) == 0
    f = lib.owq_linear_backward
    ws = lib.owq_linear_backward_workspace_bytes(8, 64, 2)
    L = _layer(owq)
    assert f(None, FAKE, FAKE, 3, FAKE, FAKE, FAKE, ws, None) == 1
    assert f(L, FAKE, None, 3, FAKE, FAKE, FAKE, ws, None) == 1
    assert f(L, None, FAKE, 3, None, FAKE, FAKE, ws, None) == 1       # dw_weak needs x
    assert f(L, FAKE, FAKE, 3, FAKE, None, None, ws, None) == 1       # dx needs the workspace
    assert f(L, FAKE, FAKE, 3, FAKE, None, FAKE, ws - 1, None) == 6
    assert f(L, FAKE, FAKE, 3, FAKE + 1, None, FAKE, ws, None) == 4
    assert f(L, FAKE, FAKE, 0, FAKE, None, FAKE, ws, None) == 2


def test_linear_backward_batched_validation(lib):
    from mixed_precision_weight_amd import owq
    P = ctypes.c_void_p
    Ls = (owq.OwqLayer * 2)(_layer(owq), _layer(owq, N=16))
    per = [lib.owq_linear_backward_workspace_bytes(8, 64, 2), lib.owq_linear_backward_workspace_bytes(16, 64, 2)]
    ws = lib.owq_linear_backward_batched_workspace_bytes(Ls, 2)
    assert ws == sum((b + 255) // 256 * 256 for b in per)
    assert lib.owq_linear_backward_batched_workspace_bytes(Ls, 0) == 0
    assert lib.owq_linear_backward_batched_workspace_bytes(None, 2) == 0
    bad = (owq.OwqLayer * 2)(_layer(owq), _layer(owq, K=40))
    assert lib.owq_linear_backward_batched_workspace_bytes(bad, 2) == 0
    f = lib.owq_linear_backward_batched
    two = lambda a, b: (P * 2)(a, b)
    xs, dys, dxs, dws = two(FAKE, FAKE), two(FAKE, FAKE), two(FAKE, FAKE), two(FAKE, FAKE)
    assert f(None, xs, dys, 2, 3, dxs, dws, FAKE, ws, None) == 1
    assert f(Ls, xs, None, 2, 3, dxs, dws, FAKE, ws, None) == 1
    assert f(Ls, xs, dys, 0, 3, dxs, dws, FAKE, ws, None) == 5
    assert f(Ls, xs, dys, 65, 3, dxs, dws, FAKE, ws, None) == 5
    assert f(Ls, xs, two(FAKE, None), 2, 3, dxs, dws, FAKE, ws, None) == 1         # a NULL dy
    assert f(Ls, two(FAKE, None), dys, 2, 3, dxs, dws, FAKE, ws, None) == 1        # dw_weak needs x
    assert f(Ls, None, dys, 2, 3, dxs, dws, FAKE, ws, None) == 1
    assert f(Ls, xs, dys, 2, 3, dxs, dws, None, ws, None) == 1                      # dx needs the workspace
    assert f(Ls, xs, dys, 2, 3, dxs, dws, FAKE, ws - 1, None) == 6
    assert f(Ls, xs, dys, 2, 3, dxs, dws, FAKE + 16, ws, None) == 4
    assert f(Ls, xs, dys, 2, 3, two(FAKE, FAKE + 1), dws, FAKE, ws, None) == 4
    assert f(Ls, xs, dys, 2, 0, dxs, dws, FAKE, ws, None) == 2
    assert f(bad, xs, dys, 2, 3, dxs, dws, FAKE, ws, None) == 2
    # only the layers that want dx count towards the workspace
    assert f(Ls, xs, dys, 2, 3, two(FAKE, None), dws, FAKE, per[0] - 1, None) == 6


def test_select_weak_batched_validation(lib):
    I64, I32, P = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    f = lib.owq_select_weak_batched
    sc, out = (P * 2)(FAKE, FAKE), (P * 2)(FAKE, FAKE)
    Ks, ks = (I64 * 2)(64, 100), (I32 * 2)(3, 4)
    assert f(None, Ks, ks, out, 2, None) == 1
    assert f(sc, Ks, ks, None, 2, None) == 1
    assert f(sc, Ks, ks, out, 0, None) == 5
    assert f(sc, Ks, ks, out, 65, None) == 5
    assert f((P * 2)(FAKE, None), Ks, ks, out, 2, None) == 1
    assert f(sc, (I64 * 2)(64, 0), ks, out, 2, None) == 2
    assert f(sc, (I64 * 2)(64, (1 << 24) + 1), ks, out, 2, None) == 2
    assert f(sc, Ks, (I32 * 2)(3, 101), out, 2, None) == 3
    assert f(sc, Ks, (I32 * 2)(3, -1), out, 2, None) == 3
    assert f(sc, Ks, ks, (P * 2)(FAKE, None), 2, None) == 1
    assert f((P * 2)(FAKE, FAKE + 4), Ks, ks, out, 2, None) == 4
    assert f(sc, Ks, ks, (P * 2)(FAKE, FAKE + 2), 2, None) == 4


def _layer(owq, **kw):
    d = dict(N=8, K=64, k=2, bits=3, qcodes=FAKE, scales=FAKE, zeros=FAKE, weak_idx=FAKE, w_weak=FAKE)
    d.update(kw)
    return owq.OwqLayer(**d)


def test_linear_validation(lib):
    from mixed_precision_weight_amd import owq
    f = lib.owq_linear
    assert f(None, FAKE, 1, FAKE, None) == 1
    assert f(ctypes.byref(_layer(owq, bits=4)), FAKE, 1, FAKE, None) == 5
    assert f(ctypes.byref(_layer(owq, N=0)), FAKE, 1, FAKE, None) == 2
    assert f(ctypes.byref(_layer(owq, K=40)), FAKE, 1, FAKE, None) == 2
    assert f(ctypes.byref(_layer(owq)), FAKE, 0, FAKE, None) == 2
    assert f(ctypes.byref(_layer(owq, k=65)), FAKE, 1, FAKE, None) == 3
    assert f(ctypes.byref(_layer(owq, qcodes=None)), FAKE, 1, FAKE, None) == 1
    assert f(ctypes.byref(_layer(owq, weak_idx=None)), FAKE, 1, FAKE, None) == 1
    assert f(ctypes.byref(_layer(owq)), None, 1, FAKE, None) == 1
    assert f(ctypes.byref(_layer(owq)), FAKE + 8, 1, FAKE, None) == 4
    assert f(ctypes.byref(_layer(owq, qcodes=FAKE + 2)), FAKE, 1, FAKE, None) == 4


def test_linear_batched_validation(lib):
    from mixed_precision_weight_amd import owq
    f = lib.owq_linear_batched
    Ls = (owq.OwqLayer * 2)(_layer(owq), _layer(owq))
    xs = (ctypes.c_void_p * 2)(FAKE, FAKE)
    ys = (ctypes.c_void_p * 2)(FAKE, FAKE)
    assert f(None, xs, ys, 2, 1, None) == 1
    assert f(Ls, xs, ys, 0, 1, None) == 5
    assert f(Ls, xs, ys, 65, 1, None) == 5
    assert f(Ls, xs, ys, 2, 17, None) == 5  # the batched decode launch takes at most 16 tokens
    assert f(Ls, xs, ys, 2, 0, None) == 5
    Ls[1].bits = 2
    assert f(Ls, xs, ys, 2, 1, None) == 5
    assert "layer 1" in _err(lib)


def test_stream_read_validation(lib):
    f = lib.owq_stream_read
    assert lib.owq_stream_read_sink_words(4608) == 1
    assert lib.owq_stream_read_sink_words(4608 + 12) == 2
    assert lib.owq_stream_read_sink_words(0) == 0
    assert f(None, 4608, FAKE, 1, None) == 1
    assert f(FAKE, 4608, None, 1, None) == 1
    assert f(FAKE, 4600, FAKE, 1, None) == 2   # not a multiple of 12 bytes
    assert f(FAKE, 0, FAKE, 1, None) == 2
    assert f(FAKE + 2, 4608, FAKE, 1, None) == 4
    assert f(FAKE, 4620, FAKE, 1, None) == 3   # needs two sink words


def test_calibrate_noalloc_validation(lib):
    f = lib.owq_calibrate_score_noalloc
    cap = lib.owq_calibrate_noalloc_max_workspace()
    assert cap >= 1 << 20
    assert f(None, 64, 64, FAKE, 64, FAKE, FAKE, None) == 1
    assert f(FAKE, 64, 48, FAKE, 64, FAKE, FAKE, None) == 2
    assert f(FAKE, 64, 64, FAKE, 0, FAKE, FAKE, None) == 2
    assert f(FAKE + 2, 64, 64, FAKE, 64, FAKE, FAKE, None) == 4
    # sizes whose workspace exceeds the library's own are refused before any HIP call
    N = 1 << 23
    assert lib.owq_calibrate_workspace_bytes(N, 4096, 16) > cap
    assert f(FAKE, N, 4096, FAKE, 16, FAKE, FAKE, None) == 6
    assert "library's own" in _err(lib)


def test_pack_grouped_validation(lib):
    f = lib.owq_pack_grouped
    assert f(None, 8, 256, FAKE, 2, 128, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert f(FAKE, 8, 256, None, 2, 128, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert f(FAKE, 8, 255, FAKE, 2, 128, FAKE, FAKE, FAKE, FAKE, None) == 2
    assert f(FAKE, 0, 256, FAKE, 2, 128, FAKE, FAKE, FAKE, FAKE, None) == 2
    for G in (0, 16, 96, 512, 4096):  # not a power of two in [32, 2048] dividing K = 256
        assert f(FAKE, 8, 256, FAKE, 2, G, FAKE, FAKE, FAKE, FAKE, None) == 5, G
    assert f(FAKE, 8, 256, FAKE, 257, 128, FAKE, FAKE, FAKE, FAKE, None) == 3
    assert f(FAKE + 8, 8, 256, FAKE, 2, 128, FAKE, FAKE, FAKE, FAKE, None) == 4


def test_linear_grouped_validation(lib):
    from mixed_precision_weight_amd import owq

    def layer(N=8, K=256, G=128, k=2, bits=3):
        return ctypes.byref(owq.OwqGroupedLayer(N, K, G, k, bits, FAKE, FAKE, FAKE, FAKE, FAKE))

    f = lib.owq_linear_grouped
    assert f(None, FAKE, 1, FAKE, None) == 1
    assert f(layer(), None, 1, FAKE, None) == 1
    assert f(layer(K=250), FAKE, 1, FAKE, None) == 2
    assert f(layer(), FAKE, 0, FAKE, None) == 2
    assert f(layer(G=96), FAKE, 1, FAKE, None) == 5
    assert f(layer(G=512), FAKE, 1, FAKE, None) == 5
    assert f(layer(bits=4), FAKE, 1, FAKE, None) == 5
    assert f(layer(k=300), FAKE, 1, FAKE, None) == 3
    assert f(layer(), FAKE + 8, 1, FAKE, None) == 4


def test_linear_grouped_batched_validation(lib):
    from mixed_precision_weight_amd import owq
    P = ctypes.c_void_p
    Ls = (owq.OwqGroupedLayer * 2)(owq.OwqGroupedLayer(8, 256, 128, 2, 3, FAKE, FAKE, FAKE, FAKE, FAKE),
                                   owq.OwqGroupedLayer(8, 256, 96, 2, 3, FAKE, FAKE, FAKE, FAKE, FAKE))
    xs = (P * 2)(FAKE, FAKE)
    ys = (P * 2)(FAKE, FAKE)
    f = lib.owq_linear_grouped_batched
    assert f(None, xs, ys, 2, 1, None) == 1
    assert f(Ls, xs, ys, 0, 1, None) == 5
    assert f(Ls, xs, ys, 1, 5, None) == 5      # more than 4 tokens
    assert f(Ls, xs, ys, 2, 1, None) == 5      # layer 1: G = 96
    bad = (P * 2)(FAKE + 8, FAKE)
    assert f(Ls, bad, ys, 1, 1, None) == 4
