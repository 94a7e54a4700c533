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
