"""MI355X-native OWQ hot path: 3-bit mixed-precision linear layer and its
calibration (Hessian diagonal, column sensitivity, weak-column selection).

Every step runs in hand-written HIP kernels for gfx950 behind the C ABI of
``libowq.so`` (declared in ``include/owq.h``); ``mixed_precision_weight_amd.owq``
is the thin ctypes binding over it. ``synth`` draws the seeded synthetic
workloads. Importing the package loads nothing; the library is opened on the
first call and a missing library is an error, never a fallback.
"""

__all__ = ["owq", "synth"]
