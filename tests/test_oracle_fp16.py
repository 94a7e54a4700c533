"""Pins of the oracle's binary16 conversions against numpy's (an independent,
library implementation of IEEE 754 binary16)."""
import numpy as np


def test_f16_decode_all_patterns(orc):
    lib = orc.load()
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([lib.owq_oracle_f16_to_f64(int(b)) for b in bits])
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(np.isinf(got) & (got > 0), np.isinf(ref) & (ref > 0))


def _encode_many(orc, vals):
    lib = orc.load()
    return np.array([lib.owq_oracle_f32_to_f16(float(v)) for v in vals], dtype=np.uint16)


def test_f32_to_f16_random(orc):
    rng = np.random.default_rng(7)
    v = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(0.05),
        (rng.standard_normal(20000) * 1e-5).astype(np.float32),     # fp16 subnormal range
        (rng.standard_normal(5000) * 3e4).astype(np.float32),       # near the fp16 max
        (rng.uniform(-1, 1, 5000) * 1e-8).astype(np.float32),       # underflow to zero
    ])
    got = _encode_many(orc, v)
    ref = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


def test_f32_to_f16_ties_and_edges(orc):
    # exact halfway points between consecutive fp16 values (normal and subnormal),
    # the overflow threshold, and signed zeros: ties must go to the even pattern
    h = np.arange(0, 0x7BFF, 97, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    mids = ((lo + hi) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (lo + hi) / 2)   # exact in fp32
    edges = np.array([65504.0, 65519.99, 65520.0, 70000.0, -65520.0, 0.0, -0.0,
                      2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14 - 2.0 ** -25],
                     dtype=np.float32)
    v = np.concatenate([mids, -mids, edges])
    got = _encode_many(orc, v)
    ref = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


def test_f64_to_f16_against_numpy(orc):
    """The binary64 -> binary16 rounding (the OPTQ weak block) against numpy's
    direct float64 -> float16 conversion: random values over the whole range,
    exact midpoints between fp16 neighbours (ties go to even) and values one
    binary64 ulp either side of them, subnormals, overflow."""
    import numpy as np
    rng = np.random.default_rng(9)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-8, 5, 20000),
                        [0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e-9, -6e-8, 2.0 ** -25, 3 * 2.0 ** -25]])
    h = rng.integers(0, 0x7BFF, 5000).astype(np.uint16).view(np.float16).astype(np.float64)
    nxt = np.nextafter(h.astype(np.float16), np.float16(np.inf)).astype(np.float64)
    mid = (h + nxt) / 2.0
    v = np.concatenate([v, mid, np.nextafter(mid, np.inf), np.nextafter(mid, -np.inf), -mid])
    got = np.array([orc.f64_to_f16(x) for x in v], np.uint16)
    ref = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)
