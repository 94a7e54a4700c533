"""Pins of the bit accounting and weak-column storage shape against figures the
pages print (tests/golden/pages_figures.json carries each figure's source)."""
import json
import os

import numpy as np
import pytest

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")))


def _rounds_to(value, printed, digits):
    return round(value, digits) == printed


def test_latency_favored_bits(orc):
    g = GOLDEN["latency_vs_storage_bits"]
    # k/K that gives 3.01 storage-favoured bits: 13 k / K = 0.01  ->  K = 1300 k
    K, k = 1300, 1
    assert orc.effective_bits(K, k, False) == pytest.approx(g["storage_favored_bits"], abs=1e-12)
    lat = orc.effective_bits(K, k, True)
    assert _rounds_to(lat, g["latency_favored_bits"], g["printed_digits"])
    # a 13-bit (storage) count for the latency format would print 3.010, not 3.012
    assert not _rounds_to(orc.effective_bits(K, k, False), g["latency_favored_bits"], g["printed_digits"])


def test_memory_overhead_at_3005(orc):
    g = GOLDEN["memory_overhead_at_3005_bits"]
    K, k = 2600, 1      # 13 k / K = 0.005
    assert orc.effective_bits(K, k, False) == pytest.approx(g["storage_favored_bits"], abs=1e-12)
    overhead = 100 * (orc.effective_bits(K, k, True) - 3.0) / 3.0
    assert _rounds_to(overhead, g["memory_overhead_percent"], g["printed_digits"])
    wrong = 100 * (orc.effective_bits(K, k, False) - 3.0) / 3.0
    assert not _rounds_to(wrong, g["memory_overhead_percent"], g["printed_digits"])


@pytest.mark.slow
def test_wct_param_ratio_from_emitted_shapes(orc):
    """The fp16 weak block of each linear is [N_out][k]: summed over the seven
    LLaMA-7B linears it is 6.8 % of rank-r LoRA's r (N_in + N_out) parameters."""
    g = GOLDEN["wct_learnable_param_ratio"]
    d, D, r, k = g["d"], g["D"], g["r"], g["k"]
    shapes = [(d, d)] * 4 + [(D, d)] * 2 + [(d, D)]        # (N_out, N_in)
    wct = 0
    lora = 0
    for N, K in shapes:
        p = orc.pack(np.zeros((N, K), np.float16), np.arange(k, dtype=np.int32))
        wct += p["w_weak"].size
        lora += r * (N + K)
    assert _rounds_to(100 * wct / lora, g["percent"], g["printed_digits"])
    # the transposed shape [N_in][k] would not reproduce the figure
    wct_t = sum(K * k for _, K in shapes)
    assert not _rounds_to(100 * wct_t / lora, g["percent"], g["printed_digits"])
