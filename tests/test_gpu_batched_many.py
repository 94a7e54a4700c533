"""Batched decode beyond one launch, and the matrix-core override at M <= 2.

owq_linear_batched takes up to 64 layers and launches once per 16. Twenty layers
of mixed shapes (K of one and of several 4096-column chunks, group counts that
leave ragged tiles, k = 0, k > 128, N = 1 and ragged row blocks) must give, for
every layer, the bytes its single owq_linear call gives, on the vector-ALU
decode (M = 1, 2) and on the matrix-core decode (M = 5, 16). OWQ_DECODE=matrix
sends M = 1 and 2 to the matrix-core kernel, which must meet the oracle's bar.
"""
import numpy as np
import pytest

from mixed_precision_weight_amd import synth
from parity_util import dev, host
from test_gpu_parity import _run, _tiny_rows

pytestmark = pytest.mark.gpu

# N, K, k
SHAPES = [(37, 4096, 32), (1, 32, 0), (64, 640, 130), (130, 8192, 63), (5, 96, 1), (200, 4128, 17),
          (64, 11008, 86), (7, 64, 64), (33, 12288, 200), (300, 1024, 0)]


@pytest.fixture(scope="module")
def owq():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from mixed_precision_weight_amd import owq as o
    o.lib()
    return o


@pytest.mark.parametrize("M", [1, 2, 5, 16])
def test_twenty_layers_match_single_launches(owq, M):
    import torch
    rng = np.random.default_rng(M)
    layers, xs, singles = [], [], []
    for li in range(20):
        N, K, k = SHAPES[li % len(SHAPES)]
        W = synth.random_layer(rng, N, K, 0.02)
        idx = np.sort(rng.choice(K, k, replace=False)).astype(np.int32)
        p = owq.pack(dev(W), dev(idx))
        x = dev((rng.standard_normal((M, K)) * 2).astype(np.float16))
        layers.append(p)
        xs.append(x)
    print(f"batched: 20 layers, M={M}", flush=True)
    for p, x in zip(layers, xs):
        singles.append(owq.linear(p, x))
    ys = owq.linear_batched(layers, xs)
    torch.cuda.synchronize()
    for li, (a, b) in enumerate(zip(ys, singles)):
        assert host(a).tobytes() == host(b).tobytes(), f"layer {li} {SHAPES[li % len(SHAPES)]} M={M}"


@pytest.mark.parametrize("N,K,k", [(5, 96, 1), (37, 11008, 86), (130, 8192, 63), (64, 640, 130)])
def test_matrix_override_one_and_two_tokens(owq, monkeypatch, N, K, k):
    monkeypatch.setenv("OWQ_DECODE", "matrix")
    rng = np.random.default_rng(N * 31 + K + k)
    W = _tiny_rows(synth.random_layer(rng, N, K, 0.02))
    spec = synth.LayerSpec("edge", N, K, k, 0.02, max(1, K // 200), 20.0)
    X = synth.calibration(spec, N + K, 24)
    x = synth.activations(spec, N + K + 3, 2)
    _run(owq, W, X, k, [x[:1], x[:2]], f"matrix override N={N} K={K} k={k}")
