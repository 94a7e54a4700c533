"""GPU parity of the weak-column-tuning backward (owq_linear_backward) against
the oracle: every element of dx = dy W (fp16) and of dw_weak = dy^T x[:, idx]
(fp32) within |g - g_ref| <= 2e-3 * sum |terms| + 1e-5, on the OPT-125m and
LLaMA-7B shapes and on edge shapes (no weak column, every column weak, odd
group counts, one row, K = 65536), for token counts that cover the 4-token
chunks and their ragged ends; dx is bitwise the same on a second call."""
import numpy as np
import pytest

from mixed_precision_weight_amd import synth
from parity_util import check_linear, dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def owq():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from mixed_precision_weight_amd import owq as o
    o.lib()
    return o


def _run(owq, W, idx, M, what, seed=0):
    import torch

    import oracle
    N, K = W.shape
    rng = np.random.default_rng(seed + N + K + M)
    x = rng.standard_normal((M, K)).astype(np.float16)
    dy = rng.standard_normal((M, N)).astype(np.float16)
    print(f"{what}: N={N} K={K} k={len(idx)} M={M}", flush=True)
    p_ref = oracle.pack(W, idx)
    p = owq.pack(dev(W), dev(np.asarray(idx, np.int32)))
    dx, dw = owq.linear_backward(p, dev(x), dev(dy))
    dx2, _ = owq.linear_backward(p, dev(x), dev(dy), want_dw=False)
    torch.cuda.synchronize()
    rdx, rdxb, rdw, rdwb = oracle.linear_backward(p_ref, x, dy)
    check_linear(host(dx), rdx, rdxb, f"{what} dx M={M}")
    assert host(dx).tobytes() == host(dx2).tobytes()
    if len(idx):
        check_linear(host(dw), rdw, rdwb, f"{what} dw M={M}")
    else:
        assert tuple(dw.shape) == (N, 0)


def test_small_workload(owq):
    import oracle
    cfg = synth.OPT125M_Q_PROJ
    spec = cfg.layers[0]
    W = synth.weights(spec, cfg.seed(0))
    _, score = oracle.calibrate_score(W, synth.calibration(spec, cfg.seed(0), cfg.T))
    idx = oracle.select_weak(score, spec.k)
    for M in (1, 3, 4, 7, 64):
        _run(owq, W, idx, M, cfg.name)


@pytest.mark.parametrize("li", [0, 4, 6])
def test_llama7b_linears(owq, li):
    import oracle
    cfg = synth.LLAMA7B_LAYER_DECODE
    spec = cfg.layers[li]
    seed = cfg.seed(li)
    W = synth.weights(spec, seed)
    _, score = oracle.calibrate_score(W, synth.calibration(spec, seed, cfg.T))
    idx = oracle.select_weak(score, spec.k)
    for M in (1, 16):
        _run(owq, W, idx, M, f"{cfg.name}/{spec.name}")


EDGE = [
    # N, K, k, M
    (1, 32, 0, 1),
    (1, 32, 32, 2),
    (7, 64, 64, 5),
    (5, 96, 1, 3),
    (37, 4128, 17, 6),
    (300, 2048, 0, 4),
    (3, 65536, 5, 2),
    (130, 8192, 63, 9),
]


@pytest.mark.parametrize("N,K,k,M", EDGE)
def test_edge_shapes(owq, N, K, k, M):
    rng = np.random.default_rng(N * 5 + K + k)
    W = synth.random_layer(rng, N, K, 0.02)
    idx = np.sort(rng.choice(K, k, replace=False)).astype(np.int32)
    _run(owq, W, idx, M, "edge", seed=1)
