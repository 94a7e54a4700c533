"""GPU parity of OPTQ with the weak columns last (owq_pack_optq) against the
oracle: codes, steps, zero points and the compensated fp16 weak block
bit-exact, on the OPT-125m workload, the LLaMA-7B q_proj shape (T = 2048
calibration tokens) and edge shapes (one batch boundary, no weak column, every
column weak, zero calibration columns, one row); the linear on an OPTQ pack
meets the per-output bound."""
import numpy as np
import pytest

from mixed_precision_weight_amd import synth
from parity_util import check_linear, check_pack, dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def owq():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from mixed_precision_weight_amd import owq as o
    o.lib()
    return o


def _run(owq, W, X, idx, what, x=None):
    import torch

    import oracle
    print(f"{what}: N={W.shape[0]} K={W.shape[1]} T={X.shape[0]} k={len(idx)}", flush=True)
    got = owq.pack_optq(dev(W), dev(X), dev(np.asarray(idx, np.int32)))
    torch.cuda.synchronize()
    print(f"{what}: GPU done; oracle", flush=True)
    ref = oracle.optq_pack(W, X, idx)
    check_pack(got, ref)
    if x is not None:
        y = host(owq.linear(got, dev(x)))
        yr, b = oracle.linear_rows(ref, x)
        check_linear(y, yr, b, f"{what} OPTQ pack")


def test_small_workload(owq):
    import oracle
    cfg = synth.OPT125M_Q_PROJ
    spec = cfg.layers[0]
    W = synth.weights(spec, cfg.seed(0))
    X = synth.calibration(spec, cfg.seed(0), cfg.T)
    _, score = oracle.calibrate_score(W, X)
    idx = oracle.select_weak(score, spec.k)
    _run(owq, W, X, idx, cfg.name, synth.activations(spec, cfg.seed(0), 4))


def test_llama7b_q_proj(owq):
    import oracle
    cfg = synth.LLAMA7B_LAYER_DECODE
    spec = cfg.layers[0]
    W = synth.weights(spec, cfg.seed(0))
    X = synth.calibration(spec, cfg.seed(0), cfg.T)
    _, score = oracle.calibrate_score(W, X)
    idx = oracle.select_weak(score, spec.k)
    _run(owq, W, X, idx, f"{cfg.name}/{spec.name}", synth.activations(spec, cfg.seed(0), 1))


EDGE = [
    # N, K, T, k
    (1, 32, 40, 0),
    (6, 64, 100, 64),
    (9, 96, 200, 0),
    (12, 160, 300, 9),
    (33, 288, 256, 17),
]


@pytest.mark.parametrize("N,K,T,k", EDGE)
def test_edge_shapes(owq, N, K, T, k):
    rng = np.random.default_rng(N * 7 + K + T + k)
    W = synth.random_layer(rng, N, K, 0.02)
    spec = synth.LayerSpec("edge", N, K, k, 0.02, max(1, K // 32), 20.0)
    X = synth.calibration(spec, N + K, T)
    if K >= 96:
        X[:, [5, 50]] = 0  # columns no calibration token touches: their Hessian diagonal is 0
    idx = np.sort(rng.choice(K, k, replace=False)).astype(np.int32)
    _run(owq, W, X, idx, "edge")
