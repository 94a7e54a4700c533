"""GPU parity of the storage-favoured form (owq_pack_storage,
owq_linear_storage) against the oracle: codes, steps, zero points and the weak
block bit-exact; every output of the product within the per-output bound, at
decode (vector and matrix-core kernels) and prefill sizes, on the OPT-125m and
LLaMA-7B shapes and on edge shapes (no weak column, every column weak, K - k
not a multiple of 32, one row)."""
import numpy as np
import pytest

from mixed_precision_weight_amd import synth
from parity_util import check_linear, dev, f16_bits, host
from test_gpu_parity import _quiet_columns, _tiny_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def owq():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from mixed_precision_weight_amd import owq as o
    o.lib()
    return o


def _run(owq, W, idx, xs, what):
    import torch

    import oracle
    N, K = W.shape
    print(f"{what}: N={N} K={K} k={len(idx)}", flush=True)
    got = owq.pack_storage(dev(W), dev(np.asarray(idx, np.int32)))
    torch.cuda.synchronize()
    ref = oracle.pack_storage(W, idx)
    assert np.array_equal(host(got["qcodes"]).view(np.uint32), ref["qcodes"]), "qcodes differ"
    assert np.array_equal(f16_bits(got["scales"]), ref["scales"]), "scales differ"
    assert np.array_equal(host(got["zeros"]), ref["zeros"]), "zeros differ"
    assert np.array_equal(f16_bits(got["w_weak"]).reshape(ref["w_weak"].shape), ref["w_weak"]), "w_weak differ"
    for x in xs:
        y = host(owq.linear_storage(got, dev(x)))
        yr, b = oracle.linear_storage_rows(ref, x)
        check_linear(y, yr, b, f"{what} storage M={x.shape[0]}")


def test_small_workload(owq):
    import oracle
    cfg = synth.OPT125M_Q_PROJ
    spec = cfg.layers[0]
    W = synth.weights(spec, cfg.seed(0))
    _, score = oracle.calibrate_score(W, synth.calibration(spec, cfg.seed(0), cfg.T))
    idx = oracle.select_weak(score, spec.k)
    x = synth.activations(spec, cfg.seed(0), 64)
    _run(owq, W, idx, [x[:1], x[:2], x[:5], x[:16], x], cfg.name)


@pytest.mark.parametrize("li", [0, 4, 6])
def test_llama7b_linears(owq, li):
    import oracle
    cfg = synth.LLAMA7B_LAYER_DECODE
    spec = cfg.layers[li]
    seed = cfg.seed(li)
    W = synth.weights(spec, seed)
    _, score = oracle.calibrate_score(W, synth.calibration(spec, seed, cfg.T))
    idx = oracle.select_weak(score, spec.k)
    x = synth.activations(spec, seed, 16)
    _run(owq, W, idx, [x[:1], x[:8]], f"{cfg.name}/{spec.name}")


EDGE = [
    # N, K, k, Ms
    (1, 32, 0, (1,)),
    (1, 32, 32, (1, 3)),
    (7, 64, 64, (1, 20)),
    (5, 96, 1, (1, 3, 4)),
    (37, 4128, 17, (1, 5, 33)),
    (130, 8192, 63, (1, 4, 130)),
    (64, 640, 7, (2, 17)),
]


@pytest.mark.parametrize("N,K,k,Ms", EDGE)
def test_edge_shapes(owq, N, K, k, Ms):
    rng = np.random.default_rng(N * 13 + K + k)
    W = _tiny_rows(synth.random_layer(rng, N, K, 0.02))
    idx = np.sort(rng.choice(K, k, replace=False)).astype(np.int32)
    spec = synth.LayerSpec("edge", N, K, k, 0.02, max(1, K // 200), 20.0)
    x = _quiet_columns(synth.activations(spec, N + K + 3, max(Ms)))
    _run(owq, W, idx, [x[:m] for m in Ms], "edge")


def test_batched_matches_per_layer(owq):
    """owq_linear_storage_batched (three launches for all the layers) gives every
    layer's owq_linear_storage output bit for bit: layers of several K, one with
    no weak column and one with every column weak, at decode M (vector and
    matrix-core kernels, one launch for all) and at a prefill M (per-layer GEMM)."""
    import torch
    shapes = [(37, 4096, 32), (300, 4128, 17), (5, 96, 0), (7, 64, 64), (64, 11008, 86), (1, 32, 1)]
    rng = np.random.default_rng(31)
    layers = []
    for N, K, k in shapes:
        W = _tiny_rows(synth.random_layer(rng, N, K, 0.02))
        idx = np.sort(rng.choice(K, k, replace=False)).astype(np.int32)
        layers.append(owq.pack_storage(dev(W), dev(idx)))
    for M in (1, 2, 5, 16, 40):
        print(f"storage batched: M={M}", flush=True)
        xs = [dev(_quiet_columns(synth.activations(synth.LayerSpec("b", N, K, k, 0.02, max(1, K // 200), 20.0),
                                                   N + K + M, M))) for N, K, k in shapes]
        single = [owq.linear_storage(l, x) for l, x in zip(layers, xs)]
        got = owq.linear_storage_batched(layers, xs)
        torch.cuda.synchronize()
        for i in range(len(shapes)):
            assert host(got[i]).tobytes() == host(single[i]).tobytes(), (M, shapes[i])
