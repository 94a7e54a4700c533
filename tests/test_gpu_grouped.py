"""GPU parity of the group-wise form (owq_pack_grouped, owq_linear_grouped)
against the oracle: codes, per-group steps and zero points and the weak block
bit-exact; every output of the product within the per-output bound, for one to
nine tokens (token slices of four), at the OPT-125m and LLaMA-7B shapes with the
pages' group size of 128, and on edge shapes (one code group per scale group,
2048-column groups, no weak column, every column weak, a group of weak columns
only, a group of zeros, one row)."""
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


def _run(owq, W, idx, G, xs, what):
    import torch

    import oracle
    N, K = W.shape
    print(f"{what}: N={N} K={K} k={len(idx)} G={G}", flush=True)
    got = owq.pack_grouped(dev(W), dev(np.asarray(idx, np.int32)), G)
    torch.cuda.synchronize()
    ref = oracle.pack_grouped(W, idx, G)
    assert np.array_equal(host(got["qcodes"]).view(np.uint32), ref["qcodes"]), "qcodes differ"
    assert np.array_equal(f16_bits(got["scales"]).reshape(ref["scales"].shape), ref["scales"]), "scales differ"
    assert np.array_equal(host(got["zeros"]), ref["zeros"]), "zeros differ"
    assert np.array_equal(f16_bits(got["w_weak"]).reshape(ref["w_weak"].shape), ref["w_weak"]), "w_weak differ"
    for x in xs:
        y = host(owq.linear_grouped(got, dev(x)))
        yr, b = oracle.linear_grouped_rows(ref, x)
        check_linear(y, yr, b, f"{what} grouped M={x.shape[0]}")


@pytest.mark.parametrize("G", [128, 256])
def test_small_workload(owq, G):
    import oracle
    cfg = synth.OPT125M_Q_PROJ
    spec = cfg.layers[0]
    W = synth.weights(spec, cfg.seed(0))
    _, score = oracle.calibrate_score(W, synth.calibration(spec, cfg.seed(0), cfg.T))
    idx = oracle.select_weak(score, spec.k)
    x = synth.activations(spec, cfg.seed(0), 9)
    _run(owq, W, idx, G, [x[:1], x[:2], x[:3], x[:4], x], cfg.name)


@pytest.mark.parametrize("li", [0, 4, 6])
def test_llama7b_linears(owq, li):
    import oracle
    cfg = synth.LLAMA7B_LAYER_DECODE
    spec = cfg.layers[li]
    seed = cfg.seed(li)
    W = synth.weights(spec, seed)
    _, score = oracle.calibrate_score(W, synth.calibration(spec, seed, cfg.T))
    idx = oracle.select_weak(score, spec.k)
    x = synth.activations(spec, seed, 4)
    _run(owq, W, idx, 128, [x[:1], x], f"{cfg.name}/{spec.name}")


EDGE = [
    # N, K, k, G, Ms
    (1, 32, 0, 32, (1,)),
    (1, 64, 64, 32, (1, 3)),
    (5, 96, 1, 32, (1, 2, 4)),
    (64, 640, 7, 128, (2, 5)),
    (37, 4096, 130, 2048, (1, 4)),
    (130, 8192, 63, 64, (1, 3)),
]


@pytest.mark.parametrize("N,K,k,G,Ms", EDGE)
def test_edge_shapes(owq, N, K, k, G, Ms):
    rng = np.random.default_rng(N * 7 + K + k + G)
    W = _tiny_rows(synth.random_layer(rng, N, K, 0.02))
    idx = np.sort(rng.choice(K, k, replace=False)).astype(np.int32)
    spec = synth.LayerSpec("edge", N, K, k, 0.02, max(1, K // 200), 20.0)
    x = _quiet_columns(synth.activations(spec, N + K + 11, max(Ms)))
    _run(owq, W, idx, G, [x[:m] for m in Ms], f"edge N={N} K={K} k={k} G={G}")


def test_degenerate_groups(owq):
    """A group of weak columns only and a group of zeros: step 1, zero point 0."""
    N, K, G = 6, 256, 64
    rng = np.random.default_rng(12)
    W = synth.random_layer(rng, N, K, 0.02)
    W[:, 128:192] = np.float16(0.0)
    idx = np.concatenate([np.arange(64, 128), [200, 255]]).astype(np.int32)
    x = synth.activations(synth.LayerSpec("deg", N, K, len(idx), 0.02, 2, 20.0), 13, 2)
    _run(owq, W, idx, G, [x[:1], x], "degenerate groups")


@pytest.mark.parametrize("M", [1, 3])
def test_batched_matches_single(owq, M):
    """owq_linear_grouped_batched: several group-wise layers of different shapes
    and group sizes in one launch give the single calls' outputs bit for bit."""
    import torch
    rng = np.random.default_rng(40 + M)
    layers, xs = [], []
    for N, K, k, G in [(37, 4096, 130, 2048), (64, 640, 7, 128), (5, 96, 1, 32), (130, 8192, 63, 64), (16, 256, 0, 256)]:
        W = synth.random_layer(rng, N, K, 0.02)
        idx = np.sort(rng.choice(K, k, replace=False)).astype(np.int32)
        layers.append(owq.pack_grouped(dev(W), dev(idx), G))
        xs.append(dev((rng.standard_normal((M, K)) * 2).astype(np.float16)))
    print(f"grouped batched: {len(layers)} layers, M={M}", flush=True)
    singles = [owq.linear_grouped(p, x) for p, x in zip(layers, xs)]
    ys = owq.linear_grouped_batched(layers, xs)
    torch.cuda.synchronize()
    for li, (a, b) in enumerate(zip(ys, singles)):
        assert host(a).tobytes() == host(b).tobytes(), f"layer {li} M={M}"
