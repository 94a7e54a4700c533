"""GPU parity at the full workload sizes: one LLaMA-7B decoder layer (decode,
batch sweep, batched launch), the large 8192/28672 shapes, and prefill plus
long calibration at the MLP shapes. Inputs come from the seeded generator.
Every output of every call is checked against the oracle (its linear runs
the rows on all host cores); none is sampled."""
import numpy as np
import pytest

from mixed_precision_weight_amd import synth
from parity_util import check_linear, dev, host
from test_gpu_parity import _run

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def owq():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from mixed_precision_weight_amd import owq as o
    o.lib()
    return o


def _inputs(cfg, li, M):
    spec = cfg.layers[li]
    seed = cfg.seed(li)
    return (spec, synth.weights(spec, seed), synth.calibration(spec, seed, cfg.T),
            synth.activations(spec, seed, M))


@pytest.mark.parametrize("li", range(7))
def test_llama7b_layer_decode(owq, li):
    cfg = synth.LLAMA7B_LAYER_DECODE
    spec, W, X, x = _inputs(cfg, li, 1)
    _run(owq, W, X, spec.k, [x], f"{cfg.name}/{spec.name}")


@pytest.mark.parametrize("li", range(7))
def test_llama7b_batch_sweep(owq, li):
    cfg = synth.LLAMA7B_BATCH_SWEEP
    spec, W, X, x = _inputs(cfg, li, 16)
    _run(owq, W, X, spec.k, [x[:m] for m in cfg.Ms], f"{cfg.name}/{spec.name}")


def test_llama7b_layer_batched_launch(owq):
    """One launch over the 7 linears equals the 7 single launches bit for bit."""
    import torch
    import oracle
    cfg = synth.LLAMA7B_LAYER_DECODE
    layers, xs, singles = [], [], []
    for li, spec in enumerate(cfg.layers):
        seed = cfg.seed(li)
        W = synth.weights(spec, seed)
        idx = np.sort(np.random.default_rng(li).choice(spec.K, spec.k, replace=False)).astype(np.int32)
        p = owq.pack(dev(W), dev(idx))
        x = dev(synth.activations(spec, seed, 1))
        layers.append(p)
        xs.append(x)
        singles.append(owq.linear(p, x))
    ys = owq.linear_batched(layers, xs)
    yp = [torch.zeros_like(y) for y in ys]
    call = owq.PreparedBatched(layers, xs, yp)  # arguments marshalled once, called twice
    call()
    call()
    torch.cuda.synchronize()
    for a, b, c in zip(ys, singles, yp):
        assert host(a).tobytes() == host(b).tobytes()
        assert host(c).tobytes() == host(b).tobytes()
    # and the batched outputs meet the oracle bound
    o = oracle.pack(synth.weights(cfg.layers[6], cfg.seed(6)), host(layers[6]["weak_idx"]))
    yr, bnd = oracle.linear_rows(o, host(xs[6]))
    check_linear(host(ys[6]), yr, bnd, "batched down_proj")


@pytest.mark.parametrize("g", [0, 7])
def test_llama7b_layer_shard_g8(owq, g):
    """One GPU's share at 8-way column-parallel sharding: rows [g N/8, (g+1) N/8)
    of each of the 7 packed linears, decoded in one batched launch at M = 1,
    equal bit for bit to the same rows of the full layer's output, and every
    output within the oracle's bound."""
    import torch
    import oracle
    cfg = synth.LLAMA7B_LAYER_DECODE
    full, shard, xs, Ws = [], [], [], []
    for li, spec in enumerate(cfg.layers):
        seed = cfg.seed(li)
        W = synth.weights(spec, seed)
        idx = np.sort(np.random.default_rng(li).choice(spec.K, spec.k, replace=False)).astype(np.int32)
        p = owq.pack(dev(W), dev(idx))
        a, b = (spec.N // 8) * g, (spec.N // 8) * (g + 1)
        shard.append({key: (v if key == "weak_idx" else v[a:b].clone()) for key, v in p.items()})
        full.append(p)
        xs.append(dev(synth.activations(spec, seed, 1)))
        Ws.append((W[a:b], idx))
    print(f"shard g={g} of 8: rows {[s.N // 8 for s in cfg.layers]}", flush=True)
    yf = owq.linear_batched(full, xs)
    ys = owq.linear_batched(shard, xs)
    torch.cuda.synchronize()
    for li, spec in enumerate(cfg.layers):
        a, b = (spec.N // 8) * g, (spec.N // 8) * (g + 1)
        assert host(ys[li]).tobytes() == host(yf[li])[:, a:b].tobytes(), spec.name
        Wsh, idx = Ws[li]
        yr, bnd = oracle.linear_rows(oracle.pack(np.ascontiguousarray(Wsh), idx), host(xs[li]))
        check_linear(host(ys[li]), yr, bnd, f"shard {g} {spec.name}")


@pytest.mark.parametrize("li", range(3))
def test_large_shapes(owq, li):
    cfg = synth.LARGE_SHAPES
    spec, W, X, x = _inputs(cfg, li, 8)
    _run(owq, W, X, spec.k, [x[:1], x], f"{cfg.name}/{spec.name}")


@pytest.mark.parametrize("li", range(2))
def test_prefill_and_long_calibration(owq, li):
    cfg = synth.LLAMA7B_MLP_PREFILL_CALIB
    spec, W, X, x = _inputs(cfg, li, 2048)
    _run(owq, W, X, spec.k, [x], f"{cfg.name}/{spec.name}")
