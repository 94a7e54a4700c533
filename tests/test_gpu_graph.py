"""The whole path recorded once in a HIP graph and replayed.

Calibration, weak-column selection, packing, decode on the vector ALUs
(M = 1, and M = 2 with its products on the matrix cores) and on the matrix
cores (M = 8), prefill (M = 256), and the group-wise pack and product are captured
with torch's graph API. The library launches kernels only: no allocation, no
copy-engine clears, no host synchronisation. Every replay must then equal the
eager result bit for bit, since the kernels are deterministic. The outputs are
cleared by an eager kernel before each replay, and eager runs of the same path
go in between.
"""
import pytest

from mixed_precision_weight_amd import synth
from parity_util import dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def owq():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from mixed_precision_weight_amd import owq as o
    o.lib()
    return o


def _path(owq, W, X, xs, ws, k):
    lam, score = owq.calibrate(W, X, workspace=ws)
    idx = owq.select_weak(score, k)
    p = owq.pack(W, idx)
    ys = [owq.linear(p, x) for x in xs]
    # the group-wise form (groups of 128 columns) on the same weak set
    g = owq.pack_grouped(W, idx, 128)
    yg = owq.linear_grouped_batched([g], [xs[1][:2]])[0]
    return [lam, score, idx, p["qcodes"], p["scales"], p["zeros"], p["w_weak"]] + ys + \
        [g["qcodes"], g["scales"], g["zeros"], yg]


@pytest.mark.parametrize("workload,li", [("opt125m_q_proj", 0), ("llama7b_layer_decode", 6)])
def test_graph_replay_matches_eager(owq, workload, li):
    import torch
    cfg = synth.CONFIGS[workload]
    spec = cfg.layers[li]
    seed = cfg.seed(li)
    W = dev(synth.weights(spec, seed))
    X = dev(synth.calibration(spec, seed, cfg.T))
    x = dev(synth.activations(spec, seed, 8))
    xp = dev(synth.activations(spec, seed + 500, 256))
    xs = [x[:1], x[:2], x, xp]
    ws = torch.empty(max(owq.calibrate_workspace_bytes(spec.N, spec.K, cfg.T), 256), dtype=torch.uint8,
                     device="cuda:0")
    print(f"graph replay: {cfg.name}/{spec.name} {spec.N}x{spec.K} k={spec.k} T={cfg.T}", flush=True)

    eager = [host(t).copy() for t in _path(owq, W, X, xs, ws, spec.k)]
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _path(owq, W, X, xs, ws, spec.k)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = _path(owq, W, X, xs, ws, spec.k)
    torch.cuda.synchronize()

    names = ["lambda", "score", "weak_idx", "qcodes", "scales", "zeros", "w_weak", "y(M=1)", "y(M=2)", "y(M=8)",
             "y(M=256)", "grouped qcodes", "grouped scales", "grouped zeros", "grouped y(M=2)"]
    for rep in range(3):
        for t in outs:
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for name, a, t in zip(names, eager, outs):
            assert host(t).tobytes() == a.tobytes(), f"replay {rep}: {name} differs from the eager result"
        again = _path(owq, W, X, xs, ws, spec.k)  # eager work between replays
        torch.cuda.synchronize()
        assert host(again[-5]).tobytes() == eager[-5].tobytes()
        assert host(again[-1]).tobytes() == eager[-1].tobytes()
