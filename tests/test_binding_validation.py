"""CPU tests of the Python binding's argument checks.

The binding is the one layer that sees tensor shapes, so it must reject a
mismatched shape, dtype or layout before anything reaches the library: a
narrower x or X would make the kernels read past the allocation, a smaller y
write past it. These run on host tensors: a shape mistake must be reported as
such (ValueError / TypeError naming the argument), and a call whose shapes are
right must stop at the device check, never at a launch."""
import pytest
import torch

from mixed_precision_weight_amd import owq

N, K, k = 64, 128, 4


def _layer(N=N, K=K, k=k):
    return {"qcodes": torch.zeros((N, K // 32, 3), dtype=torch.int32),
            "scales": torch.zeros(N, dtype=torch.float16),
            "zeros": torch.zeros(N, dtype=torch.uint8),
            "w_weak": torch.zeros((N, k), dtype=torch.float16),
            "weak_idx": torch.arange(k, dtype=torch.int32)}


def _host_only(fn, *a, **kw):
    """Shapes are right: the call must stop at the device check."""
    with pytest.raises(TypeError, match="CUDA"):
        fn(*a, **kw)


def test_calibrate_checks_shapes():
    W = torch.zeros((N, K), dtype=torch.float16)
    with pytest.raises(ValueError, match="columns"):
        owq.calibrate(W, torch.zeros((16, K - 32), dtype=torch.float16))
    with pytest.raises(ValueError, match="2-D"):
        owq.calibrate(W, torch.zeros(K, dtype=torch.float16))
    with pytest.raises(TypeError, match="float16"):
        owq.calibrate(W.float(), torch.zeros((16, K), dtype=torch.float16))
    with pytest.raises(ValueError, match="contiguous"):
        owq.calibrate(torch.zeros((K, N), dtype=torch.float16).t(), torch.zeros((16, N), dtype=torch.float16))
    with pytest.raises(TypeError, match="uint8"):
        owq.calibrate(W, torch.zeros((16, K), dtype=torch.float16), workspace=torch.zeros(64))
    _host_only(owq.calibrate, W, torch.zeros((16, K), dtype=torch.float16))


def test_calibrate_batched_checks_shapes():
    W = torch.zeros((N, K), dtype=torch.float16)
    X = torch.zeros((16, K), dtype=torch.float16)
    with pytest.raises(ValueError, match="one X per W"):
        owq.calibrate_batched([W, W], [X])
    with pytest.raises(ValueError, match=r"\[1\] X has"):
        owq.calibrate_batched([W, W], [X, torch.zeros((16, K - 32), dtype=torch.float16)])
    with pytest.raises(TypeError, match=r"\[0\] W must be torch.float16"):
        owq.calibrate_batched([W.float(), W], [X, X])
    _host_only(owq.calibrate_batched, [W, W], [X, X])


def test_pack_batched_checks_shapes():
    W = torch.zeros((N, K), dtype=torch.float16)
    ix = torch.arange(k, dtype=torch.int32)
    with pytest.raises(ValueError, match="one weak_idx"):
        owq.pack_batched([W, W], [ix])
    with pytest.raises(ValueError, match=r"\[1\] K = 40"):
        owq.pack_batched([W, torch.zeros((N, 40), dtype=torch.float16)], [ix, ix])
    with pytest.raises(TypeError, match=r"\[0\] weak_idx must be torch.int32"):
        owq.pack_batched([W, W], [ix.long(), ix])
    bad = _layer()
    bad["scales"] = torch.zeros(N + 1, dtype=torch.float16)
    with pytest.raises(ValueError, match=r"\[1\] out\['scales'\]"):
        owq.pack_batched([W, W], [ix, ix], outs=[_layer(), bad])
    _host_only(owq.pack_batched, [W, W], [ix, ix])


def test_linear_storage_batched_checks_shapes():
    L = _layer()
    L["qcodes"] = torch.zeros((N, (K - k + 31) // 32, 3), dtype=torch.int32)
    L["K"] = K
    x = torch.zeros((2, K), dtype=torch.float16)
    with pytest.raises(ValueError, match="one x"):
        owq.linear_storage_batched([L, L], [x])
    with pytest.raises(ValueError, match=r"\[1\] x has"):
        owq.linear_storage_batched([L, L], [x, torch.zeros((2, K - 32), dtype=torch.float16)])
    with pytest.raises(ValueError, match="same M"):
        owq.linear_storage_batched([L, L], [x, torch.zeros((3, K), dtype=torch.float16)])
    _host_only(owq.linear_storage_batched, [L, L], [x, x])


def test_select_checks_k_and_out():
    s = torch.zeros(K, dtype=torch.float64)
    with pytest.raises(ValueError, match="outside"):
        owq.select_weak(s, K + 1)
    with pytest.raises(ValueError, match="outside"):
        owq.select_weak(s, -1)
    with pytest.raises(ValueError, match="at least"):
        owq.select_weak(s, 8, out=torch.zeros(4, dtype=torch.int32))
    with pytest.raises(ValueError, match="1-D"):
        owq.select_weak(s.view(2, -1), 4)
    _host_only(owq.select_weak, s, 8)


def test_pack_checks_out_shapes():
    W = torch.zeros((N, K), dtype=torch.float16)
    idx = torch.arange(k, dtype=torch.int32)
    bad = _layer()
    bad["w_weak"] = torch.zeros((N, k - 1), dtype=torch.float16)
    with pytest.raises(ValueError, match="w_weak"):
        owq.pack(W, idx, out=bad)
    bad = _layer()
    bad["qcodes"] = torch.zeros((N - 1, K // 32, 3), dtype=torch.int32)
    with pytest.raises(ValueError, match="qcodes"):
        owq.pack(W, idx, out=bad)
    bad = _layer()
    bad["zeros"] = torch.zeros(N, dtype=torch.int32)
    with pytest.raises(TypeError, match="zeros"):
        owq.pack(W, idx, out=bad)
    with pytest.raises(ValueError, match="multiple of 32"):
        owq.pack(torch.zeros((N, K - 16), dtype=torch.float16), idx)
    _host_only(owq.pack, W, idx, out=_layer())


def test_linear_checks_x_y_and_layer():
    L = _layer()
    with pytest.raises(ValueError, match="columns"):
        owq.linear(L, torch.zeros((1, K - 32), dtype=torch.float16))
    with pytest.raises(ValueError, match="y has shape"):
        owq.linear(L, torch.zeros((2, K), dtype=torch.float16), torch.zeros((1, N), dtype=torch.float16))
    with pytest.raises(ValueError, match="y has shape"):
        owq.linear(L, torch.zeros((2, K), dtype=torch.float16), torch.zeros((2, N - 1), dtype=torch.float16))
    with pytest.raises(TypeError, match="y must be"):
        owq.linear(L, torch.zeros((2, K), dtype=torch.float16), torch.zeros((2, N), dtype=torch.float32))
    with pytest.raises(ValueError, match="contiguous"):
        owq.linear(L, torch.zeros((K, 2), dtype=torch.float16).t())
    bad = _layer()
    bad["scales"] = torch.zeros(N - 1, dtype=torch.float16)
    with pytest.raises(ValueError, match="scales"):
        owq.linear(bad, torch.zeros((1, K), dtype=torch.float16))
    bad = _layer()
    bad["weak_idx"] = torch.arange(k + 1, dtype=torch.int32)  # w_weak still holds k columns
    with pytest.raises(ValueError, match="w_weak"):
        owq.linear(bad, torch.zeros((1, K), dtype=torch.float16))
    _host_only(owq.linear, L, torch.zeros((3, K), dtype=torch.float16))
    _host_only(owq.linear, L, torch.zeros(K, dtype=torch.float16))


def test_batched_checks_common_m_and_counts():
    Ls = [_layer(), _layer(N=32, K=256, k=2)]
    xs = [torch.zeros((2, K), dtype=torch.float16), torch.zeros((2, 256), dtype=torch.float16)]
    with pytest.raises(ValueError, match="rows, the batch has M"):
        owq.linear_batched(Ls, [xs[0], torch.zeros((3, 256), dtype=torch.float16)])
    with pytest.raises(ValueError, match="as many"):
        owq.linear_batched(Ls, xs[:1])
    with pytest.raises(ValueError, match="columns"):
        owq.linear_batched(Ls, [xs[0], torch.zeros((2, K), dtype=torch.float16)])
    with pytest.raises(ValueError, match="y has shape"):
        owq.PreparedBatched(Ls, xs, [torch.zeros((2, N), dtype=torch.float16), torch.zeros((2, 31), dtype=torch.float16)])
    _host_only(owq.linear_batched, Ls, xs)


def test_backward_batched_checks_shapes_and_common_m():
    a, b = _layer(), _layer(N=32)
    dy_a, dy_b = torch.zeros((3, N), dtype=torch.float16), torch.zeros((3, 32), dtype=torch.float16)
    x = torch.zeros((3, K), dtype=torch.float16)
    with pytest.raises(ValueError, match="as many"):
        owq.linear_backward_batched([a, b], [x, x], [dy_a])
    with pytest.raises(ValueError, match=r"\[1\] dy has shape"):
        owq.linear_backward_batched([a, b], [x, x], [dy_a, dy_a])
    with pytest.raises(ValueError, match="tokens"):
        owq.linear_backward_batched([a, b], [x, x], [dy_a, torch.zeros((2, 32), dtype=torch.float16)])
    with pytest.raises(ValueError, match="x is needed"):
        owq.linear_backward_batched([a, b], [x, None], [dy_a, dy_b])
    with pytest.raises(ValueError, match="columns|shape"):
        owq.linear_backward_batched([a, b], [x, torch.zeros((3, K - 32), dtype=torch.float16)], [dy_a, dy_b])
    with pytest.raises(TypeError, match="float16"):
        owq.linear_backward_batched([a, b], [x, x], [dy_a, dy_b.float()])
    _host_only(owq.linear_backward_batched, [a, b], [x, x], [dy_a, dy_b])
    _host_only(owq.linear_backward_batched, [a, b], None, [dy_a, dy_b], want_dw=False)


def test_select_batched_checks_shapes():
    a, b = torch.zeros(K, dtype=torch.float64), torch.zeros(2 * K, dtype=torch.float64)
    with pytest.raises(ValueError, match="one k .*per score"):
        owq.select_weak_batched([a, b], [3])
    with pytest.raises(ValueError, match="outside"):
        owq.select_weak_batched([a, b], [3, 2 * K + 1])
    with pytest.raises(TypeError, match="float64"):
        owq.select_weak_batched([a, b.float()], [3, 4])
    with pytest.raises(ValueError, match="1-D"):
        owq.select_weak_batched([a, b.reshape(2, K)], [3, 4])
    _host_only(owq.select_weak_batched, [a, b], [3, 4])


def _grouped_layer(N=N, K=K, k=k, G=64):
    lay = _layer(N, K, k)
    lay["scales"] = torch.zeros((N, K // G), dtype=torch.float16)
    lay["zeros"] = torch.zeros((N, K // G), dtype=torch.uint8)
    lay["group"] = G
    return lay


def test_grouped_checks_shapes():
    W = torch.zeros((N, K), dtype=torch.float16)
    idx = torch.arange(k, dtype=torch.int32)
    for G in (48, 256, 4096):
        with pytest.raises(ValueError, match="G ="):
            owq.pack_grouped(W, idx, G)
    bad_out = {"qcodes": torch.zeros((N, K // 32, 3), dtype=torch.int32),
               "scales": torch.zeros(N, dtype=torch.float16),  # per-row shape, not [N][K/G]
               "zeros": torch.zeros((N, K // 64), dtype=torch.uint8),
               "w_weak": torch.zeros((N, k), dtype=torch.float16)}
    with pytest.raises(ValueError, match="scales"):
        owq.pack_grouped(W, idx, 64, out=bad_out)
    _host_only(owq.pack_grouped, W, idx, 64)
    lay = _grouped_layer()
    with pytest.raises(ValueError, match="columns"):
        owq.linear_grouped(lay, torch.zeros((1, K - 32), dtype=torch.float16))
    with pytest.raises(ValueError, match="scales"):
        owq.linear_grouped(dict(lay, group=32), torch.zeros((1, K), dtype=torch.float16))
    with pytest.raises(ValueError, match="y has shape"):
        owq.linear_grouped(lay, torch.zeros((2, K), dtype=torch.float16), torch.zeros((1, N), dtype=torch.float16))
    _host_only(owq.linear_grouped, lay, torch.zeros((3, K), dtype=torch.float16))
