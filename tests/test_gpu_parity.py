"""GPU parity of the whole hot path against the CPU oracle, through the C ABI.

Bars: lambda and score within 1e-12 relative (fp64 sums in another order);
weak set equal up to score ties within 1e-6 relative; pack (codes, scales,
zeros, weak block) bit-exact; y within 2e-3 * sum_j |Wdeq_ij x_j| + 1e-5 per
output. Small shapes are checked on every output; full-size workloads on every
output at M = 1 and on seeded samples of (token, row) pairs for larger M.
"""
import numpy as np
import pytest

from mixed_precision_weight_amd import synth
from parity_util import check_linear, check_pack, check_weak_set, dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def owq():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from mixed_precision_weight_amd import owq as o
    o.lib()
    return o


def _tiny_rows(W: np.ndarray):
    """Plant the quantiser's special rows: all-zero, positive-only, negative-only,
    sub-normal-only (step rounds to fp16 zero), and one wide-range row."""
    n = W.shape[0]
    if n > 0:
        W[0] = 0
    if n > 1:
        W[1] = np.abs(W[1])
    if n > 2:
        W[2] = -np.abs(W[2])
    if n > 3:
        W[3] = 0
        W[3, ::7] = np.uint16(0x0001).view(np.float16)
    if n > 4:
        W[4, ::3] *= np.float16(50.0)
    return W


def _run(owq, W, X, k, xs, what, sample=None, rng=None):
    """Calibrate, select, pack and linear on the GPU; compare with the oracle."""
    import torch
    import oracle
    N, K = W.shape
    Wd, Xd = dev(W), dev(X)
    lam, score = owq.calibrate(Wd, Xd)
    o_lam, o_score = oracle.calibrate_score(W, X)
    np.testing.assert_allclose(host(lam), o_lam, rtol=1e-12, atol=0, err_msg=f"{what}: lambda")
    np.testing.assert_allclose(host(score), o_score, rtol=1e-12, atol=1e-300, err_msg=f"{what}: score")
    idx = owq.select_weak(score, k)
    o_idx = oracle.select_weak(o_score, k)
    check_weak_set(host(idx), o_idx, o_score)
    # pack with the oracle's weak set: the format is checked independently of ties
    packed = owq.pack(Wd, dev(o_idx.astype(np.int32)))
    o_pack = oracle.pack(W, o_idx)
    torch.cuda.synchronize()
    check_pack(packed, o_pack)
    worst = 0.0
    for x in xs:
        M = x.shape[0]
        y = host(owq.linear(packed, dev(x)))
        if sample is None or M * N <= sample:
            yr, b = oracle.linear_full(o_pack, x)
            worst = max(worst, check_linear(y, yr, b, f"{what} M={M}"))
        else:
            pm = rng.integers(0, M, sample)
            pi = rng.integers(0, N, sample)
            yr, b = oracle.linear_pairs(o_pack, x, pm, pi)
            worst = max(worst, check_linear(y[pm, pi], yr, b, f"{what} M={M} sampled"))
    return packed, o_pack, worst


def test_small_config_full(owq):
    cfg = synth.OPT125M_Q_PROJ
    spec = cfg.layers[0]
    seed = cfg.seed(0)
    W = synth.weights(spec, seed)
    X = synth.calibration(spec, seed, cfg.T)
    x = synth.activations(spec, seed, 16)
    xs = [x[:m] for m in (1, 2, 3, 4, 5, 16)]
    _run(owq, W, X, spec.k, xs, "opt125m_q_proj")


EDGE = [
    # N, K, k, Ms
    (1, 32, 0, (1,)),
    (1, 32, 32, (1, 2)),
    (5, 96, 1, (1, 3, 4)),
    (7, 64, 64, (1, 4)),
    (37, 11008, 86, (1, 2)),
    (130, 8192, 63, (1, 4, 5)),
    (3, 65536, 5, (1,)),
    (64, 640, 7, (1, 2, 3, 17)),
    (300, 4096, 0, (1,)),
    (17, 28672, 221, (1, 2)),
    # matrix-core path: ragged token and row blocks, odd group counts, all-weak
    (200, 4128, 17, (5, 33, 300)),
    (1, 32, 32, (5, 128)),
    (300, 96, 0, (128, 130)),
    (7, 64, 64, (6, 129)),
    (33, 65536, 20, (8, 129)),
    (513, 2048, 40, (512, 700)),
]


@pytest.mark.parametrize("N,K,k,Ms", EDGE)
def test_edge_shapes(owq, N, K, k, Ms):
    rng = np.random.default_rng(N * 131 + K + k)
    W = _tiny_rows(synth.random_layer(rng, N, K, 0.02))
    spec = synth.LayerSpec("edge", N, K, k, 0.02, max(1, K // 200), 20.0)
    X = synth.calibration(spec, N + K, 24)
    x = synth.activations(spec, N + K + 1, max(Ms))
    _run(owq, W, X, k, [x[:m] for m in Ms], f"edge N={N} K={K} k={k}")


@pytest.mark.parametrize("K,k", [(1, 1), (5, 2), (100, 37), (4096, 32), (28672, 221), (65536, 65536),
                                 (1 << 20, 1000)])
def test_select_exact(owq, K, k):
    import oracle
    rng = np.random.default_rng(K + k)
    score = rng.random(K) * np.exp(rng.normal(0, 5, K))
    score[rng.integers(0, K, K // 10 + 1)] = 0.0
    got = host(owq.select_weak(dev(score), k))
    assert np.array_equal(got, oracle.select_weak(score, k))
    if K == 4096:  # into a caller's buffer: the indices land there
        import torch
        out = torch.full((k + 3,), -1, dtype=torch.int32, device="cuda:0")
        r = owq.select_weak(dev(score), k, out=out)
        assert r.data_ptr() == out.data_ptr()
        assert np.array_equal(host(out)[:k], oracle.select_weak(score, k))
        assert (host(out)[k:] == -1).all()


def test_select_ties(owq):
    import oracle
    rng = np.random.default_rng(3)
    for K, k in ((64, 10), (1000, 500), (5000, 4999), (3000, 1)):
        score = rng.integers(0, 4, K).astype(np.float64)
        got = host(owq.select_weak(dev(score), k))
        assert np.array_equal(got, oracle.select_weak(score, k)), (K, k)
    # all scores equal: the lowest k indices; all negative
    for K, k in ((3000, 7), (11008, 86)):
        for score in (np.full(K, 2.5), -np.exp(rng.normal(0, 2, K))):
            got = host(owq.select_weak(dev(score), k))
            assert np.array_equal(got, oracle.select_weak(score, k)), (K, k)
    # negative, zero of both signs, and huge values
    score = np.array([-1.0, 0.0, -0.0, 3.0, -5.0, 1e300, 0.0, -0.0, 2.0, -1e-300])
    for k in range(len(score) + 1):
        got = host(owq.select_weak(dev(score), k))
        assert np.array_equal(got, oracle.select_weak(score, k)), k


def test_determinism(owq):
    import torch
    cfg = synth.LLAMA7B_LAYER_DECODE
    spec = cfg.layers[6]
    rng = np.random.default_rng(0)
    W = synth.random_layer(rng, 512, spec.K)
    X = synth.calibration(spec, 5, 256)
    x = synth.activations(spec, 5, 4)
    outs = []
    for _ in range(2):
        lam, score = owq.calibrate(dev(W), dev(X))
        idx = owq.select_weak(score, spec.k)
        p = owq.pack(dev(W), idx)
        y = owq.linear(p, dev(x))
        torch.cuda.synchronize()
        outs.append([host(t).tobytes() for t in (lam, score, idx, p["qcodes"], p["scales"], p["zeros"],
                                                 p["w_weak"], y)])
    assert outs[0] == outs[1]


def test_workspace_reuse_and_stream(owq):
    """A caller workspace full of garbage and a non-default stream give the same result."""
    import torch
    rng = np.random.default_rng(1)
    W = synth.random_layer(rng, 100, 1024)
    X = (rng.standard_normal((77, 1024))).astype(np.float16)
    ref = owq.calibrate(dev(W), dev(X))
    nbytes = owq.calibrate_workspace_bytes(100, 1024, 77)
    ws = torch.full((nbytes,), 0xAB, dtype=torch.uint8, device="cuda:0")
    s = torch.cuda.Stream()
    Wd, Xd = dev(W), dev(X)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        got = owq.calibrate(Wd, Xd, workspace=ws, stream=s)
    s.synchronize()
    assert host(got[1]).tobytes() == host(ref[1]).tobytes()


def test_pack_and_score_exact_ties(owq):
    """Rows built from multiples of a quarter of the step put w / s exactly on
    half-integers in many places: codes must round those ties to even, exactly as
    rint of the IEEE quotient does in the oracle (pack bit-exact, scores 1e-12)."""
    import oracle
    rng = np.random.default_rng(77)
    N, K, k = 96, 256, 5
    W = np.zeros((N, K), np.float16)
    for i in range(N):
        step = np.float16(2.0 ** rng.integers(-6, 1))   # exact fp16 step s = (hi - lo) / 7
        zq = int(rng.integers(0, 8))                      # lo = -zq s, hi = (7 - zq) s
        quarters = rng.integers(-4 * zq, 4 * (7 - zq) + 1, K)
        W[i] = (quarters.astype(np.float32) * np.float32(step) / 4).astype(np.float16)
        W[i, 0] = np.float16(-zq * float(step))           # pin the range ends
        W[i, 1] = np.float16((7 - zq) * float(step))
    X = synth.calibration(synth.LayerSpec("ties", N, K, k, 0.02, 2, 20.0), 5, 16)
    Wd = dev(W)
    lam, score = owq.calibrate(Wd, dev(X))
    _, o_score = oracle.calibrate_score(W, X)
    np.testing.assert_allclose(host(score), o_score, rtol=1e-12, atol=1e-300)
    o_idx = oracle.select_weak(o_score, k)
    packed = owq.pack(Wd, dev(o_idx.astype(np.int32)))
    check_pack(packed, oracle.pack(W, o_idx))


@pytest.mark.parametrize("N,K,k,Ms", [(5, 96, 1, (3, 4)), (64, 640, 7, (3,)), (37, 11008, 86, (3, 4)),
                                      (130, 8192, 63, (4,))])
def test_vector_decode_three_and_four_tokens(owq, monkeypatch, N, K, k, Ms):
    """3 and 4 tokens run on the matrix cores by default; OWQ_DECODE=vector keeps
    them on the vector-ALU kernel, which must stay at the same bar."""
    monkeypatch.setenv("OWQ_DECODE", "vector")
    rng = np.random.default_rng(N * 17 + K + k)
    W = _tiny_rows(synth.random_layer(rng, N, K, 0.02))
    spec = synth.LayerSpec("edge", N, K, k, 0.02, max(1, K // 200), 20.0)
    X = synth.calibration(spec, N + K, 24)
    x = synth.activations(spec, N + K + 2, max(Ms))
    _run(owq, W, X, k, [x[:m] for m in Ms], f"vector N={N} K={K} k={k}")
