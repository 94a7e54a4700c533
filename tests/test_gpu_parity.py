"""GPU parity of the whole hot path against the CPU oracle, through the C ABI.

Bars: lambda and score within 1e-12 relative (fp64 sums in another order);
weak set equal up to score ties within 1e-6 relative; pack (codes, scales,
zeros, weak block) bit-exact; y within 2e-3 * sum_j |Wdeq_ij x_j| + 1e-5 per
output. Every output of every call is checked, at every size (the oracle's
linear spreads the rows over the host's cores).
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
    K = W.shape[1]
    # a single nonzero dense weight each, at columns where x is made small
    # (_quiet_columns): the output bound is then tiny, and a decode that folded
    # the zero point into a sum over the row (z sum_j x_j) would cancel large terms
    if n > 5:
        W[5] = 0
        W[5, K // 3] = np.float16(0.03)    # zero point 0
    if n > 6:
        W[6] = 0
        W[6, (2 * K) // 3] = np.float16(-0.03)  # zero point 7: every other code is 7
    return W


def _quiet_columns(x: np.ndarray) -> np.ndarray:
    """Small activations at the columns of the planted single-weight rows."""
    K = x.shape[1]
    x = x.copy()
    x[:, K // 3] = np.float16(0.001)
    x[:, (2 * K) // 3] = np.float16(-0.0005)
    return x


def _run(owq, W, X, k, xs, what):
    """Calibrate, select, pack and linear on the GPU; compare with the oracle
    on every output."""
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
        print(f"{what}: linear M={M}", flush=True)
        y = host(owq.linear(packed, dev(x)))
        yr, b = oracle.linear_rows(o_pack, x)
        worst = max(worst, check_linear(y, yr, b, f"{what} M={M}"))
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
    x = _quiet_columns(synth.activations(spec, N + K + 1, max(Ms)))
    _run(owq, W, X, k, [x[:m] for m in Ms], f"edge N={N} K={K} k={k}")


def test_calibrate_batched_matches_single(owq):
    """owq_calibrate_score_batched overlaps the three passes of consecutive
    linears in shared launches: each linear's lambda and score equal its own
    owq_calibrate_score call bit for bit (and the oracle, to the calibration
    bar), for one, two and seven linears of mixed sizes, with a workspace full
    of garbage."""
    import torch
    import oracle
    shapes = [(1, 32, 1), (37, 4128, 24), (300, 96, 77), (5, 11008, 9), (64, 640, 300), (130, 8192, 16),
              (513, 2048, 48), (3, 65536, 40), (40, 24576, 33)]  # K > 32768: the two-pass form
    rng = np.random.default_rng(11)
    Ws = [_tiny_rows(synth.random_layer(rng, N, K, 0.02)) for N, K, _ in shapes]
    Xs = [synth.calibration(synth.LayerSpec("cb", N, K, 1, 0.02, max(1, K // 200), 20.0), N + K, T)
          for N, K, T in shapes]
    Wd, Xd = [dev(W) for W in Ws], [dev(X) for X in Xs]
    single = [owq.calibrate(W, X) for W, X in zip(Wd, Xd)]
    for n in (1, 2, 7, 9):
        print(f"calibrate_batched: {n} linears", flush=True)
        nbytes = owq.calibrate_batched_workspace_bytes(shapes[:n])
        ws = torch.full((nbytes,), 0xAB, dtype=torch.uint8, device="cuda:0")
        got = owq.calibrate_batched(Wd[:n], Xd[:n], workspace=ws)
        prepared = owq.PreparedCalibrate(Wd[:n], Xd[:n])
        again = [tuple(t.clone() for t in pair) for pair in prepared()]
        prepared()  # a second call on the same buffers
        torch.cuda.synchronize()
        for i in range(n):
            for a, b, c, d, what in zip(got[i], single[i], again[i], prepared.results[i], ("lambda", "score")):
                assert host(a).tobytes() == host(b).tobytes(), (n, i, shapes[i], what)
                assert host(c).tobytes() == host(b).tobytes() == host(d).tobytes(), (n, i, shapes[i], what)
    for i in (0, 1, 2, 6, 7):
        o_lam, o_score = oracle.calibrate_score(Ws[i], Xs[i])
        np.testing.assert_allclose(host(single[i][0]), o_lam, rtol=1e-12, atol=0, err_msg=str(shapes[i]))
        np.testing.assert_allclose(host(single[i][1]), o_score, rtol=1e-12, atol=1e-300, err_msg=str(shapes[i]))


def test_pack_batched_matches_single(owq):
    """owq_pack_batched puts the linears of one kernel form in one launch: every
    packed array equals its own owq_pack call bit for bit (and the oracle's),
    over all the kernel forms (a wave per row with 1-3 groups per lane, a block
    per row with 1-8 groups per thread), mixed in one batch, k = 0 included."""
    import torch
    import oracle
    shapes = [(1, 32, 0), (37, 4096, 5), (300, 4128, 17), (4, 6144, 64), (130, 8192, 63), (9, 11008, 86),
              (5, 32768, 3), (3, 65536, 5), (4100, 4096, 32), (64, 640, 0)]
    rng = np.random.default_rng(23)
    Ws, idxs = [], []
    for N, K, k in shapes:
        Ws.append(_tiny_rows(synth.random_layer(rng, N, K, 0.02)))
        idxs.append(np.sort(rng.choice(K, k, replace=False)).astype(np.int32))
    Wd = [dev(W) for W in Ws]
    Id = [dev(ix) for ix in idxs]
    single = [owq.pack(W, ix) for W, ix in zip(Wd, Id)]
    for sel in (list(range(len(shapes))), [8, 1, 8], [3]):
        print(f"pack_batched: {[shapes[i] for i in sel]}", flush=True)
        got = owq.pack_batched([Wd[i] for i in sel], [Id[i] for i in sel])
        torch.cuda.synchronize()
        for i, g in zip(sel, got):
            for name in ("qcodes", "scales", "zeros", "w_weak"):
                assert host(g[name]).tobytes() == host(single[i][name]).tobytes(), (shapes[i], name)
    for i in (1, 2, 5):
        check_pack(single[i], oracle.pack(Ws[i], idxs[i]))


def test_select_batched_matches_single(owq):
    """owq_select_weak_batched over selections of every block shape (and k = 0,
    k = K, K above 16384) gives exactly the single calls' and the oracle's
    indices."""
    import torch

    import oracle
    rng = np.random.default_rng(77)
    cases = [(100, 37), (4096, 32), (4096, 0), (4096, 4096), (5000, 7), (11008, 86), (11264, 300), (16000, 129),
             (20000, 500), (4096, 32), (11008, 86), (1, 1)]
    scores = []
    for K, _ in cases:
        sc = rng.random(K) * np.exp(rng.normal(0, 5, K))
        sc[rng.integers(0, K, K // 10 + 1)] = 0.0
        scores.append(sc)
    got = owq.select_weak_batched([dev(sc) for sc in scores], [k for _, k in cases])
    single = [owq.select_weak(dev(sc), k) for sc, (_, k) in zip(scores, cases)]
    torch.cuda.synchronize()
    for sc, (K, k), g, s1 in zip(scores, cases, got, single):
        ref = oracle.select_weak(sc, k)
        assert np.array_equal(host(g), ref), (K, k)
        assert np.array_equal(host(s1), ref), (K, k)


@pytest.mark.parametrize("K,k", [(1, 1), (5, 2), (100, 37), (4096, 32), (4097, 33), (11008, 86), (11264, 3000),
                                 (11265, 1), (16384, 129), (16385, 16385), (28672, 221), (65536, 65536),
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


def test_prepared_calls_under_graph_capture(owq):
    """PreparedBatched and PreparedCalibrate built with stream=None enqueue on
    the stream current at each call, so a HIP graph captures them. The graph
    is replayed three times, with eager work (clearing the outputs and a
    change of inputs) between replays, and every replay equals the eager
    result of its inputs."""
    import torch
    rng = np.random.default_rng(5)
    shapes = [(96, 256, 3), (40, 512, 0), (130, 1024, 9)]
    layers, xs, Ws, Xs = [], [], [], []
    for N, K, k in shapes:
        W = synth.random_layer(rng, N, K)
        idx = np.sort(rng.choice(K, k, replace=False)).astype(np.int32)
        layers.append(owq.pack(dev(W), dev(idx)))
        xs.append(dev((rng.standard_normal((1, K))).astype(np.float16)))
        Ws.append(dev(W))
        Xs.append(dev((rng.standard_normal((64, K))).astype(np.float16)))
    ys = [torch.zeros((1, N), dtype=torch.float16, device="cuda:0") for N, _, _ in shapes]
    dec = owq.PreparedBatched(layers, xs, ys)
    cal = owq.PreparedCalibrate(Ws, Xs)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capturing stream
        dec()
        cal()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dec()
        cal()
    for rep in range(3):
        for y in ys:
            y.zero_()
        for x in xs:  # new inputs each replay (same addresses)
            x.copy_(dev((rng.standard_normal(tuple(x.shape))).astype(np.float16)))
        torch.cuda.synchronize()
        want = owq.linear_batched(layers, xs)
        want_cal = owq.calibrate_batched(Ws, Xs)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(ys, want):
            assert host(a).tobytes() == host(b).tobytes(), f"replay {rep}"
        for (la, sa), (lb, sb) in zip(cal.results, want_cal):
            assert host(la).tobytes() == host(lb).tobytes(), f"replay {rep}"
            assert host(sa).tobytes() == host(sb).tobytes(), f"replay {rep}"
    del g


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
    x = _quiet_columns(synth.activations(spec, N + K + 2, max(Ms)))
    _run(owq, W, X, k, [x[:m] for m in Ms], f"vector N={N} K={K} k={k}")


@pytest.mark.parametrize("products", ["dot2", "mfma"])
@pytest.mark.parametrize("N,K,k", [(5, 96, 1), (64, 640, 7), (37, 11008, 86), (130, 8192, 63), (64, 640, 130)])
def test_vector_decode_product_forms(owq, monkeypatch, products, N, K, k):
    """The vector-ALU decode's products by v_dot2 (the default for one token) and
    on the matrix cores with the diagonal read-out (the default for two) meet the
    same bar for one and two tokens: ragged chunk tails (K = 96, 640, 11008),
    more than 128 weak columns, rows whose weights sit far below their step."""
    monkeypatch.setenv("OWQ_DECODE", "vector")
    monkeypatch.setenv("OWQ_GEMV_PRODUCTS", products)
    rng = np.random.default_rng(N * 13 + K + k)
    W = _tiny_rows(synth.random_layer(rng, N, K, 0.02))
    spec = synth.LayerSpec("edge", N, K, k, 0.02, max(1, K // 200), 20.0)
    X = synth.calibration(spec, N + K, 24)
    x = _quiet_columns(synth.activations(spec, N + K + 5, 2))
    _run(owq, W, X, k, [x[:1], x[:2]], f"products={products} N={N} K={K} k={k}")
