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


@pytest.mark.parametrize("M", [1, 6])
def test_batched_equals_per_layer(owq, M):
    """owq_linear_backward_batched over the 7 LLaMA-7B linears gives bit for bit
    what one owq_linear_backward per layer gives (the same kernels, one launch);
    q_proj and down_proj are also checked against the oracle; then dx only and
    dw only."""
    import torch

    import oracle
    cfg = synth.LLAMA7B_LAYER_DECODE
    packs, xs, dys, refs = [], [], [], []
    for li, spec in enumerate(cfg.layers):
        rng = np.random.default_rng(100 + li + M)
        W = synth.weights(spec, cfg.seed(li))
        idx = np.sort(rng.choice(spec.K, spec.k, replace=False)).astype(np.int32)
        x = rng.standard_normal((M, spec.K)).astype(np.float16)
        dy = rng.standard_normal((M, spec.N)).astype(np.float16)
        packs.append(owq.pack(dev(W), dev(idx)))
        xs.append(dev(x))
        dys.append(dev(dy))
        refs.append((W, idx, x, dy) if li in (0, 6) else None)
    print(f"batched backward: 7 linears, M={M}", flush=True)
    dxs, dws = owq.linear_backward_batched(packs, xs, dys)
    one = [owq.linear_backward(p, x, dy) for p, x, dy in zip(packs, xs, dys)]
    dxo, dwo = owq.linear_backward_batched(packs, None, dys, want_dw=False)
    _, dwonly = owq.linear_backward_batched(packs, xs, dys, want_dx=False)
    torch.cuda.synchronize()
    for li in range(7):
        assert host(dxs[li]).tobytes() == host(one[li][0]).tobytes(), li
        assert host(dws[li]).tobytes() == host(one[li][1]).tobytes(), li
        assert host(dxo[li]).tobytes() == host(dxs[li]).tobytes(), li
        assert host(dwonly[li]).tobytes() == host(dws[li]).tobytes(), li
        if refs[li] is not None:
            W, idx, x, dy = refs[li]
            rdx, rdxb, rdw, rdwb = oracle.linear_backward(oracle.pack(W, idx), x, dy)
            check_linear(host(dxs[li]), rdx, rdxb, f"batched dx [{li}] M={M}")
            check_linear(host(dws[li]), rdw, rdwb, f"batched dw [{li}] M={M}")


@pytest.mark.parametrize("M", [9, 16, 33])
def test_vector_form_above_four_tokens(owq, M, monkeypatch):
    """Above 4 tokens dx runs on the matrix cores; OWQ_BACKWARD=vector keeps the
    vector form (4 tokens per pass). Both meet the bound on every element."""
    import torch

    import oracle
    rng = np.random.default_rng(M)
    N, K, k = 300, 4128, 17
    W = synth.random_layer(rng, N, K, 0.02)
    idx = np.sort(rng.choice(K, k, replace=False)).astype(np.int32)
    x = rng.standard_normal((M, K)).astype(np.float16)
    dy = rng.standard_normal((M, N)).astype(np.float16)
    p = owq.pack(dev(W), dev(idx))
    print(f"vector/matrix forms: N={N} K={K} k={k} M={M}", flush=True)
    dx_m, dw_m = owq.linear_backward(p, dev(x), dev(dy))
    monkeypatch.setenv("OWQ_BACKWARD", "vector")
    dx_v, dw_v = owq.linear_backward(p, dev(x), dev(dy))
    torch.cuda.synchronize()
    rdx, rdxb, rdw, rdwb = oracle.linear_backward(oracle.pack(W, idx), x, dy)
    check_linear(host(dx_m), rdx, rdxb, f"matrix-core dx M={M}")
    check_linear(host(dx_v), rdx, rdxb, f"vector dx M={M}")
    assert host(dw_m).tobytes() == host(dw_v).tobytes()
    check_linear(host(dw_m), rdw, rdwb, f"dw M={M}")


@pytest.mark.parametrize("M", [16, 20])
def test_matrix_core_step_ranges(owq, M):
    """The matrix-core form splits s (q - z) into two fp16 values; a block whose
    512-row slice holds a row with s > 9352 (where 7 s overflows fp16) keeps
    fp32 products. The first slice holds two such rows (weights near +-40000,
    and -30000 .. 40000) and a row of fp16 subnormal weights; the second holds
    a row whose step (9344) is just below the limit and a row of subnormal
    steps, and runs the fp16 form: every element stays within the bound."""
    rng = np.random.default_rng(77 + M)
    N, K = 600, 4096
    W = synth.random_layer(rng, N, K, 0.02)
    W[5, :] = rng.uniform(-40000, 40000, K).astype(np.float16)
    W[300, ::3] = np.float16(40000)
    W[300, 1::3] = np.float16(-30000)
    W[7, :] = (rng.uniform(-1, 1, K) * 1e-5).astype(np.float16)
    W[540, ::2] = np.float16(32700)  # step 9344: the largest range below the limit
    W[540, 1::2] = np.float16(-32700)
    W[520, :] = (rng.uniform(-1, 1, K) * 1e-6).astype(np.float16)
    idx = np.sort(rng.choice(K, 40, replace=False)).astype(np.int32)
    _run_scaled(owq, W, idx, M, "step ranges", dy_scale=1e-2)


def _run_scaled(owq, W, idx, M, what, dy_scale):
    """_run with dy scaled down, so that rows of large weights keep dx finite."""
    import torch

    import oracle
    N, K = W.shape
    rng = np.random.default_rng(5 + N + K + M)
    x = rng.standard_normal((M, K)).astype(np.float16)
    dy = (rng.standard_normal((M, N)) * dy_scale).astype(np.float16)
    print(f"{what}: N={N} K={K} k={len(idx)} M={M}", flush=True)
    p_ref = oracle.pack(W, idx)
    p = owq.pack(dev(W), dev(np.asarray(idx, np.int32)))
    dx, dw = owq.linear_backward(p, dev(x), dev(dy))
    torch.cuda.synchronize()
    rdx, rdxb, rdw, rdwb = oracle.linear_backward(p_ref, x, dy)
    assert np.isfinite(rdx).all()
    check_linear(host(dx), rdx, rdxb, f"{what} dx M={M}")
    check_linear(host(dw), rdw, rdwb, f"{what} dw M={M}")
