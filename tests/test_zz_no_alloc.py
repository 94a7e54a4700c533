"""The allocation-free calibration entry point (owq_calibrate_score_noalloc,
the library's own workspace) gives what owq_calibrate_score gives with a caller
workspace, bit for bit, and meets the oracle's bar; two calls in a row, the
second on a smaller input, so that the second runs on the first's leftovers."""
import numpy as np
import pytest

from mixed_precision_weight_amd import synth
from parity_util import dev, host

pytestmark = pytest.mark.gpu


def test_noalloc_matches_workspace_entry_point():
    import torch

    import oracle
    from mixed_precision_weight_amd import owq
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    owq.lib()
    cfg = synth.LLAMA7B_LAYER_DECODE
    cases = [(cfg.layers[4], cfg.seed(4), 2048),     # 11008 x 4096, T = 2048
             (synth.OPT125M_Q_PROJ.layers[0], 0, 128)]  # then 768 x 768, T = 128
    for spec, seed, T in cases:
        print(f"noalloc: N={spec.N} K={spec.K} T={T}", flush=True)
        W = synth.weights(spec, seed)
        X = synth.calibration(spec, seed, T)
        Wd, Xd = dev(W), dev(X)
        need = owq.calibrate_workspace_bytes(spec.N, spec.K, T)
        assert need <= owq.calibrate_noalloc_max_workspace()
        lam_ref, score_ref = owq.calibrate(Wd, Xd)
        lam = torch.full((spec.K,), float("nan"), dtype=torch.float64, device="cuda:0")
        score = torch.full((spec.K,), float("nan"), dtype=torch.float64, device="cuda:0")
        got = owq.calibrate_noalloc(Wd, Xd, lam, score)
        torch.cuda.synchronize()
        assert got[0].data_ptr() == lam.data_ptr() and got[1].data_ptr() == score.data_ptr()
        assert host(lam).tobytes() == host(lam_ref).tobytes()
        assert host(score).tobytes() == host(score_ref).tobytes()
        o_lam, o_score = oracle.calibrate_score(W, X)
        np.testing.assert_allclose(host(lam), o_lam, rtol=1e-12, atol=0)
        np.testing.assert_allclose(host(score), o_score, rtol=1e-12, atol=1e-300)
