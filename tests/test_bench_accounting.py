"""The algorithmic bytes and flops bench.py divides by (R11: codes + steps +
zero points + weak block + x per linear), checked on the CPU against the
figures worked out by hand for each workload, and the one-GPU guard."""
import subprocess
import sys

import pytest

import bench
from mixed_precision_weight_amd import synth


def _layer_bytes(cfg, M):
    return sum(bench.eff_bytes(s.N, s.K, s.k, M) for s in cfg.layers)


def test_llama7b_layer_decode_bytes():
    # 4 x 4096x4096 (k = 32), 2 x 11008x4096 (k = 32), 4096x11008 (k = 86) at M = 1
    assert _layer_bytes(synth.LLAMA7B_LAYER_DECODE, 1) == 79_251_456


@pytest.mark.parametrize("M,mb", [(1, 79.25), (2, 79.32), (4, 79.46), (8, 79.75), (16, 80.32)])
def test_batch_sweep_bytes(M, mb):
    assert abs(_layer_bytes(synth.LLAMA7B_BATCH_SWEEP, M) / 1e6 - mb) < 0.005


def test_large_shape_bytes():
    got = [bench.eff_bytes(s.N, s.K, s.k, 1) / 1e6 for s in synth.LARGE_SHAPES.layers]
    assert [round(v, 2) for v in got] == [26.24, 91.80, 91.78]


def test_small_layer_bytes():
    s = synth.OPT125M_Q_PROJ.layers[0]
    # 768*768*3/8 codes + 768*2 steps + 768 zero points + 768*6*2 weak + 768*2 x
    assert bench.eff_bytes(s.N, s.K, s.k, 1) == 221184 + 1536 + 768 + 9216 + 1536


def test_prefill_flops_and_long_calibration_bytes():
    c = synth.LLAMA7B_MLP_PREFILL_CALIB
    assert [2 * 2048 * s.N * s.K for s in c.layers] == [184_683_593_728] * 2
    # X (T x K fp16) and W (N x K fp16) read once, lambda and score written
    assert bench.calib_bytes(11008, 4096, c.T) == 2 * 8192 * 4096 + 2 * 11008 * 4096 + 16 * 4096
    assert abs(bench.calib_bytes(4096, 11008, c.T) / 1e6 - 270.71) < 0.01


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
