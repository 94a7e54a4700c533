"""Seeded synthetic workloads for the OWQ hot path.

This module only draws random inputs: it holds none of the method's arithmetic,
and it is the one piece of Python that both the GPU side and the CPU oracle's
tests consume.

The pages evaluate on real OPT/LLaMA weights calibrated on C4 text; neither the
weights nor the data are available here, so the inputs stand in for them with
the same shapes and the structure that drives the method: Gaussian weights and
activations in which a few input channels carry large outliers, the
phenomenon the method is built around (weights fed by outlier activation
channels are the sensitive ones).

Recipe (per linear layer, seed = 1000 * config_id + layer_index):
  * four independent PCG64 streams are spawned from the seed (weights, outlier
    channel choice, calibration activations, layer-input activations);
  * W = sigma * N(0, 1), drawn in float32, rounded to fp16 (nearest-even);
  * outlier channels: n_out distinct input channels, uniform without
    replacement, sorted;
  * X (calibration, [T][K]) and x (layer input, [M][K]) are N(0, 1) in float32
    with the outlier channels multiplied by ``factor``, then rounded to fp16.
    Smaller M use the first M rows of the M_max draw.
"""
from __future__ import annotations

import dataclasses
import hashlib

import numpy as np


@dataclasses.dataclass(frozen=True)
class LayerSpec:
    name: str
    N: int          # output rows
    K: int          # input columns
    k: int          # weak columns kept in fp16
    sigma: float    # weight standard deviation
    n_out: int      # outlier input channels
    factor: float   # outlier multiplier


@dataclasses.dataclass(frozen=True)
class Config:
    seed_base: int  # layer l of this workload draws from seed seed_base + l
    name: str
    layers: tuple
    T: int          # calibration tokens
    Ms: tuple       # decode / prefill batch sizes exercised

    def seed(self, layer_index: int) -> int:
        return self.seed_base + layer_index


def _n_out(K: int) -> int:
    # 0.5 % of the input channels, rounded half-to-even
    return int(round(0.005 * K))


def _llama7b_layers(sigma=0.02, factor=20.0):
    d, D = 4096, 11008
    sq = dict(sigma=sigma, factor=factor)
    return (
        LayerSpec("q_proj", d, d, 32, n_out=_n_out(d), **sq),
        LayerSpec("k_proj", d, d, 32, n_out=_n_out(d), **sq),
        LayerSpec("v_proj", d, d, 32, n_out=_n_out(d), **sq),
        LayerSpec("o_proj", d, d, 32, n_out=_n_out(d), **sq),
        LayerSpec("gate_proj", D, d, 32, n_out=_n_out(d), **sq),
        LayerSpec("up_proj", D, d, 32, n_out=_n_out(d), **sq),
        LayerSpec("down_proj", d, D, 86, n_out=_n_out(D), **sq),
    )


def _k_large(K: int) -> int:
    return int(round(0.0077 * K))


# The OPT-125m q_proj shape: the small case the oracle finishes in seconds.
OPT125M_Q_PROJ = Config(0, "opt125m_q_proj", (LayerSpec("q_proj", 768, 768, 6, 0.02, 6, 20.0),),
                        T=128, Ms=(1,))
# One LLaMA-7B decoder layer (7 linears), decode M = 1.
LLAMA7B_LAYER_DECODE = Config(1000, "llama7b_layer_decode", _llama7b_layers(), T=2048, Ms=(1,))
# Same shapes, decode batch sweep.
LLAMA7B_BATCH_SWEEP = Config(2000, "llama7b_layer_batch_sweep", _llama7b_layers(), T=2048, Ms=(1, 2, 4, 8, 16))
# Large-model shapes.
LARGE_SHAPES = Config(3000, "large_8192_28672", (
    LayerSpec("attn_8192x8192", 8192, 8192, _k_large(8192), 0.01, _n_out(8192), 30.0),
    LayerSpec("up_28672x8192", 28672, 8192, _k_large(8192), 0.01, _n_out(8192), 30.0),
    LayerSpec("down_8192x28672", 8192, 28672, _k_large(28672), 0.01, _n_out(28672), 30.0),
), T=2048, Ms=(1, 8))
# Prefill (M = 2048) and long calibration (T = 8192) at the MLP shapes.
LLAMA7B_MLP_PREFILL_CALIB = Config(4000, "llama7b_mlp_prefill_calib", (
    LayerSpec("gate_proj", 11008, 4096, 32, 0.02, _n_out(4096), 20.0),
    LayerSpec("down_proj", 4096, 11008, 86, 0.02, _n_out(11008), 20.0),
), T=8192, Ms=(2048,))

CONFIGS = {c.name: c for c in (OPT125M_Q_PROJ, LLAMA7B_LAYER_DECODE, LLAMA7B_BATCH_SWEEP, LARGE_SHAPES,
                               LLAMA7B_MLP_PREFILL_CALIB)}


def _streams(seed: int):
    ss = np.random.SeedSequence(seed)
    return [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(4)]


def weights(spec: LayerSpec, seed: int) -> np.ndarray:
    rng = _streams(seed)[0]
    w = rng.standard_normal((spec.N, spec.K), dtype=np.float32)
    w *= np.float32(spec.sigma)
    return w.astype(np.float16)


def outlier_channels(spec: LayerSpec, seed: int) -> np.ndarray:
    rng = _streams(seed)[1]
    return np.sort(rng.choice(spec.K, spec.n_out, replace=False)).astype(np.int64)


def _acts(spec: LayerSpec, seed: int, rows: int, stream: int) -> np.ndarray:
    rng = _streams(seed)[stream]
    a = rng.standard_normal((rows, spec.K), dtype=np.float32)
    a[:, outlier_channels(spec, seed)] *= np.float32(spec.factor)
    return a.astype(np.float16)


def calibration(spec: LayerSpec, seed: int, T: int) -> np.ndarray:
    """X [T][K] fp16 calibration activations."""
    return _acts(spec, seed, T, 2)


def activations(spec: LayerSpec, seed: int, M: int) -> np.ndarray:
    """x [M][K] fp16 layer input."""
    return _acts(spec, seed, M, 3)


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).view(np.uint8).tobytes()).hexdigest()


def random_layer(rng: np.random.Generator, N: int, K: int, sigma: float = 0.02):
    """Small ad-hoc weight matrix for edge-case tests."""
    return (sigma * rng.standard_normal((N, K), dtype=np.float32)).astype(np.float16)
