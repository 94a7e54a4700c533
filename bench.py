"""Benchmark of the OWQ hot path on one MI355X.

One step = one pass of every hot-path stage over one LLaMA-7B decoder layer
(q/k/v/o 4096x4096, gate/up 11008x4096, down 4096x11008; k = 32 / 32 / 86 weak
columns, ~3.1 bits per weight), on seeded synthetic inputs:
  1. calibration: owq_calibrate_score on T = 2048 tokens, owq_select_weak and
     owq_pack, for each of the 7 linears;
  2. decode: owq_linear_batched over the 7 linears at M = 1 (one launch);
  3. prefill: owq_linear at M = 2048 for each of the 7 linears.
Decode reads one of R = 8 packed copies of the layer (8 x 79 MB > 2 x the 256 MB
Infinity Cache), written by the calibration stage R/2 steps earlier, so its
bytes come from HBM. Inputs are resident in HBM before timing starts.

Reported value: effective GB/s of the decode stage (packed codes + fp16 scales +
uint8 zeros + fp16 weak columns + fp16 x, per linear, summed over the layer) per
second of decode-launch time, measured with HIP events around each decode
launch on the launch stream. Other stages are reported alongside.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "OWQ 3.1-bit linear: effective GB/s and % HBM peak at M=1 (7B shapes); TFLOP/s at M=2048"
HBM_PEAK_GBS = 8000.0
MFMA_FP16_PEAK_TFLOPS = 2500.0
ROTATE = 8
PREFILL_M = 2048


def eff_bytes(N, K, k, M):
    """Algorithmic bytes of one linear: codes + scales + zeros + weak block + x."""
    return 3 * N * K // 8 + 2 * N + N + 2 * N * k + 2 * M * K


def cpu_baseline(cfg, min_seconds=10.0):
    """The CPU oracle's mixed-precision linear timed on the host (single thread),
    over the full 7-linear layer at M = 1, repeated until >= min_seconds."""
    import numpy as np

    import oracle
    from mixed_precision_weight_amd import synth
    layers = []
    for li, spec in enumerate(cfg.layers):
        seed = cfg.seed(li)
        W = synth.weights(spec, seed)
        idx = np.sort(np.random.default_rng(li).choice(spec.K, spec.k, replace=False)).astype(np.int32)
        p = oracle.pack(W, idx)
        x = synth.activations(spec, seed, 1)
        layers.append((spec, p, x))
    total_bytes = 0
    reps = 0
    t0 = time.perf_counter()
    while True:
        for spec, p, x in layers:
            oracle.linear_pairs(p, x, np.zeros(spec.N, np.int64), np.arange(spec.N, dtype=np.int64))
            total_bytes += eff_bytes(spec.N, spec.K, spec.k, 1)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    return {"value": total_bytes / el / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"full 7-linear layer decode at M=1 (202.4M weights), {reps} repetition(s), "
                      f"{el:.1f} s, single-threaded C oracle with fp64 accumulation"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU; --gpus {args.gpus} is not supported "
              "(the hot path runs on one GPU's share, see the design notes for sharding)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from mixed_precision_weight_amd import owq, synth

    dev = torch.device("cuda:0")
    cfg = synth.CONFIGS[1]
    specs = cfg.layers
    print(f"bench: {cfg.name}: generating inputs", file=sys.stderr, flush=True)
    W, X, x1, xp = [], [], [], []
    for li, spec in enumerate(specs):
        seed = cfg.seed(li)
        W.append(torch.from_numpy(synth.weights(spec, seed)).to(dev))
        X.append(torch.from_numpy(synth.calibration(spec, seed, cfg.T)).to(dev))
        x1.append(torch.from_numpy(synth.activations(spec, seed, 1)).to(dev))
        xp.append(torch.from_numpy(synth.activations(spec, seed + 500, PREFILL_M)).to(dev))

    ws = torch.empty(max(owq.calibrate_workspace_bytes(s.N, s.K, cfg.T) for s in specs), dtype=torch.uint8,
                     device=dev)
    lam = [torch.empty(s.K, dtype=torch.float64, device=dev) for s in specs]
    slots = []
    for r in range(ROTATE):
        slot = []
        for s in specs:
            slot.append({"qcodes": torch.empty((s.N, s.K // 32, 3), dtype=torch.int32, device=dev),
                         "scales": torch.empty(s.N, dtype=torch.float16, device=dev),
                         "zeros": torch.empty(s.N, dtype=torch.uint8, device=dev),
                         "w_weak": torch.empty((s.N, s.k), dtype=torch.float16, device=dev)})
        slots.append(slot)
    y1 = [torch.empty((1, s.N), dtype=torch.float16, device=dev) for s in specs]
    yp = [torch.empty((PREFILL_M, s.N), dtype=torch.float16, device=dev) for s in specs]

    def calibrate_pack(slot):
        for li, s in enumerate(specs):
            _, score = owq.calibrate(W[li], X[li], workspace=ws)
            idx = owq.select_weak(score, s.k)
            owq.pack(W[li], idx, out=slot[li])

    # fill every rotation slot before timing
    for r in range(ROTATE):
        calibrate_pack(slots[r])
    torch.cuda.synchronize()

    decode_bytes = sum(eff_bytes(s.N, s.K, s.k, 1) for s in specs)
    prefill_flops = sum(2 * PREFILL_M * s.N * s.K for s in specs)
    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def step(i, ev):
        cal_slot = slots[i % ROTATE]
        dec_slot = slots[(i + ROTATE // 2) % ROTATE]
        ev[0].record()
        calibrate_pack(cal_slot)
        ev[1].record()
        owq.linear_batched(dec_slot, x1, y1)
        ev[2].record()
        for li in range(len(specs)):
            owq.linear(cal_slot[li], xp[li], yp[li])
        ev[3].record()

    print(f"bench: warmup {args.warmup}", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i, [E() for _ in range(4)])
    torch.cuda.synchronize()

    print(f"bench: timing {args.steps} steps", file=sys.stderr, flush=True)
    evs = [[E() for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    cal_ms = [e[0].elapsed_time(e[1]) for e in evs]
    dec_ms = [e[1].elapsed_time(e[2]) for e in evs]
    pre_ms = [e[2].elapsed_time(e[3]) for e in evs]
    dec_avg_s = float(np.mean(dec_ms)) / 1e3
    value = decode_bytes / dec_avg_s / 1e9
    pre_tflops = prefill_flops / (float(np.mean(pre_ms)) / 1e3) / 1e12

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": "llama7b_layer_decode (7 linears: 4x 4096x4096 k=32, 2x 11008x4096 k=32, "
                               "4096x11008 k=86)",
                   "decode_M": 1, "calib_T": cfg.T, "prefill_M": PREFILL_M, "bits": 3,
                   "decode_effective_bytes": decode_bytes, "rotation_copies": ROTATE},
        "roofline": {"kernel": "k_gemv (decode, 7-linear batched launch)", "bound": "hbm",
                     "achieved": round(value, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(value / HBM_PEAK_GBS, 4), "traffic": None},
        "stages": {
            "decode_us_per_layer": round(dec_avg_s * 1e6, 2),
            "decode_pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 1),
            "calibrate_select_pack_ms_per_layer": round(float(np.mean(cal_ms)), 3),
            "prefill_ms_per_layer": round(float(np.mean(pre_ms)), 3),
            "prefill_tflops": round(pre_tflops, 2),
            "prefill_pct_mfma_peak": round(100 * pre_tflops / MFMA_FP16_PEAK_TFLOPS, 2),
        },
    }
    if not args.no_cpu_baseline:
        print("bench: CPU oracle baseline", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
