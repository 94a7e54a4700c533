"""Benchmark of the OWQ hot path on one MI355X.

One step = one pass of every hot-path stage over one LLaMA-7B decoder layer
(q/k/v/o 4096x4096, gate/up 11008x4096, down 4096x11008; k = 32 / 32 / 86 weak
columns, ~3.1 bits per weight), on seeded synthetic inputs:
  1. calibration: owq_calibrate_score_batched on T = 2048 tokens over the 7
     linears, owq_select_weak_batched and owq_pack_batched for the 7;
  2. decode: owq_linear_batched over the 7 linears at M = 1 (one launch per
     layer), for R = 8 distinct packed layers in a row, as a token passes
     through consecutive decoder layers;
  3. prefill: owq_linear at M = 2048 for each of the 7 linears.
The R = 8 packed copies of the layer take 8 x 79 MB, more than twice the 256 MB
Infinity Cache. Decode visits them starting after the copy this step's
calibration wrote and ending with it, so at least 7 x 79 MB stream between two
touches of a copy and its bytes come from HBM. Inputs are resident in HBM
before timing starts.

Reported value: effective GB/s of decode (packed codes + fp16 scales + uint8
zeros + fp16 weak columns + fp16 x, per linear, summed over the layer) over the
average duration of one layer's decode launch, measured with HIP events
recorded on the launch stream around the R back-to-back decode launches of each
timed step. The other stages are timed with events around each launch and
reported under "kernels", each against its own roofline; the calibration is
also timed on its own after the timed steps (median of 10 calls, each after a
read-only pass over 1 GiB, so that no other stage's writes are still draining to
HBM while it reads), which is its reported time ("us_in_step": inside the step).

After the timed steps it also reports, each under its own key: the decode batch
sweep (M = 1, 2, 4, 8, 16), the same M = 1 decode as one launch per linear
replayed from a HIP graph, the M = 1 decode and the prefill products as plain
fp16 products on the unquantised weights (torch, for comparison), a 1 GiB device-copy rate, and
calibration at T = 8192 on the two MLP shapes, and the decode of the large
shapes (8192 and 28672) at M = 1 and 8 (flags --no-sweep, --no-extras,
--no-long-calibration and --no-large skip them, e.g. under a profiler). The
extras also time the storage-favoured form, one GPU's share of the layer at
8-way column-parallel sharding (N / 8 rows of each linear), the
weak-column-tuning backward, the OPTQ pack and the truncation-aware pack.

--copy-reference adds, after the timed steps, three copies of a 512 MiB buffer
(a plain copy kernel of known size) so that hardware-counter runs of this script
can scale FETCH_SIZE / WRITE_SIZE to bytes.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "OWQ 3.1-bit linear: effective GB/s and % HBM peak at M=1 (7B shapes); TFLOP/s at M=2048"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_FP16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix peak
ROTATE = 8
PREFILL_M = 2048
SWEEP_MS = (1, 2, 4, 8, 16)
PMC_SUMMARY = os.path.join(ROOT, "profiles", "k_gemv_llama7b_layer_decode_m1_hbm_traffic.txt")
# vector ALU issue: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz = 39.3e12 lane operations/s (fp32 and fp64 alike)
ALU_PEAK_TOPS = 39.3
SEARCH_GRID = 32 * 8          # (step, zero point) grid points per row
# arithmetic of one grid point and one weight, a fused IEEE operation counted
# once: the quotient w / s, its rounding, the clamp to [-z, 7 - z], the exact
# residual w - s (q - z) (one fused multiply-add), its square, the weight, the sum
SEARCH_OPS_PER_EVAL = 7
GEMV_SOURCES = ("gemv.hip", "owq_decode.h", "owq_device.h")


def eff_bytes(N, K, k, M):
    """Algorithmic bytes of one linear: codes + scales + zeros + weak block + x."""
    return 3 * N * K // 8 + 2 * N + N + 2 * N * k + 2 * M * K


def calib_bytes(N, K, T):
    """Algorithmic bytes of owq_calibrate_score: X and W read once, lambda and score written."""
    return 2 * T * K + 2 * N * K + 16 * K


def pack_bytes(N, K, k):
    """Algorithmic bytes of owq_pack: W and weak_idx read, codes, scales, zeros, weak block written."""
    return 2 * N * K + 4 * k + 3 * N * K // 8 + 3 * N + 2 * N * k


def gemv_source_digest() -> str:
    h = hashlib.sha256()
    for name in GEMV_SOURCES:
        with open(os.path.join(ROOT, "mixed_precision_weight_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per decode launch from the committed counter summary, or None when
    there is none or the decode kernel's sources changed since it was taken."""
    try:
        text = open(PMC_SUMMARY).read()
    except OSError:
        return None
    src = re.search(r"^source_sha256:\s*([0-9a-f]{64})", text, re.M)
    val = re.search(r"^traffic_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    if not src or not val or src.group(1) != gemv_source_digest():
        return None
    return float(val.group(1))


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
    return {"value": round(total_bytes / el / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"full 7-linear layer decode at M=1 (202.4M weights), {reps} repetition(s) in "
                      f"{el:.1f} s, single-threaded C oracle with fp64 accumulation",
            "input_sha256_16": {spec.name: synth.sha256(x)[:16] for spec, _, x in layers}}, layers


def host_description():
    """The host the CPU legs ran on: CPU model, logical CPUs, the process's
    affinity set, and the OpenMP threads the threaded oracle uses."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    aff = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    omp = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or aff
    return {"cpu_model": model, "nproc": os.cpu_count(), "affinity_cpus": aff, "omp_threads": omp}


def cpu_extra_legs(threads, layers):
    """The oracle on the host, beside the GPU: OpenMP over output rows for the
    decode batch sweep's largest batch (the 7 LLaMA-7B linears packed for the
    single-thread leg, M = 16), the 8192x8192 large shape at M = 1 and 8, and a
    prefill sample (the first 64 rows of each MLP linear, all 2048 tokens);
    single-threaded for the long calibration (both MLP shapes, T = 8192, whole).
    Each leg is timed once; the numbers are the oracle as it stands."""
    import numpy as np

    import oracle
    from mixed_precision_weight_amd import synth
    legs = {}
    sweep = synth.LLAMA7B_BATCH_SWEEP
    xs = [synth.activations(spec, sweep.seed(li), 16) for li, (spec, _, _) in enumerate(layers)]
    t0 = time.perf_counter()
    for (spec, p, _), x in zip(layers, xs):
        oracle.linear_rows(p, x, threads=threads)
    el = time.perf_counter() - t0
    nb = sum(eff_bytes(spec.N, spec.K, spec.k, 16) for spec, _, _ in layers)
    legs["decode_m16_threaded"] = {"value": round(nb / el / 1e9, 4), "unit": "GB/s", "cores": threads,
                                   "seconds": round(el, 2),
                                   "sample": "the 7 LLaMA-7B linears at M=16 (batch-sweep inputs), every output"}

    def packed(cfg, li, rows=None):
        spec = cfg.layers[li]
        W = synth.weights(spec, cfg.seed(li))
        if rows is not None:  # the pack is row by row: the first rows alone pack the same
            W = np.ascontiguousarray(W[:rows])
        idx = np.sort(np.random.default_rng(li).choice(spec.K, spec.k, replace=False)).astype(np.int32)
        return spec, oracle.pack(W, idx)

    big = synth.LARGE_SHAPES
    spec, p = packed(big, 0)
    x = synth.activations(spec, big.seed(0), 8)
    for M in (1, 8):
        t0 = time.perf_counter()
        oracle.linear_rows(p, x[:M], threads=threads)
        el = time.perf_counter() - t0
        legs[f"large_8192x8192_m{M}_threaded"] = {
            "value": round(eff_bytes(spec.N, spec.K, spec.k, M) / el / 1e9, 4), "unit": "GB/s", "cores": threads,
            "seconds": round(el, 3), "sample": f"8192x8192 (k=63) at M={M}, every output"}
    cfg = synth.LLAMA7B_MLP_PREFILL_CALIB
    flops, el = 0, 0.0
    for li, spec in enumerate(cfg.layers):
        _, p = packed(cfg, li, rows=64)
        x = synth.activations(spec, cfg.seed(li) + 500, PREFILL_M)
        t0 = time.perf_counter()
        oracle.linear_rows(p, x, threads=threads)
        el += time.perf_counter() - t0
        flops += 2 * PREFILL_M * 64 * spec.K
    legs["prefill_sample_threaded"] = {"value": round(flops / el / 1e9, 3), "unit": "GFLOP/s", "cores": threads,
                                       "seconds": round(el, 2),
                                       "sample": "first 64 rows x 2048 tokens of 11008x4096 and 4096x11008"}
    cal = {}
    for li, spec in enumerate(cfg.layers):
        W = synth.weights(spec, cfg.seed(li))
        X = synth.calibration(spec, cfg.seed(li), cfg.T)
        t0 = time.perf_counter()
        oracle.calibrate_score(W, X)
        el = time.perf_counter() - t0
        cal[f"{spec.name} {spec.N}x{spec.K} T={cfg.T}"] = {
            "us": round(el * 1e6, 0), "value": round(calib_bytes(spec.N, spec.K, cfg.T) / el / 1e9, 4),
            "unit": "GB/s"}
    legs["calibration_single_thread"] = dict(cal, cores=1, sample="the whole long-calibration workload")
    return legs


def hbm_entry(nbytes, seconds, what):
    gbs = nbytes / seconds / 1e9
    return {"what": what, "us": round(seconds * 1e6, 2), "bound": "hbm", "achieved": round(gbs, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
            "algorithmic_bytes": int(nbytes)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-sweep", action="store_true", help="skip the decode batch sweep")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the per-linear decode from a HIP graph and the device-copy rate (their "
                         "dispatches, of other sizes, would mix into a profiler's per-kernel averages)")
    ap.add_argument("--no-large", action="store_true",
                    help="skip the decode timing of the large shapes (8192 and 28672)")
    ap.add_argument("--no-long-calibration", action="store_true",
                    help="skip the long-calibration (T = 8192) timing")
    ap.add_argument("--copy-reference", action="store_true",
                    help="end with three 512 MiB device copies (counter scaling)")
    ap.add_argument("--no-search", action="store_true",
                    help="skip the timing of the truncation-aware pack (owq_pack_search)")
    ap.add_argument("--no-cpu-extra", action="store_true",
                    help="skip the threaded and calibration legs of the CPU oracle")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the hot path runs on one GPU's share of a layer; multi-GPU sharding is design only)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from mixed_precision_weight_amd import owq, synth

    dev = torch.device("cuda:0")
    owq.lib()  # fails loudly if the HIP library is missing
    cfg = synth.LLAMA7B_LAYER_DECODE
    specs = cfg.layers
    L = len(specs)
    print(f"bench: {cfg.name}: generating inputs", file=sys.stderr, flush=True)
    W, X, x1, xp = [], [], [], []
    for li, spec in enumerate(specs):
        seed = cfg.seed(li)
        W.append(torch.from_numpy(synth.weights(spec, seed)).to(dev))
        X.append(torch.from_numpy(synth.calibration(spec, seed, cfg.T)).to(dev))
        x1.append(torch.from_numpy(synth.activations(spec, seed, max(SWEEP_MS))).to(dev))
        xp.append(torch.from_numpy(synth.activations(spec, seed + 500, PREFILL_M)).to(dev))
    xd = [x[:1] for x in x1]

    ws = torch.empty(max(owq.calibrate_workspace_bytes(s.N, s.K, cfg.T) for s in specs), dtype=torch.uint8,
                     device=dev)
    slots = []
    for r in range(ROTATE):
        slot = []
        for s in specs:
            slot.append({"qcodes": torch.empty((s.N, s.K // 32, 3), dtype=torch.int32, device=dev),
                         "scales": torch.empty(s.N, dtype=torch.float16, device=dev),
                         "zeros": torch.empty(s.N, dtype=torch.uint8, device=dev),
                         "w_weak": torch.empty((s.N, s.k), dtype=torch.float16, device=dev),
                         "weak_idx": torch.empty(s.k, dtype=torch.int32, device=dev)})
        slots.append(slot)
    y1 = [torch.empty((max(SWEEP_MS), s.N), dtype=torch.float16, device=dev) for s in specs]
    yd = [y[:1] for y in y1]
    yp = [torch.empty((PREFILL_M, s.N), dtype=torch.float16, device=dev) for s in specs]

    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    flush_buf = []

    def clean_time(fn, reps):
        """Median device time of fn() over reps calls, each after a read-only
        stream over 1 GiB (the caches then hold clean lines of another buffer)."""
        if not flush_buf:
            flush_buf.append(torch.ones((1 << 30) // 12 * 12, dtype=torch.uint8, device=dev))
        ts = []
        for _ in range(reps):
            owq.stream_read(flush_buf[0])
            a, b = E(), E()
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) / 1e3)
        return float(np.median(ts))

    def graph_time(fn, reps=5):
        """Device time of fn() (ROTATE layers' calls) replayed from a HIP graph."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        g.replay()
        torch.cuda.synchronize()
        a, b = E(), E()
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        del g
        return a.elapsed_time(b) / 1e3 / (reps * ROTATE)


    # the layer's calibration, with its arguments marshalled once
    cal_call = owq.PreparedCalibrate(W, X)

    # events of the calibration phase: ev[0] before calibrating the 7 linears
    # (one batched call), ev[1] after it, ev[2] after the selection (one batched
    # call for the 7), ev[3] after packing them (one batched call)
    def calibrate_pack(slot, ev=None):
        if ev is not None:
            ev[0].record()
        scores = [sc for _, sc in cal_call()]
        if ev is not None:
            ev[1].record()
        idxs = owq.select_weak_batched(scores, [s.k for s in specs], outs=[slot[li]["weak_idx"] for li in range(L)])
        if ev is not None:
            ev[2].record()
        owq.pack_batched(W, idxs, outs=slot)
        if ev is not None:
            ev[3].record()

    # fill every rotation slot before timing
    for r in range(ROTATE):
        calibrate_pack(slots[r])
    torch.cuda.synchronize()

    # the decode launches of each copy, with their arguments marshalled once (the
    # packed copies are rewritten in place, so the pointers stay valid)
    cur = torch.cuda.current_stream()  # the timed calls' stream, fixed once
    dec_calls = [owq.PreparedBatched(slots[r], xd, yd, stream=cur) for r in range(ROTATE)]
    decode_bytes = sum(eff_bytes(s.N, s.K, s.k, 1) for s in specs)
    CE = 4  # calibration-phase events
    NE = CE + 2 + L + 1  # calibration phase, decode pair, prefill boundaries

    def step(i, ev):
        cal_slot = slots[i % ROTATE]
        calibrate_pack(cal_slot, ev)
        o = CE
        ev[o].record()
        for r in range(1, ROTATE + 1):  # the copy written above comes last
            dec_calls[(i + r) % ROTATE]()
        ev[o + 1].record()
        o += 2
        for li in range(L):
            ev[o + li].record()
            owq.linear(cal_slot[li], xp[li], yp[li])
        ev[o + L].record()

    print(f"bench: warmup {args.warmup}", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i, [E() for _ in range(NE)])
    torch.cuda.synchronize()

    print(f"bench: timing {args.steps} steps", file=sys.stderr, flush=True)
    evs = [[E() for _ in range(NE)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    print("bench: timed steps done", file=sys.stderr, flush=True)

    def mean_ms(a, b):
        return float(np.mean([e[a].elapsed_time(e[b]) for e in evs]))

    cal_in_step = mean_ms(0, 1) / 1e3
    # the calibration again on its own, each repetition after a read-only pass
    # over 1 GiB: in the step it follows the previous step's prefill, whose
    # output writes are still draining to HBM while it reads
    cal_s = [clean_time(cal_call, 10)]
    sel_s = [mean_ms(1, 2) / 1e3]
    pak_s = [mean_ms(2, 3) / 1e3]
    o = CE
    dec_s = mean_ms(o, o + 1) / 1e3 / ROTATE
    dec_min_s = min(e[o].elapsed_time(e[o + 1]) for e in evs) / 1e3 / ROTATE
    o += 2
    pre_s = [mean_ms(o + li, o + li + 1) / 1e3 for li in range(L)]

    value = decode_bytes / dec_s / 1e9
    cal_bytes = sum(calib_bytes(s.N, s.K, cfg.T) for s in specs)
    pk_bytes = sum(pack_bytes(s.N, s.K, s.k) for s in specs)
    pre_flops = sum(2 * PREFILL_M * s.N * s.K for s in specs)
    pre_tflops = pre_flops / sum(pre_s) / 1e12
    per_linear_prefill = {}
    for li, s in enumerate(specs):
        tf = 2 * PREFILL_M * s.N * s.K / pre_s[li] / 1e12
        per_linear_prefill[f"{s.name} {s.N}x{s.K}"] = {"us": round(pre_s[li] * 1e6, 1), "tflops": round(tf, 1)}

    traffic = measured_traffic()
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
        "data": "synthetic (seeded Gaussian weights and activations with planted outlier channels)",
        "config": {"workload": "llama7b_layer_decode: one LLaMA-7B decoder layer, 7 linears (4x 4096x4096 k=32, "
                               "2x 11008x4096 k=32, 4096x11008 k=86), 3-bit codes + fp16 weak columns; "
                               "decode M=1, calibration T=2048, prefill M=2048",
                   "decode_M": 1, "calib_T": cfg.T, "prefill_M": PREFILL_M, "bits": 3,
                   "decode_effective_bytes": decode_bytes, "rotation_copies": ROTATE,
                   "decode_layers_per_step": ROTATE},
        "roofline": {"kernel": "k_gemv<1> (decode GEMV, one launch over the 7 linears)", "bound": "hbm",
                     "achieved": round(value, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(value / HBM_PEAK_GBS, 4), "traffic": traffic},
        "kernels": {
            "decode": dict(hbm_entry(decode_bytes, dec_s, "k_gemv<1>, 7 linears in one launch; "
                                     "per layer, 8 layers back to back"),
                           us_min=round(dec_min_s * 1e6, 2)),
            "prefill": {"what": "k_gemm_dma (MFMA 32x32x16 f16), 7 linears at M=2048", "us": round(sum(pre_s) * 1e6, 1),
                        "bound": "mfma", "achieved": round(pre_tflops, 1), "peak": MFMA_FP16_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(pre_tflops / MFMA_FP16_PEAK_TFLOPS, 4),
                        "algorithmic_flops": pre_flops, "per_linear": per_linear_prefill},
            "calibrate_score": dict(hbm_entry(cal_bytes, sum(cal_s), "k_calib_fused, the 7 linears in one "
                                              "owq_calibrate_score_batched call (3 launches: the K = 4096 linears, "
                                              "the K = 11008 linear with the others' final sums, its final sums); "
                                              "median of 10 calls, each after a read-only pass over 1 GiB"),
                                    us_in_step=round(cal_in_step * 1e6, 2)),
            "select_weak": {"what": "k_topk_reg_batched, the 7 linears in one owq_select_weak_batched call (one "
                                    "launch, 11 keys x 16 waves per selection)",
                            "us": round(sum(sel_s) * 1e6, 1), "bound": "latency"},
            "pack": hbm_entry(pk_bytes, sum(pak_s), "owq_pack_batched over the 7 linears: k_pack_w (a wave per "
                                                    "row) for the six K = 4096 linears in one launch, k_pack (a "
                                                    "block per row) for down_proj"),
        },
    }

    if not args.no_sweep:
        print("bench: decode batch sweep", file=sys.stderr, flush=True)
        sweep = {}
        reps = 2 * ROTATE
        for M in SWEEP_MS:
            xs = [x[:M] for x in x1]
            ys = [y[:M] for y in y1]
            calls = [owq.PreparedBatched(slots[r], xs, ys, stream=cur) for r in range(ROTATE)]
            for r in range(ROTATE):
                calls[r]()
            a, b = E(), E()
            a.record()
            for r in range(reps):  # back to back, as in the timed steps
                calls[r % ROTATE]()
            b.record()
            torch.cuda.synchronize()
            t = a.elapsed_time(b) / 1e3 / reps
            nb = sum(eff_bytes(s.N, s.K, s.k, M) for s in specs)
            sweep[f"M={M}"] = {"us_per_layer": round(t * 1e6, 2), "effective_GBps": round(nb / t / 1e9, 1),
                               "frac_hbm": round(nb / t / 1e9 / HBM_PEAK_GBS, 4),
                               "path": ("k_gemv, one launch" if M == 1 else "k_gemv_mfma (products on the matrix cores), one launch"
                                        if M == 2 else "k_mfv, one launch")}
        result["decode_batch_sweep"] = sweep

    if not args.no_extras:
        # the layer's calibration as one owq_calibrate_score call per linear (2
        # launches each), for comparison with the batched call timed above
        one = [owq.PreparedCalibrate([W[li]], [X[li]]) for li in range(L)]
        reps = 5
        evc = [(E(), E()) for _ in range(reps)]
        for r in range(reps):
            evc[r][0].record()
            for li in range(L):
                one[li]()
            evc[r][1].record()
        torch.cuda.synchronize()
        t = float(np.median([a.elapsed_time(b) for a, b in evc])) / 1e3
        result["kernels"]["calibrate_score"]["us_one_call_per_linear"] = round(t * 1e6, 2)
        del one

        # the same decode as 7 launches per layer (one per linear), recorded in a HIP graph
        print("bench: decode as per-linear launches in a graph", file=sys.stderr, flush=True)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for r in range(ROTATE):
                for li in range(L):
                    owq.linear(slots[r][li], xd[li], yd[li])
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for r in range(ROTATE):
                for li in range(L):
                    owq.linear(slots[(r + 1) % ROTATE][li], xd[li], yd[li])
        g.replay()
        torch.cuda.synchronize()
        reps = 10
        a, b = E(), E()
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        t = a.elapsed_time(b) / 1e3 / (reps * ROTATE)
        result["kernels"]["decode_graph"] = hbm_entry(
            decode_bytes, t, f"k_gemv<1>, 7 launches per layer ({ROTATE} layers) replayed from a HIP graph")
        del g

        # the same prefill products as plain fp16 GEMMs on the unquantised weights
        # (torch / hipBLASLt), for comparison with the fused 3-bit kernel
        ref = {}
        for li, s in enumerate(specs):
            for _ in range(3):
                torch.nn.functional.linear(xp[li], W[li])
            a, b = E(), E()
            a.record()
            for _ in range(5):
                torch.nn.functional.linear(xp[li], W[li])
            b.record()
            torch.cuda.synchronize()
            t = a.elapsed_time(b) / 1e3 / 5
            ref[f"{s.name} {s.N}x{s.K}"] = round(2 * PREFILL_M * s.N * s.K / t / 1e12, 1)
        tot = sum(2 * PREFILL_M * s.N * s.K for s in specs)
        tt = sum(2 * PREFILL_M * s.N * s.K / (v * 1e12) for s, v in zip(specs, ref.values()))
        result["kernels"]["prefill_fp16_gemm_reference"] = {
            "what": "torch.nn.functional.linear on the fp16 weights (not the product path)",
            "achieved": round(tot / tt / 1e12, 1), "unit": "TFLOP/s", "per_linear_tflops": ref}

        # the M = 1 decode of the layer as fp16 matrix-vector products on the
        # unquantised weights (torch), for the speed-up of the 3.1-bit format
        for li in range(L):
            torch.nn.functional.linear(xd[li], W[li])
        a, b = E(), E()
        a.record()
        for _ in range(5):
            for li in range(L):
                torch.nn.functional.linear(xd[li], W[li])
        b.record()
        torch.cuda.synchronize()
        t = a.elapsed_time(b) / 1e3 / 5
        fp16_bytes = sum(2 * s.N * s.K + 2 * s.K for s in specs)
        result["kernels"]["decode_fp16_gemv_reference"] = {
            "what": "torch.nn.functional.linear at M = 1 on the fp16 weights, 7 launches (not the product path)",
            "us": round(t * 1e6, 2), "achieved": round(fp16_bytes / t / 1e9, 1), "unit": "GB/s",
            "speedup_of_owq_decode": round(t / dec_s, 2)}

        # measured device-copy rate over 1 GiB (read + write), for comparison with the 8 TB/s peak
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        a, b = E(), E()
        a.record()
        for _ in range(5):
            dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        t = a.elapsed_time(b) / 1e3 / 5
        result["kernels"]["hbm_copy_reference"] = {"what": "device copy of 1 GiB (torch copy_)",
                                                   "read_plus_write_GBps": round(2 * n / t / 1e9, 1),
                                                   "frac": round(2 * n / t / 1e9 / HBM_PEAK_GBS, 4)}
        del src, dst

        # measured read-only stream rates: torch.sum over 1 GiB, and over copies of the
        # decode layer's size (one launch each, copies rotated so the last-level cache
        # holds none of them), for comparison with the decode kernel's one launch
        rd = {}
        for label, nbytes, copies in (("1GiB", 1 << 30, 1), ("layer_size", decode_bytes, ROTATE)):
            bufs = [torch.ones(nbytes // 2, dtype=torch.float16, device=dev) for _ in range(copies)]
            for t_ in bufs:
                torch.sum(t_)
            reps = 8 * copies if copies > 1 else 5
            a, b = E(), E()
            a.record()
            for r in range(reps):
                torch.sum(bufs[r % copies])
            b.record()
            torch.cuda.synchronize()
            t = a.elapsed_time(b) / 1e3 / reps
            rd[label] = {"bytes": nbytes // 2 * 2, "us": round(t * 1e6, 2),
                         "read_GBps": round(nbytes // 2 * 2 / t / 1e9, 1),
                         "frac": round(nbytes // 2 * 2 / t / 1e9 / HBM_PEAK_GBS, 4)}
            del bufs
        result["kernels"]["hbm_read_reference"] = dict(
            what="torch.sum over fp16 buffers (read-only stream, one launch per sum; not the product path)", **rd)

        # the library's read-only stream at the decode kernel's geometry and the decode
        # layer's size (one launch per copy, copies rotated): the rate one launch of
        # this shape reaches when it does nothing with the bytes
        sr = {}
        for label, nbytes, copies in (("layer_size", decode_bytes // 12 * 12, ROTATE), ("1GiB", (1 << 30) // 12 * 12, 1)):
            bufs = [torch.ones(nbytes, dtype=torch.uint8, device=dev) for _ in range(copies)]
            sinks = [owq.stream_read(b) for b in bufs]
            reps = 8 * copies if copies > 1 else 5
            a, b = E(), E()
            a.record()
            for r in range(reps):
                owq.stream_read(bufs[r % copies], sinks[r % copies])
            b.record()
            torch.cuda.synchronize()
            t = a.elapsed_time(b) / 1e3 / reps
            sr[label] = {"bytes": nbytes, "us": round(t * 1e6, 2), "read_GBps": round(nbytes / t / 1e9, 1),
                         "frac": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4)}
            del bufs, sinks
        sr["decode_vs_layer_size_stream"] = round(value / sr["layer_size"]["read_GBps"], 4)
        result["kernels"]["stream_read_reference"] = dict(
            what="owq_stream_read: loads only, the M = 1 decode geometry (6 x 768 B per wavefront, non-temporal, 4-wave "
                 "blocks), one launch per buffer (not the product path)", **sr)

    if not args.no_long_calibration:
        # long calibration (T = 8192 tokens) at the MLP shapes: X and W read once
        print("bench: long calibration", file=sys.stderr, flush=True)
        c4 = synth.LLAMA7B_MLP_PREFILL_CALIB
        long_cal, long_sel = {}, {}
        for li, s in enumerate(c4.layers):
            seed = c4.seed(li)
            Wl = torch.from_numpy(synth.weights(s, seed)).to(dev)
            Xl = torch.from_numpy(synth.calibration(s, seed, c4.T)).to(dev)
            call = owq.PreparedCalibrate([Wl], [Xl])  # one linear: owq_calibrate_score's launches
            _, score_l = call()[0]
            owq.select_weak(score_l, s.k)
            t = clean_time(call, 5)
            ts = clean_time(lambda: owq.select_weak(score_l, s.k), 5)
            key = f"{s.name} {s.N}x{s.K} T={c4.T}"
            long_cal[key] = hbm_entry(calib_bytes(s.N, s.K, c4.T), t, "k_calib_fused (W row fits and errors, X "
                                                                       "column tiles) + k_calib_fin, one linear; "
                                                                       "median of 5 calls, each after a read-only "
                                                                       "pass over 1 GiB")
            long_sel[key] = {"what": f"top-{s.k} of K = {s.K}", "us": round(ts * 1e6, 2), "bound": "latency"}
            del Wl, Xl, call
        result["kernels"]["calibrate_score_long"] = long_cal
        result["kernels"]["select_weak_long"] = long_sel

    if not args.no_large:
        # decode of the large shapes (8192x8192, 28672x8192, 8192x28672) at M = 1
        # and 8: calibrated and packed like the layer above, three copies rotated
        # (3 x 210 MB) so the bytes come from HBM, one launch per copy
        print("bench: large shapes", file=sys.stderr, flush=True)
        c3 = synth.LARGE_SHAPES
        RL = 3
        big = [[] for _ in range(RL)]
        for li, s in enumerate(c3.layers):
            seed = c3.seed(li)
            Wl = torch.from_numpy(synth.weights(s, seed)).to(dev)
            Xl = torch.from_numpy(synth.calibration(s, seed, c3.T)).to(dev)
            wsl = torch.empty(owq.calibrate_workspace_bytes(s.N, s.K, c3.T), dtype=torch.uint8, device=dev)
            _, score_l = owq.calibrate(Wl, Xl, workspace=wsl)
            p = owq.pack(Wl, owq.select_weak(score_l, s.k))
            for r in range(RL):
                big[r].append(p if r == 0 else {key: v.clone() for key, v in p.items()})
            del Wl, Xl, wsl, score_l
        xb = [torch.from_numpy(synth.activations(s, c3.seed(li), 8)).to(dev) for li, s in enumerate(c3.layers)]
        yb = [torch.empty((8, s.N), dtype=torch.float16, device=dev) for s in c3.layers]
        large = {}
        for M in (1, 8):
            calls = [owq.PreparedBatched(big[r], [x[:M] for x in xb], [y[:M] for y in yb], stream=cur)
                     for r in range(RL)]
            for r in range(RL):
                calls[r]()
            reps = 4 * RL
            a, b = E(), E()
            a.record()
            for r in range(reps):
                calls[r % RL]()
            b.record()
            torch.cuda.synchronize()
            t = a.elapsed_time(b) / 1e3 / reps
            nb = sum(eff_bytes(s.N, s.K, s.k, M) for s in c3.layers)
            large[f"M={M}"] = hbm_entry(nb, t, ("k_gemv" if M <= 2 else "k_mfv") +
                                        ", 8192x8192 + 28672x8192 + 8192x28672 in one launch")
        result["kernels"]["large_shapes_decode"] = large
        del big, xb, yb

    if not args.no_extras:
        # the storage-favoured form of the same layer at M = 1 (the pages' other
        # format): the dense codes of K - k columns, x gathered at the dense
        # columns, the weak columns in the decode's own sum; 2 launches per
        # layer, compared with the one launch per layer of the latency form
        print("bench: storage-favoured decode", file=sys.stderr, flush=True)
        # ROTATE copies in the storage form, the 7 linears of a copy in one
        # owq_linear_storage_batched call; device time from a HIP graph
        sto = [[owq.pack_storage(W[li], slots[r][li]["weak_idx"]) for li in range(L)] for r in range(ROTATE)]
        wss = torch.empty(owq.linear_storage_batched_workspace_bytes(sto[0], 1), dtype=torch.uint8, device=dev)

        def storage_batched():
            for r in range(ROTATE):
                owq.linear_storage_batched(sto[r], xd, yd, workspace=wss)

        def storage_per_linear():
            for r in range(ROTATE):
                for li in range(L):
                    owq.linear_storage(sto[r][li], xd[li], yd[li], wss)

        t = graph_time(storage_batched)
        t_one = graph_time(storage_per_linear)
        sto_bytes = sum(3 * s.N * (s.K - s.k) // 8 + 3 * s.N + 2 * s.N * s.k + 2 * s.K for s in specs)
        result["kernels"]["decode_storage_form"] = dict(
            hbm_entry(sto_bytes, t, "storage-favoured form at M=1: owq_linear_storage_batched over the 7 linears "
                                    "(x gathered at the dense columns, then k_gemv<1> over K - k columns with the weak "
                                    "columns from the full x in the same sum: 2 launches per layer), 8 copies "
                                    "rotated, replayed from a HIP graph (device time)"),
            us_one_call_per_linear_graph=round(t_one * 1e6, 2),
            us_latency_form=round(dec_s * 1e6, 2))
        del sto, wss

        # group-wise scales on top of OWQ (the pages' grouped comparison, groups
        # of 128 columns): pack of the 7 linears, and their product at M = 1
        # (one launch per linear), 8 copies rotated, from a HIP graph
        print("bench: group-wise form", file=sys.stderr, flush=True)
        GW = 128
        grp = [[owq.pack_grouped(W[li], slots[r][li]["weak_idx"], GW) for li in range(L)] for r in range(ROTATE)]
        torch.cuda.synchronize()

        def grouped_decode():
            for r in range(ROTATE):
                owq.linear_grouped_batched(grp[r], xd, yd)

        def grouped_pack():
            for r in range(ROTATE):
                for li in range(L):
                    owq.pack_grouped(W[li], slots[r][li]["weak_idx"], GW, out=grp[r][li])

        t = graph_time(grouped_decode)
        tp = graph_time(grouped_pack)
        g_bytes = sum(3 * s.N * s.K // 8 + 3 * s.N * (s.K // GW) + 2 * s.N * s.k + 2 * s.K for s in specs)
        gp_bytes = sum(2 * s.N * s.K + 4 * s.k + 3 * s.N * s.K // 8 + 3 * s.N * (s.K // GW) + 2 * s.N * s.k
                       for s in specs)
        result["kernels"]["decode_grouped_form"] = dict(
            hbm_entry(g_bytes, t, f"group-wise form (a step and zero point per row and {GW} columns) at M=1: "
                                  "owq_linear_grouped_batched over the 7 linears (k_gemv_grouped<1>: the decode kernel "
                                  "with a zero point and step per 32-column code group), one launch per layer, 8 "
                                  "copies rotated, replayed from a HIP graph (device time)"),
            us_latency_form=round(dec_s * 1e6, 2))
        result["kernels"]["pack_grouped"] = hbm_entry(
            gp_bytes, tp, f"owq_pack_grouped, G = {GW}, the 7 linears (k_pack_grouped, a thread per 32 columns, "
                          "+ k_weak_copy), from a HIP graph (device time)")
        del grp

        # one GPU's share of the layer under 8-way column-parallel sharding (the
        # multi-GPU layout: every GPU holds N / 8 rows of each linear, x and the
        # weak index set replicated, no exchange for y = W x): the same batched
        # M = 1 decode over row slices of the packed layers, 56 copies (the 8
        # shards of 7 layer copies, 555 MB) rotated so the footprint exceeds the
        # 256 MB Infinity Cache
        print("bench: one GPU's share at 8-way sharding", file=sys.stderr, flush=True)
        G, NSH = 8, 56
        shard = []
        for r in range(NSH):
            g, src = r % G, slots[r % ROTATE]
            lay = []
            for li, sp in enumerate(specs):
                a, b = (sp.N // G) * g, (sp.N // G) * (g + 1)
                lay.append({"qcodes": src[li]["qcodes"][a:b].clone(), "scales": src[li]["scales"][a:b].clone(),
                            "zeros": src[li]["zeros"][a:b].clone(), "w_weak": src[li]["w_weak"][a:b].clone(),
                            "weak_idx": src[li]["weak_idx"]})
            shard.append(lay)
        ysh = [torch.empty((1, sp.N // G), dtype=torch.float16, device=dev) for sp in specs]

        def shard_all():  # the stream is taken at each call (graph capture)
            for r in range(NSH):
                owq.linear_batched(shard[r], xd, ysh)

        t = graph_time(shard_all) * ROTATE / NSH
        sh_bytes = sum(eff_bytes(sp.N // G, sp.K, sp.k, 1) for sp in specs)
        result["kernels"]["decode_shard_g8"] = dict(
            hbm_entry(sh_bytes, t, "one GPU's share of the layer at 8-way column-parallel sharding (N / 8 rows of "
                                   "each linear, x replicated): owq_linear_batched at M = 1, one k_gemv<1> launch, "
                                   "56 copies rotated, replayed from a HIP graph (device time); the collective "
                                   "(an all-gather of y, if the next layer needs it whole) is not measured"),
            rows_per_gpu={sp.name: sp.N // G for sp in specs})
        del shard

    if not args.no_extras:
        # weak-column-tuning backward of the layer: dx = dy W and dw_weak = dy^T
        # x[:, idx] for the 7 linears, at M = 1 and 16 (8 packed copies rotated)
        print("bench: weak-column-tuning backward", file=sys.stderr, flush=True)
        bw = {}
        bws = torch.empty(owq.linear_backward_batched_workspace_bytes(slots[0]), dtype=torch.uint8, device=dev)
        for M in (1, 16):
            dys = [torch.randn((M, s.N), device=dev).to(torch.float16) for s in specs]
            xs_b = [x1[li][:M] for li in range(L)]

            def batched():
                for r in range(ROTATE):
                    owq.linear_backward_batched(slots[r], xs_b, dys, workspace=bws)

            def per_linear():
                for r in range(ROTATE):
                    for li in range(L):
                        owq.linear_backward(slots[r][li], x1[li][:M], dys[li], workspace=bws)

            batched()
            torch.cuda.synchronize()
            a, b = E(), E()
            a.record()
            batched()
            b.record()
            torch.cuda.synchronize()
            t_eager = a.elapsed_time(b) / 1e3 / ROTATE
            t = graph_time(batched)
            t_one = graph_time(per_linear)
            nb = sum(3 * s.N * s.K // 8 + 3 * s.N + 2 * s.N * s.k + 2 * M * s.N + 2 * M * s.K + 2 * M * s.k
                     + 4 * s.N * s.k for s in specs)
            bw[f"M={M}"] = dict(
                hbm_entry(nb, t, "owq_linear_backward_batched over the 7 linears, replayed from a HIP graph "
                                 "(device time): up to 4 tokens k_bwd_part (dx slice partials with the weak columns, "
                                 "and dw_weak) + k_bwd_dx_finalize per 4 tokens; more tokens k_bwd_mma (dx on the "
                                 "matrix cores in fp16, 16 tokens per pass, weak-column partials, dw_weak) + "
                                 "k_bwd_mma_finalize + k_bwd_mma_weak_finalize per 16 tokens"),
                us_eager_python_call=round(t_eager * 1e6, 2),
                us_one_call_per_linear_graph=round(t_one * 1e6, 2))
        result["kernels"]["backward_weak_column_tuning"] = bw
        del bws

    if not args.no_search:
        # OPTQ with the weak columns last (owq_pack_optq) on the two K = 4096
        # shapes of the layer: an offline step, timed whole
        print("bench: OPTQ pack", file=sys.stderr, flush=True)
        oq = {}
        for li in (0, 4):
            s = specs[li]
            _, score_o = owq.calibrate(W[li], X[li], workspace=ws)
            idx_o = owq.select_weak(score_o, s.k)
            wso = torch.empty(owq.pack_optq_workspace_bytes(s.N, s.K, s.k), dtype=torch.uint8, device=dev)
            outo = owq.pack_optq(W[li], X[li], idx_o, workspace=wso)
            a, b = E(), E()
            a.record()
            owq.pack_optq(W[li], X[li], idx_o, out=outo, workspace=wso)
            b.record()
            torch.cuda.synchronize()
            oq[f"{s.name} {s.N}x{s.K} T={cfg.T}"] = {"ms": round(a.elapsed_time(b), 2)}
            del wso, outo
        result["kernels"]["pack_optq"] = dict(
            oq, what="owq_pack_optq: Hessian, damping, reversed-order Cholesky and triangular inverse (blocked, each "
                     "entry's sum in the definition's order), column-by-column quantisation in batches of 128 with "
                     "compensation, pack (offline step)")

    # share of the total column score carried by the k selected columns, per
    # linear (most of the output error comes from a few channels)
    share = {}
    for li, s in enumerate(specs):
        _, score = owq.calibrate(W[li], X[li], workspace=ws)
        sc = score.cpu().numpy()
        top = np.sort(sc)[::-1][:s.k].sum()
        share[f"{s.name} {s.N}x{s.K}"] = {"k": s.k, "K": s.K, "topk_share_of_score": round(float(top / sc.sum()), 4),
                                          "k_over_K": round(s.k / s.K, 5)}
    result["topk_score_share"] = share

    if not args.no_search:
        # truncation-aware (step, zero point) search + pack for the 7 linears,
        # weighted by the Hessian diagonal (owq_pack_search): ALU-bound
        print("bench: truncation-aware pack", file=sys.stderr, flush=True)
        lams, idxs = [], []
        for li, s in enumerate(specs):
            lam_l, score_l = owq.calibrate(W[li], X[li], workspace=ws)
            lams.append(lam_l)
            idxs.append(owq.select_weak(score_l, s.k))
        outs = [owq.pack_search(W[li], idxs[li], lams[li]) for li in range(L)]
        reps = 3
        ev = [[E() for _ in range(L + 1)] for _ in range(reps)]
        for r in range(reps):
            for li in range(L):
                ev[r][li].record()
                owq.pack_search(W[li], idxs[li], lams[li], out=outs[li])
            ev[r][L].record()
        torch.cuda.synchronize()
        t = float(np.median([ev[r][0].elapsed_time(ev[r][L]) for r in range(reps)])) / 1e3
        evals = sum(s.N * (s.K - s.k) * SEARCH_GRID for s in specs)
        ops = evals * SEARCH_OPS_PER_EVAL
        result["kernels"]["pack_search"] = {
            "what": "k_search (32 steps x 8 zero points per row, Hessian-diagonal weighted) + k_pack with the "
                    "chosen parameters, 7 linears", "us": round(t * 1e6, 1), "bound": "alu",
            "achieved": round(ops / t / 1e12, 2), "peak": ALU_PEAK_TOPS, "unit": "Tops/s (lane ops)",
            "frac": round(ops / t / 1e12 / ALU_PEAK_TOPS, 4), "grid_point_evaluations": evals,
            "ops_per_evaluation": SEARCH_OPS_PER_EVAL}

    if args.copy_reference:
        n = 512 << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_reference_bytes"] = n

    if not args.no_cpu_baseline:
        print("bench: CPU oracle baseline", file=sys.stderr, flush=True)
        result["cpu_baseline"], packed_layers = cpu_baseline(cfg, args.cpu_seconds)
        host = host_description()
        result["cpu_baseline"]["host"] = host
        if not args.no_cpu_extra:
            print("bench: CPU oracle, threaded and calibration legs", file=sys.stderr, flush=True)
            result["cpu_baseline_extra"] = cpu_extra_legs(host["omp_threads"], packed_layers)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
