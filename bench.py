"""Benchmark: decode GEMV and prefill GEMM of weight-only quantized linear layers
on one MI355X.

Headline (the JSON `value`): 4-bit gs64 qGEMV weight GB/s, decode W[14336, 4096]
(8B-class MLP shape) with bf16 scales/biases and x bf16 [1, 4096]. One step =
one qmatmul call (the whole hot path of the decode step: stream + unpack +
affine + reduce). Weight bytes = codes + scales + biases = 33,030,144 B.
The timed region cycles through >= 512 MB of distinct weight copies so every
launch streams from HBM, not from the 256 MB Infinity Cache.

Secondary (in `secondary`): 4-bit prefill qGEMM TFLOP/s on x bf16 [2048, 4096]
x W[14336, 4096]^T, against the bf16 dense MFMA peak.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
MALL_BYTES = 256 << 20


def weight_bytes(n, k, bits, gs, sb_bytes):
    return n * k * bits // 8 + 2 * n * (k // gs) * sb_bytes


def make_weights(n, k, bits, gs, copies, seed, dev):
    import torch
    import weight_only_quantized_qgemv_amd as qp
    from weight_only_quantized_qgemv_amd import synth
    w = torch.from_numpy(synth.normal_f32((n, k), 0.02, seed)).to(dev)
    base = qp.qpack_quantize(w, bits, gs, torch.bfloat16)
    del w
    sets = [base] + [tuple(t.clone() for t in base) for _ in range(copies - 1)]
    torch.cuda.synchronize()
    return sets


def time_calls(fn, steps, warmup, stream):
    """Average ms per call over `steps` back-to-back calls, events on `stream`."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        fn(i)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def cpu_baseline(n, k, bits, gs, budget_s=10.0):
    """The oracle (plain C, OpenMP over outputs) on the same decode workload:
    whole M=1 calls on the full weight matrix, repeated for ~budget_s."""
    import numpy as np
    import torch
    from oracle import qref
    from weight_only_quantized_qgemv_amd import synth
    w = synth.normal_f32((n, k), 0.02, 21)
    wq, s, b = qref.quantize(w, bits, gs, qref.BF16)
    x = torch.from_numpy(synth.normal_f32((1, k), 1.0, 22)).to(torch.bfloat16)
    xs = x.view(torch.int16).numpy().view(np.uint16)
    runs, t0 = 0, time.perf_counter()
    while True:
        qref.qmatmul(xs, qref.BF16, wq, s, b, qref.BF16, k, bits, gs)
        runs += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    wb = weight_bytes(n, k, bits, gs, 2)
    return {"value": round(wb * runs / el / 1e9, 4), "unit": "GB/s", "cores": qref.num_threads(),
            "kind": "oracle",
            "sample": f"{runs} whole decode calls (M=1, W[{n},{k}] {bits}-bit gs{gs} bf16), "
                      f"{el:.1f} s; dequant + fp64 dot per output, OpenMP over outputs"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this build measures one GPU only (no multi-GPU path); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import weight_only_quantized_qgemv_amd as qp
    from weight_only_quantized_qgemv_amd import synth

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    N, K, BITS, GS = 14336, 4096, 4, 64
    wb = weight_bytes(N, K, BITS, GS, 2)
    copies = max(2, -(-2 * MALL_BYTES // wb))   # > 2x the Infinity Cache in total
    sets = make_weights(N, K, BITS, GS, copies, 21, dev)
    x = torch.from_numpy(synth.normal_f32((1, K), 1.0, 22)).to(torch.bfloat16).to(dev)
    y = torch.empty((1, N), dtype=torch.bfloat16, device=dev)

    def step(i):
        wq, s, b = sets[i % copies]
        qp.qmatmul(x, wq, s, b, BITS, GS, out=y)

    ms = time_calls(step, args.steps, args.warmup, stream)
    gbs = wb / (ms * 1e-3) / 1e9
    result = {
        "metric": "4-bit gs64 qGEMV weight GB/s (% HBM peak); qGEMM TFLOP/s (% bf16 MFMA)",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) weights quantized on device, N(0,1) activations)",
        "config": {"workload": "decode qGEMV W[14336,4096] 4-bit gs64 bf16 scales/biases, "
                               "x bf16 [1,4096], fp32 accumulation",
                   "weight_bytes_per_call": wb, "weight_copies": copies,
                   "rotation_bytes": wb * copies},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "qgemv_stream_kernel (4-bit, bf16, MT=1, U=2)",
                     "us_per_launch": round(ms * 1e3, 3)},
    }
    del sets
    torch.cuda.empty_cache()

    if not args.no_secondary:
        # Prefill qGEMM: x bf16 [2048, 4096] x W[14336, 4096]^T (4-bit gs64).
        M = 2048
        psets = make_weights(N, K, BITS, GS, 2, 41, dev)
        xp = torch.from_numpy(synth.normal_f32((M, K), 1.0, 43)).to(torch.bfloat16).to(dev)
        yp = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

        def pstep(i):
            wq, s, b = psets[i % 2]
            qp.qmatmul(xp, wq, s, b, BITS, GS, out=yp)

        pms = time_calls(pstep, max(5, args.steps // 20), 3, stream)
        tflops = 2.0 * M * N * K / (pms * 1e-3) / 1e12
        result["secondary"] = {
            "qgemm_prefill": {"workload": "x bf16 [2048,4096] x W[14336,4096]^T 4-bit gs64",
                              "tflops": round(tflops, 2), "ms": round(pms, 4),
                              "frac_of_bf16_mfma_peak": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)}}
        del psets
        torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(N, K, BITS, GS)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
