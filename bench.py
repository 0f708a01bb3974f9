"""Benchmark: weight-only quantized linear layers (qGEMV decode, qGEMM prefill,
routed MoE) on one MI355X.

Headline (the JSON `value`): 4-bit gs64 qGEMV weight GB/s on the decode shape
W[14336, 4096] (8B-class MLP) with bf16 scales/biases and x bf16 [1, 4096].
One step = one qmatmul call: the whole hot path of a decode linear layer
(stream the packed codes, unpack, affine dequant, contract, reduce, store).
Weight bytes = codes + scales + biases = 33,030,144 B per call. The timed
region cycles through >= 512 MB of distinct weight copies (more than twice the
256 MB Infinity Cache), so every launch streams its weights from HBM.

Every other row of the hot path is measured too, in `rows`: decode at 2/4/8
bits and M = 1/4/16, the cross-word 3/6-bit layouts over three group sizes,
both prefill GEMM shapes against the bf16 MFMA peak, the MoE gate+up+SiLU
and down calls at T = 1/64/512 tokens, the unfused two-kernel form
(qpack_dequantize to a dense bf16 weight, then torch.matmul) at M = 1 and
2048 beside the fused call, and the microscaled modes (mxfp4, nvfp4, mxfp8)
at decode, prefill and dense-weight shapes.

Usage:
  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-rows]
  python bench.py --copy-calibration   # plain 1 GiB copies, to scale HBM counters
  python bench.py --case NAME          # one workload (profiler runs); NAME in CASES
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, TFLOP/s
MALL_BYTES = 256 << 20
ROTATE_BYTES = 2 * MALL_BYTES
CSRC = os.path.join(ROOT, "weight_only_quantized_qgemv_amd", "csrc")

# HBM traffic of the headline kernel per launch, from two rocprofv3 --pmc runs
# (FETCH_SIZE, WRITE_SIZE) of `bench.py --case decode_b4_m1 --steps 20
# --warmup 2`, each scaled by the same counter on a plain 1 GiB copy.
# It holds only while the decode kernel's sources are the ones it was taken on.
TRAFFIC = {"src_sha": "f3905fab68b2293d", "fetch_bytes": 33205382, "write_bytes": 57344,
           "fetch_scale": 2.0, "write_scale": 1.0}
DECODE_SOURCES = ("rowstream.hpp", "codepair.hpp", "gemv_core.hpp", "common.hpp", "qgemv.hip")

# Shader clock under the prefill's own load, from rocprofv3 --pmc GRBM_GUI_ACTIVE
# (summed over the 8 XCDs) against the kernel trace of the same command
# (`bench.py --case NAME --steps 10 --warmup 2`): the chip runs the matrix
# cores below the 2.4 GHz of the nominal peak. The prefill rows report their
# fraction of the bf16 matrix peak at this clock beside the nominal one.
PROFILED_CLOCK_GHZ = {"prefill_m2048_n14336_k4096": 1.77, "prefill_m2048_n4096_k14336": 1.86}
NOMINAL_CLOCK_GHZ = 2.4


def decode_src_sha() -> str:
    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def weight_bytes(n, k, bits, gs, sb_bytes):
    return n * k * bits // 8 + 2 * n * (k // gs) * sb_bytes


def make_weights(n, k, bits, gs, sb_dtype, copies, seed, dev):
    import torch
    import weight_only_quantized_qgemv_amd as qp
    from weight_only_quantized_qgemv_amd import synth
    w = torch.from_numpy(synth.normal_f32((n, k), 0.02, seed)).to(dev)
    base = qp.qpack_quantize(w, bits, gs, sb_dtype)
    del w
    sets = [base] + [tuple(t.clone() for t in base) for _ in range(copies - 1)]
    torch.cuda.synchronize()
    return sets


def copies_for(nbytes):
    return max(2, -(-ROTATE_BYTES // nbytes))


_SLEEP_CYCLES_PER_MS = None


def hold_stream(stream, calls, us_per_call=10.0):
    """Keeps `stream` busy on a device spin (torch's sleep kernel) for about
    `calls` x `us_per_call` microseconds, so that the host has queued all of
    the timed calls before the start event that follows it is reached. The
    timed region then holds device work only: without it, its first call
    starts one host issue time (about 5 us) after the start event, which at
    20 timed calls adds about 0.25 us to every call. The spin runs before the
    start event and is not part of any timed region."""
    import torch
    global _SLEEP_CYCLES_PER_MS
    if not hasattr(torch.cuda, "_sleep"):
        return   # no sleep kernel in this torch: time without the hold
    if _SLEEP_CYCLES_PER_MS is None:
        probe = 2_000_000
        with torch.cuda.stream(stream):
            torch.cuda._sleep(probe)   # first launch (module load), untimed
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        with torch.cuda.stream(stream):
            torch.cuda._sleep(probe)
        b.record(stream)
        torch.cuda.synchronize()
        _SLEEP_CYCLES_PER_MS = probe / max(a.elapsed_time(b), 1e-3)
    cycles = int(_SLEEP_CYCLES_PER_MS * calls * us_per_call * 1e-3)
    with torch.cuda.stream(stream):
        torch.cuda._sleep(max(cycles, 1))


def time_calls(fn, steps, warmup, stream, reps=5):
    """Median over `reps` of the mean ms per call over `steps` back-to-back
    calls, HIP events recorded on `stream` (the stream the kernels run on).
    Each repetition starts from a synchronized device, holds the stream
    (`hold_stream`) while the host queues the calls, and times exactly the
    `steps` calls between its two events."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    out = []
    for _ in range(reps):
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        hold_stream(stream, steps, 12.0)
        start.record(stream)
        for i in range(steps):
            fn(i)
        end.record(stream)
        torch.cuda.synchronize()
        out.append(start.elapsed_time(end) / steps)
    return statistics.median(out)


def graph_ms(fn, n, stream, reps=5):
    """Median over `reps` of the device period per call of n calls replayed from
    one captured HIP graph (no host issue between the launches), HIP events
    recorded on `stream` around each replay. For calls shorter than the host's
    issue time of one call, where back-to-back eager calls time the host."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        fn(0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    out = []
    for _ in range(reps):
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        hold_stream(stream, 1, 50.0)
        start.record(stream)
        g.replay()
        end.record(stream)
        torch.cuda.synchronize()
        out.append(start.elapsed_time(end) / n)
    del g
    return statistics.median(out)


def bench_dense(N, K, M, bits, gs, dt, steps, warmup, stream, dev, seed=21, graph=False,
                graph_calls=None):
    import torch
    import weight_only_quantized_qgemv_amd as qp
    from weight_only_quantized_qgemv_amd import synth
    es = torch.finfo(dt).bits // 8
    wb = weight_bytes(N, K, bits, gs, es)
    copies = copies_for(wb)
    sets = make_weights(N, K, bits, gs, dt, copies, seed, dev)
    x = torch.from_numpy(synth.normal_f32((M, K), 1.0, seed + 1)).to(dt).to(dev)
    y = torch.empty((M, N), dtype=dt, device=dev)

    def step(i):
        wq, s, b = sets[i % copies]
        qp.qmatmul(x, wq, s, b, bits, gs, out=y)

    ms = time_calls(step, steps, warmup, stream)
    if graph:
        ms = (ms, graph_ms(step, graph_calls or 8 * copies, stream))
    del sets
    torch.cuda.empty_cache()
    return ms, wb, copies


def bench_unfused(N, K, M, bits, gs, dt, steps, warmup, stream, dev, seed=21):
    """The two-kernel form the fused product replaces: qpack_dequantize to a
    dense [N, K] weight in the scales' type, then a dense torch.matmul. Returns
    (ms of the dequantize alone, ms of both, weight bytes)."""
    import torch
    import weight_only_quantized_qgemv_amd as qp
    from weight_only_quantized_qgemv_amd import synth
    es = torch.finfo(dt).bits // 8
    wb = weight_bytes(N, K, bits, gs, es)
    copies = copies_for(wb)
    sets = make_weights(N, K, bits, gs, dt, copies, seed, dev)
    x = torch.from_numpy(synth.normal_f32((M, K), 1.0, seed + 1)).to(dt).to(dev)
    y = torch.empty((M, N), dtype=dt, device=dev)
    wd = torch.empty((N, K), dtype=dt, device=dev)

    def deq(i):
        wq, s, b = sets[i % copies]
        qp.qpack_dequantize(wq, s, b, bits, gs, out=wd)

    def both(i):
        deq(i)
        torch.matmul(x, wd.t(), out=y)

    ms_deq = time_calls(deq, steps, warmup, stream)
    ms_both = time_calls(both, steps, warmup, stream)
    del sets, wd
    torch.cuda.empty_cache()
    return ms_deq, ms_both, wb


def bench_mx(mode, M, steps, warmup, stream, dev, no_nan_codes=False, what="matmul"):
    """Microscaled W[14336, 4096] (mode 1 mxfp4, 2 mxfp8, 3 nvfp4): seeded
    uniform random codes (mxfp8: optionally without the 0x7F / 0xFF codes) and
    scale bytes (E8M0 118..133; nvfp4 E4M3 0x20..0x5F), x bf16 [M, 4096].
    Returns (ms, weight bytes)."""
    import torch
    import weight_only_quantized_qgemv_amd as qp
    from weight_only_quantized_qgemv_amd import synth
    N, K = 14336, 4096
    bits, gs = qp.MX_LAYOUT[mode]
    wb = N * K * bits // 8 + N * (K // gs)
    copies = copies_for(wb)
    gen = torch.Generator(device=dev)
    gen.manual_seed(61 + mode)
    sets = []
    for _ in range(copies):
        codes = torch.randint(0, 256, (N, K * bits // 8), dtype=torch.uint8, device=dev,
                              generator=gen)
        if no_nan_codes:
            codes[(codes & 0x7F) == 0x7F] -= 1          # 0x7F -> 0x7E, 0xFF -> 0xFE
        lo, hi = (0x20, 0x5F) if mode == qp.NVFP4 else (118, 133)
        sb = torch.randint(lo, hi + 1, (N, K // gs), dtype=torch.uint8, device=dev,
                           generator=gen)
        sets.append((codes.view(torch.int32), sb))
    x = torch.from_numpy(synth.normal_f32((M, K), 1.0, 62)).to(torch.bfloat16).to(dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    w = torch.empty((N, K), dtype=torch.bfloat16, device=dev)

    def step(i):
        wq, sb = sets[i % copies]
        if what == "dequantize":
            qp.qpack_dequantize_mx(wq, sb, mode, out=w)
        else:
            qp.qmatmul_mx(x, wq, sb, mode, out=y)

    ms = time_calls(step, steps, warmup, stream)
    del sets
    torch.cuda.empty_cache()
    return ms, wb


def moe_id_sets(T, top_k, E):
    """Expert-id sets the MoE rows cycle through. One token touches only top_k
    experts, so at T = 1 the calls walk a seeded permutation of all E experts
    in disjoint sets of top_k (with two weight sets, every expert's weights of
    both sets pass once per cycle: far more than the Infinity Cache holds).
    Larger T touch nearly every expert per call and keep one id set."""
    import numpy as np
    from weight_only_quantized_qgemv_amd import synth
    if T == 1:
        perm = synth.rng(57).permutation(E).astype(np.int32)
        return [perm[i:i + top_k] for i in range(0, E - top_k + 1, top_k)]
    return [synth.moe_ids(T, top_k, E, seed=55).ravel()]


def bench_moe(T, steps, warmup, stream, dev):
    """Gate+up+SiLU then down of a 128-expert top-8 MoE block (d = 2048,
    ffn = 768), 4-bit gs64 bf16; two weight sets alternate, and at T = 1 the
    expert ids cycle through disjoint sets (moe_id_sets)."""
    import numpy as np
    import torch
    import weight_only_quantized_qgemv_amd as qp
    from weight_only_quantized_qgemv_amd import synth
    E, top_k, D, F, bits, gs = 128, 8, 2048, 768, 4, 64
    wsets = []
    for c in range(2):
        g = [t.reshape(E, F, -1) for t in make_weights(E * F, D, bits, gs, torch.bfloat16, 1,
                                                       51 + 10 * c, dev)[0]]
        u = [t.reshape(E, F, -1) for t in make_weights(E * F, D, bits, gs, torch.bfloat16, 1,
                                                       52 + 10 * c, dev)[0]]
        d = [t.reshape(E, D, -1) for t in make_weights(E * D, F, bits, gs, torch.bfloat16, 1,
                                                       53 + 10 * c, dev)[0]]
        wsets.append((g, u, d))
    id_sets = moe_id_sets(T, top_k, E)
    ids_d = [torch.from_numpy(i).to(dev) for i in id_sets]
    n_ids = len(ids_d)
    a = torch.from_numpy(synth.normal_f32((T, D), 1.0, 54)).to(torch.bfloat16).to(dev)
    P = T * top_k
    h = torch.empty((P, F), dtype=torch.bfloat16, device=dev)
    o = torch.empty((P, D), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(qp.qgemv_moe_workspace_bytes(P, E), dtype=torch.uint8, device=dev)

    def pick(i):
        return wsets[i % 2], ids_d[(i // 2) % n_ids]

    def gate_up(i):
        (g, u, _), ids = pick(i)
        qp.qgemv_moe_id_gate_up_silu(a, ids, T, top_k, D, 0, g, u, bits, gs, out=h, workspace=ws)

    def down(i):
        (_, _, d), ids = pick(i)
        qp.qgemv_moe_id(h, ids, T, top_k, top_k * F, F, *d, bits, gs, out=o, workspace=ws)

    rw = torch.from_numpy(synth.normal_f32((P,), 0.4, 56)).to(dev)
    out = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
    ffn_ws = torch.empty(qp.qgemv_moe_ffn_workspace_bytes(T, top_k, E, D, F, torch.bfloat16),
                         dtype=torch.uint8, device=dev)

    def ffn(i):
        (g, u, d), ids = pick(i)
        qp.qgemv_moe_ffn(a, ids, rw, top_k, g, u, d, bits, gs, out=out, workspace=ffn_ws)

    ms_gu = time_calls(gate_up, steps, warmup, stream)
    ms_d = time_calls(down, steps, warmup, stream)
    ms_ffn = time_calls(ffn, steps, warmup, stream)
    graph = {"gate_up_silu_us_graph": graph_ms(gate_up, max(40, 2 * n_ids), stream),
             "down_us_graph": graph_ms(down, max(40, 2 * n_ids), stream),
             "ffn_block_us_graph": graph_ms(ffn, max(40, 2 * n_ids), stream)}
    touched = int(np.mean([len(np.unique(i)) for i in id_sets]))
    per_expert = weight_bytes(F, D, bits, gs, 2)   # one [768, 2048] matrix
    rotation = 2 * len({int(e) for i in id_sets for e in np.unique(i)}) * 3 * per_expert
    del wsets
    torch.cuda.empty_cache()
    return ms_gu, ms_d, ms_ffn, touched, per_expert, graph, rotation


def moe_call_bytes(T, touched, per_expert, top_k=8, D=2048, F=768, E=128):
    """Bytes one MoE call moves at the least: the touched experts' weights, the
    activations read, the outputs written, the ids, and the routing tables
    (pair list and tile descriptors written, then read back)."""
    P = T * top_k
    route = 2 * (4 * P + 12 * (P + E))
    gate_up = 2 * touched * per_expert + T * D * 2 + P * F * 2 + 4 * P + route
    down = touched * per_expert + P * F * 2 + P * D * 2 + 4 * P + route
    # The block: gate+up, down, then the weighted combine of the P rows into T.
    ffn = 3 * touched * per_expert + T * D * 2 + 2 * P * F * 2 + 2 * P * D * 2 + T * D * 2 + \
        4 * P * 2 + 2 * route
    return gate_up, down, ffn


def cpu_baseline(n, k, bits, gs, budget_s=12.0):
    """The oracle (plain C, OpenMP over outputs) on the headline decode workload:
    whole M=1 calls on the full weight matrix, repeated for about budget_s."""
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
            "sample": f"{runs} whole decode calls (M=1, W[{n},{k}] {bits}-bit gs{gs} bf16 "
                      f"scales/biases), {el:.1f} s wall; dequant + fp64 dot per output, "
                      f"OpenMP over outputs"}


def oracle_single_core():
    """Run in a child process with one OpenMP thread: the oracle on the small
    dense workload (W[256,1024], M = 1 and 8), one headline decode call
    (W[14336,4096], M = 1), one MoE T = 1 call (gate+up+SiLU then down over
    8 of 128 experts), and the quantizer on the headline weight."""
    import numpy as np
    from oracle import qref
    from weight_only_quantized_qgemv_amd import synth

    def timed(fn, min_s=0.5):
        runs, t0 = 0, time.perf_counter()
        while True:
            fn()
            runs += 1
            el = time.perf_counter() - t0
            if el >= min_s:
                return el / runs

    out = {"cores": qref.num_threads()}
    w1 = synth.normal_f32((256, 1024), 0.02, 11)
    q1 = qref.quantize(w1, 4, 64, qref.F32)
    for m in (1, 8):
        x = synth.normal_f32((m, 1024), 1.0, 12)
        out[f"tiny_256x1024_m{m}_ms"] = round(1e3 * timed(lambda: qref.qmatmul(x, qref.F32, *q1, qref.F32,
                                                                                 1024, 4, 64)), 4)
    w2 = synth.normal_f32((14336, 4096), 0.02, 21)
    t0 = time.perf_counter()
    q2 = qref.quantize(w2, 4, 64, qref.BF16)
    out["quantize_14336x4096_b4_ms"] = round(1e3 * (time.perf_counter() - t0), 1)
    xb = synth.normal_f32((1, 4096), 1.0, 22)
    xs = np.frombuffer(np.float32(xb).tobytes(), np.uint32).reshape(1, 4096)
    xs = (xs >> 16).astype(np.uint16)   # bf16 bit patterns (truncated: timing only)
    t0 = time.perf_counter()
    qref.qmatmul(xs, qref.BF16, *q2, qref.BF16, 4096, 4, 64)
    el = time.perf_counter() - t0
    out["decode_14336x4096_m1_ms"] = round(1e3 * el, 1)
    out["decode_14336x4096_m1_weight_GBps"] = round(weight_bytes(14336, 4096, 4, 64, 2) / el / 1e9, 3)
    del w2, q2
    E, top_k, D, F = 128, 8, 2048, 768
    wg = qref.quantize(synth.normal_f32((E * F, D), 0.02, 51), 4, 64, qref.BF16)
    wu = qref.quantize(synth.normal_f32((E * F, D), 0.02, 52), 4, 64, qref.BF16)
    wd = qref.quantize(synth.normal_f32((E * D, F), 0.02, 53), 4, 64, qref.BF16)
    ids = synth.moe_ids(1, top_k, E, seed=55).ravel()
    a = (np.frombuffer(synth.normal_f32((1, D), 1.0, 54).tobytes(), np.uint32) >> 16).astype(np.uint16)
    rs = lambda t, r: tuple(v.reshape(E, r, -1) for v in t)
    t0 = time.perf_counter()
    ref = qref.moe_gate_up_silu(a, qref.BF16, ids, 1, top_k, D, 0, rs(wg, F), rs(wu, F), qref.BF16,
                                E, F, D, 4, 64)
    hb = (np.frombuffer(np.float32(ref["silu_out"]).tobytes(), np.uint32) >> 16).astype(np.uint16)
    qref.moe(hb.reshape(top_k, F), qref.BF16, ids, 1, top_k, top_k * F, F, *rs(wd, D), qref.BF16,
             E, D, F, 4, 64)
    out["moe_t1_gate_up_down_ms"] = round(1e3 * (time.perf_counter() - t0), 1)
    return out


def copy_calibration():
    """Plain device copies of a known size: the reference that scales the
    FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    dev = torch.device("cuda:0")
    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "launches": 5}), flush=True)


# One workload at a time, for profiler runs (counters per kernel):
#   python bench.py --case NAME --steps 20 --warmup 2
CASES = {
    "decode_b4_m1": (14336, 4096, 1, 4, 64, "bf16"),
    "skinny_b4_m16": (14336, 4096, 16, 4, 64, "bf16"),
    "skinny_b3_m8": (4096, 4096, 8, 3, 64, "f16"),
    "rows_b3_m1": (4096, 4096, 1, 3, 64, "f16"),
    "prefill_b4_m2048": (14336, 4096, 2048, 4, 64, "bf16"),
    "prefill_b4_m2048_k14336": (4096, 14336, 2048, 4, 64, "bf16"),
    "moe_t1": 1,
    "moe_t64": 64,
    "moe_t512": 512,
}


def run_case(name, steps, warmup):
    import torch
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    spec = CASES[name]
    if isinstance(spec, int):
        ms_gu, ms_d, ms_ffn, touched, per_expert, _, rotation = bench_moe(spec, steps, warmup,
                                                                           stream, dev)
        print(json.dumps({"case": name, "gate_up_silu_us": round(ms_gu * 1e3, 3),
                          "down_us": round(ms_d * 1e3, 3), "ffn_block_us": round(ms_ffn * 1e3, 3),
                          "experts_touched": touched, "rotation_bytes": rotation}), flush=True)
        return
    N, K, M, bits, gs, dt = spec
    dt = torch.bfloat16 if dt == "bf16" else torch.float16
    ms, wb, copies = bench_dense(N, K, M, bits, gs, dt, steps, warmup, stream, dev)
    print(json.dumps({"case": name, "us": round(ms * 1e3, 3), "weight_bytes": wb,
                      "weight_GBps": round(wb / (ms * 1e-3) / 1e9, 1), "copies": copies}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rows", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--case", choices=sorted(CASES), help="time one workload (for profiler runs)")
    ap.add_argument("--oracle-single-core", action="store_true", help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.oracle_single_core:
        print(json.dumps(oracle_single_core()), flush=True)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: there is no multi-GPU path in this library "
              "(see the sharding design); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.case:
        run_case(args.case, args.steps, args.warmup)
        return

    import torch
    import weight_only_quantized_qgemv_amd as qp
    from weight_only_quantized_qgemv_amd.synth import normal_f32 as synth_normal

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    bf16 = torch.bfloat16
    N, K, BITS, GS = 14336, 4096, 4, 64
    # The timed K steps: eager calls, back to back, rotating over the weight
    # copies. Beside them, the same calls (at least 136 of them, so that the
    # graph's own start-up is spread thin) captured once into a HIP graph and
    # replayed (no launch API between the kernels).
    (ms, ms_graph), wb, copies = bench_dense(N, K, 1, BITS, GS, bf16, args.steps, args.warmup,
                                             stream, dev, graph=True,
                                             graph_calls=max(args.steps, 136))
    gbs = wb / (ms * 1e-3) / 1e9
    traffic = None
    if TRAFFIC is not None and TRAFFIC.get("src_sha") == decode_src_sha():
        traffic = TRAFFIC["fetch_bytes"] + TRAFFIC["write_bytes"]
    result = {
        "metric": "4-bit gs64 qGEMV weight GB/s (decode W[14336,4096], M=1)",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "ms_per_step_graph": round(ms_graph, 6),
        "value_graph": round(wb / (ms_graph * 1e-3) / 1e9, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,0.02) fp32 weights quantized on the device, "
                "N(0,1) bf16 activations",
        "config": {"workload": "decode qGEMV W[14336,4096] 4-bit gs64, bf16 scales/biases, "
                               "x bf16 [1,4096], fp32 accumulation",
                   "weight_bytes_per_call": wb, "weight_copies": copies,
                   "rotation_bytes": wb * copies},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "qgemv_rowstream_kernel<BITS=4, bf16, MT=1, UPL=2, WPB=4, WIDE=true, KL=64>",
                     "us_per_launch": round(ms * 1e3, 3),
                     "algorithmic_bytes_per_launch": wb},
    }
    del_steps = max(20, args.steps // 4)

    if not args.no_rows:
        rows = {}
        # Decode rows: W[14336,4096] gs64 bf16 at 4/8/2 bits, M = 1/4/16.
        # Eager back-to-back calls, and the same calls replayed from a graph.
        for bits in (4, 8, 2):
            for M in (1, 4, 16):
                (ms_r, ms_g), wb_r, _ = bench_dense(N, K, M, bits, 64, bf16, del_steps, 5, stream,
                                                    dev, graph=True)
                g = wb_r / (ms_r * 1e-3) / 1e9
                rows[f"decode_b{bits}_m{M}"] = {
                    "us": round(ms_r * 1e3, 3), "weight_GBps": round(g, 1),
                    "frac_hbm": round(g / HBM_PEAK_GBS, 4),
                    "tokens_per_s": round(M / (ms_r * 1e-3), 1),
                    "us_graph": round(ms_g * 1e3, 3),
                    "weight_GBps_graph": round(wb_r / (ms_g * 1e-3) / 1e9, 1)}
        # The down-projection shape, W[4096,14336], 4-bit gs64 bf16, M = 1.
        (ms_r, ms_g), wb_r, _ = bench_dense(4096, 14336, 1, 4, 64, bf16, del_steps, 5, stream, dev,
                                            seed=23, graph=True)
        g = wb_r / (ms_r * 1e-3) / 1e9
        rows["decode_b4_k14336_m1"] = {"us": round(ms_r * 1e3, 3), "weight_GBps": round(g, 1),
                                       "frac_hbm": round(g / HBM_PEAK_GBS, 4),
                                       "us_graph": round(ms_g * 1e3, 3),
                                       "weight_GBps_graph": round(wb_r / (ms_g * 1e-3) / 1e9, 1)}
        # Launch floor and the streaming rate: the 4-bit row kernel over N rows
        # of K = 4096 (graph-replayed), from a 256-row matrix (about the fixed
        # cost of one launch) to 114688 rows (264 MB).
        sweep = {}
        for n_s in (256, 4096, 14336, 57344, 114688):
            (_, ms_g), wb_s, _ = bench_dense(n_s, K, 1, 4, 64, bf16, 20, 3, stream, dev, seed=25,
                                             graph=True, graph_calls=400)
            sweep[str(n_s)] = {"us_graph": round(ms_g * 1e3, 3),
                               "weight_GBps": round(wb_s / (ms_g * 1e-3) / 1e9, 1)}
        rows["decode_b4_rows_sweep"] = sweep
        # Cross-word rows: W[4096,4096] fp16 at 3/6 bits over gs 32/64/128, M = 1/8.
        for bits in (3, 6):
            for gs in (32, 64, 128):
                for M in (1, 8):
                    (ms_r, ms_g), wb_r, _ = bench_dense(4096, 4096, M, bits, gs, torch.float16,
                                                        del_steps, 5, stream, dev, seed=31,
                                                        graph=True)
                    g = wb_r / (ms_r * 1e-3) / 1e9
                    rows[f"crossword_b{bits}_gs{gs}_m{M}"] = {
                        "us": round(ms_r * 1e3, 3), "weight_GBps": round(g, 1),
                        "frac_hbm": round(g / HBM_PEAK_GBS, 4),
                        "us_graph": round(ms_g * 1e3, 3),
                        "weight_GBps_graph": round(wb_r / (ms_g * 1e-3) / 1e9, 1)}
        # Prefill rows: x bf16 [2048, K] against the two MLP shapes.
        for (n, k) in ((14336, 4096), (4096, 14336)):
            ms_r, _, _ = bench_dense(n, k, 2048, 4, 64, bf16, 20, 3, stream, dev, seed=41)
            tf = 2.0 * 2048 * n * k / (ms_r * 1e-3) / 1e12
            key = f"prefill_m2048_n{n}_k{k}"
            rows[key] = {
                "us": round(ms_r * 1e3, 2), "tflops": round(tf, 1),
                "frac_bf16_mfma": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                "tokens_per_s": round(2048 / (ms_r * 1e-3), 1)}
            clk = PROFILED_CLOCK_GHZ.get(key)
            if clk:
                rows[key]["profiled_clock_ghz"] = clk
                rows[key]["frac_bf16_mfma_at_profiled_clock"] = round(
                    tf / (MFMA_BF16_PEAK_TFLOPS * clk / NOMINAL_CLOCK_GHZ), 4)
        # Unfused rows: dequantize to a dense bf16 weight, then torch.matmul, on
        # the decode and prefill shapes, beside the fused call measured above.
        for M, fused_key in ((1, "decode_b4_m1"), (2048, "prefill_m2048_n14336_k4096")):
            st = del_steps if M == 1 else 20
            ms_deq, ms_both, wb_r = bench_unfused(N, K, M, 4, 64, bf16, st, 3, stream, dev)
            fused_us = rows[fused_key]["us"]
            rows[f"unfused_b4_m{M}"] = {
                "dequantize_us": round(ms_deq * 1e3, 3),
                "dequantize_GBps": round((wb_r + N * K * 2) / (ms_deq * 1e-3) / 1e9, 1),
                "dequantize_then_matmul_us": round(ms_both * 1e3, 3),
                "fused_us": fused_us,
                "fused_speedup": round(ms_both * 1e3 / fused_us, 2)}
        # Microscaled rows: decode M = 1, prefill M = 2048, dense weight.
        for mode, name in ((1, "mxfp4"), (3, "nvfp4"), (2, "mxfp8")):
            for variant in ((False, True) if mode == 2 else (False,)):
                tag = name + ("_no480" if variant else "")
                ms_r, wb_r = bench_mx(mode, 1, del_steps, 5, stream, dev, no_nan_codes=variant)
                g = wb_r / (ms_r * 1e-3) / 1e9
                rows[f"mx_decode_{tag}_m1"] = {"us": round(ms_r * 1e3, 3), "weight_GBps": round(g, 1),
                                               "frac_hbm": round(g / HBM_PEAK_GBS, 4)}
                ms_r, _ = bench_mx(mode, 2048, 20, 3, stream, dev, no_nan_codes=variant)
                tf = 2.0 * 2048 * N * K / (ms_r * 1e-3) / 1e12
                rows[f"mx_prefill_{tag}_m2048"] = {
                    "us": round(ms_r * 1e3, 2), "tflops": round(tf, 1),
                    "frac_bf16_mfma": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}
            ms_r, wb_r = bench_mx(mode, 1, 50, 5, stream, dev, what="dequantize")
            moved = wb_r + N * K * 2
            rows[f"mx_dequantize_{name}"] = {
                "us": round(ms_r * 1e3, 3), "GBps": round(moved / (ms_r * 1e-3) / 1e9, 1),
                "frac_hbm": round(moved / (ms_r * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        # Per-tensor dynamic-range int8 W[14336, 4096], seeded random codes.
        gen = torch.Generator(device=dev)
        gen.manual_seed(71)
        wb_i8 = N * K
        i8_copies = copies_for(wb_i8)
        i8_sets = [torch.randint(-128, 128, (N, K), dtype=torch.int8, device=dev, generator=gen)
                   for _ in range(i8_copies)]
        i8_rng = torch.tensor([-0.1, 0.1], dtype=torch.float32, device=dev)
        for M in (1, 2):
            x_i8 = torch.from_numpy(synth_normal((M, K), 1.0, 72)).to(bf16).to(dev)
            y_i8 = torch.empty((M, N), dtype=bf16, device=dev)
            ms_r = time_calls(lambda i: qp.qmatmul_int8_tensor(x_i8, i8_sets[i % i8_copies], i8_rng,
                                                               out=y_i8), del_steps, 5, stream)
            g = wb_i8 / (ms_r * 1e-3) / 1e9
            rows[f"int8_tensor_decode_m{M}"] = {"us": round(ms_r * 1e3, 3), "weight_GBps": round(g, 1),
                                                "frac_hbm": round(g / HBM_PEAK_GBS, 4)}
        del i8_sets
        torch.cuda.empty_cache()
        # transpose = false: W [4096, 14336] stored [k, n], 4-bit gs64 bf16, M = 1.
        wb_t = weight_bytes(K, N, 4, 64, 2)
        t_copies = copies_for(wb_t)
        t_sets = make_weights(K, N, 4, 64, bf16, t_copies, 81, dev)
        x_t = torch.from_numpy(synth_normal((1, K), 1.0, 82)).to(bf16).to(dev)
        y_t = torch.empty((1, N), dtype=bf16, device=dev)
        ws_t = torch.empty(qp.qmatmul_t_workspace_bytes(1, K, N, 4), dtype=torch.uint8, device=dev)
        ms_r = time_calls(lambda i: qp.qmatmul_t(x_t, *t_sets[i % t_copies], 4, 64, out=y_t,
                                                 workspace=ws_t), del_steps, 5, stream)
        g = wb_t / (ms_r * 1e-3) / 1e9
        rows["transpose_false_b4_m1"] = {"us": round(ms_r * 1e3, 3), "weight_GBps": round(g, 1),
                                         "frac_hbm": round(g / HBM_PEAK_GBS, 4)}
        del t_sets
        torch.cuda.empty_cache()
        # MoE rows: 128 experts, top-8, 4-bit gs64 bf16.
        for T in (1, 64, 512):
            ms_gu, ms_d, ms_ffn, touched, per_expert, graph, rotation = bench_moe(
                T, del_steps, 5, stream, dev)
            gu_bytes, d_bytes = 2 * touched * per_expert, touched * per_expert
            gu_all, d_all, ffn_all = moe_call_bytes(T, touched, per_expert)
            rows[f"moe_t{T}"] = {
                "experts_touched": touched,
                "rotation_bytes": rotation,
                "gate_up_silu_us": round(ms_gu * 1e3, 3),
                "gate_up_weight_GBps": round(gu_bytes / (ms_gu * 1e-3) / 1e9, 1),
                "gate_up_total_bytes": gu_all,
                "gate_up_total_GBps": round(gu_all / (ms_gu * 1e-3) / 1e9, 1),
                "down_us": round(ms_d * 1e3, 3),
                "down_weight_GBps": round(d_bytes / (ms_d * 1e-3) / 1e9, 1),
                "down_total_bytes": d_all,
                "down_total_GBps": round(d_all / (ms_d * 1e-3) / 1e9, 1),
                "tflops_total": round(2.0 * T * 8 * 3 * 768 * 2048 / ((ms_gu + ms_d) * 1e-3)
                                      / 1e12, 2),
                "ffn_block_us": round(ms_ffn * 1e3, 3),
                "ffn_block_weight_GBps": round(3 * touched * per_expert / (ms_ffn * 1e-3) / 1e9, 1),
                "ffn_block_total_bytes": ffn_all,
                "ffn_block_total_GBps": round(ffn_all / (ms_ffn * 1e-3) / 1e9, 1),
                "tokens_per_s": {"gate_up_silu": round(T / (ms_gu * 1e-3), 1),
                                 "down": round(T / (ms_d * 1e-3), 1),
                                 "ffn_block": round(T / (ms_ffn * 1e-3), 1)},
                **{k: round(v * 1e3, 3) for k, v in graph.items()}}
        result["rows"] = rows

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(N, K, BITS, GS)
        import subprocess
        env = dict(os.environ, OMP_NUM_THREADS="1")
        p = subprocess.run([sys.executable, os.path.abspath(__file__), "--oracle-single-core"],
                           capture_output=True, text=True, env=env, timeout=600)
        if p.returncode == 0:
            result["cpu_baseline"]["single_core"] = json.loads(p.stdout.strip().splitlines()[-1])
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
