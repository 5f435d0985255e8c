#!/usr/bin/env python3
"""Throughput of the W4 hot path on one MI355X.

Default workload: the decode GEMV layer (K = N = 8192) at M = 1, 4 and 16
tokens, with INT4 asymmetric (group 128, fp16 scale + zero) and NF4 (block
64, fp16 absmax) weights.  One step = those six products, each on the next
weight set of a rotation that spans more than 512 MB, so the 256 MB
Infinity Cache cannot serve repeats.  The timed region replays a HIP graph
of whole steps (the kernels are shorter than a host launch), with all inputs
resident in HBM.

Prints one JSON line.  Other workloads (``--workload``) are for measurement
runs; the default line is the one reported.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0         # MI355X HBM3E, published
FP16_MFMA_PEAK_TFLOPS = 2500.0  # dense fp16 matrix cores, published
INT8_MFMA_PEAK_TOPS = 5000.0    # dense int8 matrix cores, published


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=512)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--workload", default="decode_gemv", choices=["decode_gemv"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel-reps", type=int, default=64,
                    help="eager launches per variant for the live per-kernel timing")
    ap.add_argument("--gemm-reps", type=int, default=20,
                    help="timed launches per prefill GEMM path (0 skips the GEMM section)")
    return ap.parse_args()


def weight_stream_bytes(fmt, K, N, G):
    packed = N * K // 2
    scales = N * (K // G) * 2
    zeros = N * (K // G) * 2 if fmt == 0 else 0
    return packed + scales + zeros


def make_weight_sets(w4, torch, fmt, K, N, G, count, seed0):
    """Seeded N(0, 0.02^2) fp32 weights drawn on the GPU, quantized and packed
    by the library; only the packed form is kept."""
    sets = []
    gen = torch.Generator(device="cuda")
    for i in range(count):
        gen.manual_seed(seed0 + i)
        w = torch.randn((N, K), generator=gen, device="cuda", dtype=torch.float32) * 0.02
        codes, scale, zero = w4.quantize(w, G, fmt)
        packed = w4.pack(codes)
        del w, codes
        sets.append((packed, scale, zero))
    torch.cuda.synchronize()
    return sets


def cpu_baseline_decode(variants, K, N, n_rows, min_seconds=10.0):
    """The fp64 oracle (dequantize, then matmul) on a row sample of each
    variant's weights, repeated until about `min_seconds` of CPU work;
    returns (GB/s of weight stream, seconds, threads, repetitions)."""
    import oracle as o
    import workloads as wl
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover - informational only
        threads = 1
    total_bytes = 0
    total_s = 0.0
    w = wl.make_weight(2, 0, n_rows, K)
    prepared = {}
    for fmt, G in {(v[0], v[2]) for v in variants}:
        if fmt == 0:
            prepared[(fmt, G)] = o.quantize_int4_asym(w, G)
        else:
            c, a = o.quantize_nf4(w, G)
            prepared[(fmt, G)] = (c, a, None)
    xs = {M: wl.make_activations(2, 0, M, K) for _, M, _ in variants}
    reps = 0
    while total_s < min_seconds:
        for fmt, M, G in variants:
            codes, scale, zero = prepared[(fmt, G)]
            t0 = time.perf_counter()
            y = o.matmul_ref(xs[M], o.dequant(fmt, codes, scale, zero, G))
            total_s += time.perf_counter() - t0
            assert y.shape == (M, n_rows)
            total_bytes += weight_stream_bytes(fmt, K, n_rows, G)
        reps += 1
    return total_bytes / total_s / 1e9, total_s, threads, reps


def bench_gemm_prefill(w4, torch, reps):
    """Prefill product M = 2048, K = 5120, N = 25600, INT4 g128, three ways:
    dequantize-to-fp16 MFMA, post-scaled fp16 MFMA, and the two-slice
    Multi-Scale Dequant int8 MFMA (its activation decomposition included).
    Back-to-back launches between HIP events on the launch stream."""
    import workloads as wl
    M, K, N, G = 2048, 5120, 25600, 128
    gen = torch.Generator(device="cuda")
    gen.manual_seed(40000)
    w = torch.randn((N, K), generator=gen, device="cuda", dtype=torch.float32) * 0.02
    codes, scale, zero = w4.quantize(w, G, w4.INT4_ASYM)
    packed = w4.pack(codes)
    del w, codes
    x = torch.from_numpy(wl.make_activations(4, 0, M, K)).cuda()
    y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    ws = torch.empty(w4.workspace_bytes(w4.OP_GEMM_DECOMP, M, K, N, G, 2), dtype=torch.uint8, device="cuda")
    flops = 2.0 * M * N * K
    paths = {
        "dq_f16": (lambda: w4.gemm(x, packed, scale, zero, G, w4.INT4_ASYM, w4.DQ_F16, out=y), 1, FP16_MFMA_PEAK_TFLOPS),
        "postscale": (lambda: w4.gemm(x, packed, scale, zero, G, w4.INT4_ASYM, w4.POSTSCALE, out=y), 1,
                      FP16_MFMA_PEAK_TFLOPS),
        "msd2": (lambda: w4.gemm_decomp(x, packed, scale, zero, G, 2, out=y, workspace=ws), 2, INT8_MFMA_PEAK_TOPS),
    }
    res = {}
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        for name, (fn, mfma_mult, peak) in paths.items():
            for _ in range(3):
                fn()
            st.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(st)
            for _ in range(reps):
                fn()
            b.record(st)
            st.synchronize()
            us = a.elapsed_time(b) * 1e3 / reps
            mfma_rate = flops * mfma_mult / (us * 1e-6) / 1e12
            res[name] = {"us_per_call": round(us, 1), "tflops_useful": round(flops / (us * 1e-6) / 1e12, 1),
                         "mfma_tops": round(mfma_rate, 1), "mfma_peak": peak,
                         "frac": round(mfma_rate / peak, 4)}
    return {"workload": "prefill_gemm_m2048_k5120_n25600", "M": M, "K": K, "N": N, "fmt": "int4_asym_g128",
            "flops_per_call": flops, "calls_timed": reps,
            "note": "fp16 paths against the dense fp16 MFMA peak; msd2 issues 2 int8 products per useful "
                    "multiply-add and is measured against the dense int8 peak; msd2 time includes the "
                    "activation decomposition",
            "paths": res}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); every box here has one GPU "
              "and this library has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_weight_quantized_amd as w4
    import workloads as wl

    torch.cuda.set_device(0)
    K = N = 8192
    Ms = (1, 4, 16)
    fmts = ((w4.INT4_ASYM, 128), (w4.NF4, 64))
    variants = [(fmt, M, G) for fmt, G in fmts for M in Ms]
    per_set = weight_stream_bytes(0, K, N, 128)
    n_sets = max(2, -(-(2 * 256 * 2 ** 20) // per_set) + 1)  # > 512 MB per format

    sets = {fmt: make_weight_sets(w4, torch, fmt, K, N, G, n_sets, 20000 + 1000 * fmt) for fmt, G in fmts}
    xs = {M: torch.from_numpy(wl.make_activations(2, 0, M, K)).cuda() for M in Ms}
    ys = {M: torch.empty((M, N), dtype=torch.float16, device="cuda") for M in Ms}
    # zero-filled once; every call leaves its workspace zero again (no memset in the graph)
    wss = {(fmt, M): torch.zeros(max(16, w4.workspace_bytes(w4.OP_GEMV, M, K, N, G, fmt)), dtype=torch.uint8,
                                 device="cuda") for fmt, M, G in variants}

    def step(i):
        for fmt, M, G in variants:
            packed, scale, zero = sets[fmt][(i * len(Ms) + Ms.index(M)) % n_sets]
            w4.gemv(xs[M], packed, scale, zero, G, fmt, out=ys[M], workspace=wss[(fmt, M)])

    # ---- capture one rotation of steps in a graph
    stream = torch.cuda.Stream()
    steps_per_graph = n_sets
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for i in range(2):  # eager warm-up on the capture stream (also loads code objects)
            step(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for i in range(steps_per_graph):
            step(i)
    torch.cuda.synchronize()

    replays_warm = max(1, -(-args.warmup // steps_per_graph))
    replays = max(1, -(-args.steps // steps_per_graph))
    steps_timed = replays * steps_per_graph
    for _ in range(replays_warm):
        graph.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(replays):
        graph.replay()
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / steps_timed
    step_bytes = sum(weight_stream_bytes(fmt, K, N, G) for fmt, M, G in variants)
    value = step_bytes * steps_timed / (total_ms * 1e-3) / 1e9

    # ---- live per-kernel timing: HIP events around eager launches queued
    # behind a spin kernel, on the stream the kernels run on
    per = []
    kstream = torch.cuda.Stream()
    with torch.cuda.stream(kstream):
        for fmt, M, G in variants:
            reps = args.kernel_reps
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
            torch.cuda._sleep(50_000_000)
            for r in range(reps):
                packed, scale, zero = sets[fmt][r % n_sets]
                evs[r][0].record(kstream)
                w4.gemv(xs[M], packed, scale, zero, G, fmt, out=ys[M], workspace=wss[(fmt, M)])
                evs[r][1].record(kstream)
            torch.cuda.synchronize()
            durs = sorted(a.elapsed_time(b) * 1e3 for a, b in evs[2:])  # us
            avg = float(np.mean(durs))
            b = weight_stream_bytes(fmt, K, N, G)
            per.append({"fmt": "int4_g128" if fmt == 0 else "nf4_b64", "M": M, "us_avg": round(avg, 3),
                        "us_median": round(durs[len(durs) // 2], 3), "weight_bytes": b,
                        "GBps": round(b / (avg * 1e-6) / 1e9, 1)})
    sum_bytes = sum(p["weight_bytes"] for p in per)
    sum_us = sum(p["us_avg"] for p in per)
    achieved = sum_bytes / (sum_us * 1e-6) / 1e9

    gemm = bench_gemm_prefill(w4, torch, args.gemm_reps) if args.gemm_reps > 0 else None

    cpu = None
    if not args.no_cpu_baseline:
        gbs, secs, threads, reps = cpu_baseline_decode(variants, K, N, n_rows=2048)
        cpu = {"value": round(gbs, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
               "sample": f"fp64 dequantize + matmul of 2048 of the 8192 weight rows, all 6 variants, "
                         f"{reps} passes ({secs:.1f} s of CPU time)"}

    out = {
        "metric": "W4 GEMV weight-stream GB/s (decode layer K=N=8192, M in {1,4,16}, INT4 g128 + NF4 b64)",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps_timed,
        "warmup": replays_warm * steps_per_graph,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic: weights N(0,0.02^2) fp32 quantized on the GPU, activations N(0,1) fp16 with 1%% x20 "
                "outlier channels; weights rotate over %d sets per format (%.0f MB)" % (n_sets, n_sets * per_set / 1e6),
        "config": {"workload": "decode_gemv_k8192_n8192", "M": list(Ms), "K": K, "N": N,
                   "formats": ["int4_asym_g128", "nf4_b64"], "launches_per_step": len(variants),
                   "timed": "HIP graph replays, %d steps per graph" % steps_per_graph},
        "roofline": {"bound": "hbm", "kernel": "gemv_kernel (all 6 launches of a step)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "bytes_per_launch": "packed N*K/2 + fp16 scales (+ zeros) = %d" % per_set},
        "per_launch": per,
        "gemm_prefill": gemm,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
