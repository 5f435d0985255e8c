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
FP4_MFMA_PEAK_TFLOPS = 10100.0  # dense fp4 matrix cores, published


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=512)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--workload", default="decode_gemv", choices=["decode_gemv"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel-replays", type=int, default=4,
                    help="graph replays per variant for the live per-launch timing (each replay launches "
                         "the variant once on every weight set of the rotation)")
    ap.add_argument("--profile-pass", action="store_true",
                    help="instead of the bench: launch each GEMV variant --profile-launches times eagerly, "
                         "then a plain device copy of a known size (the reference for rocprofv3 --pmc "
                         "FETCH_SIZE / WRITE_SIZE); prints what ran")
    ap.add_argument("--profile-launches", type=int, default=16)
    ap.add_argument("--profile-gemm", action="store_true",
                    help="instead of the bench: launch each prefill path (M=2048, K=5120, N=25600) "
                         "--profile-launches times eagerly, for rocprofv3 --pmc counter passes over the "
                         "matrix-core kernels; prints what ran")
    ap.add_argument("--profile-attention", action="store_true",
                    help="instead of the bench: launch the KV-cache attention call --profile-launches times "
                         "eagerly and the plain copy, for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU: from the counter_collection CSVs of two --profile-pass runs (rocprofv3 "
                         "--pmc FETCH_SIZE, then --pmc WRITE_SIZE) print the HBM traffic summary of the GEMV "
                         "variants, calibrated on the plain copy")
    ap.add_argument("--kernels", metavar="REGEX", default=None,
                    help="with --summarize: only kernels whose name matches")
    ap.add_argument("--counters", nargs="+", metavar="CSV",
                    help="no GPU: per-kernel table of the counter_collection CSVs of several rocprofv3 --pmc "
                         "passes over the same command (--profile-gemm or --profile-attention), with the "
                         "derived matrix-core, clock, instruction-mix, LDS and HBM-traffic figures")
    ap.add_argument("--summarize", nargs="+", metavar="CSV",
                    help="no GPU: print a markdown summary of rocprofv3 CSV output (kernel_stats or "
                         "counter_collection files)")
    ap.add_argument("--no-attention", dest="attention", action="store_false",
                    help="skip the KV-cache attention timing")
    ap.add_argument("--no-residual", dest="residual", action="store_false",
                    help="skip the residual-compensation timing")
    ap.add_argument("--no-layers", dest="layers", action="store_false",
                    help="skip the MLP-shaped GEMV and decoder-layer timings")
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
    """Prefill product M = 2048, K = 5120, N = 25600, INT4 g128: dequantize-to-
    fp16 MFMA, post-scaled fp16 MFMA, and the Multi-Scale Dequant int8 MFMA
    with two slices (adaptive and fixed-ratio scales), one and three slices
    (each with its activation decomposition included), and MXFP4 weights with
    one and two MXFP4 slices.  Back-to-back launches between HIP events on the
    launch stream."""
    (M, K, N), paths = prefill_paths(w4, torch)
    flops = 2.0 * M * N * K
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
            "note": "fp16 paths against the dense fp16 MFMA peak; msdJ issues J int8 products per useful "
                    "multiply-add and is measured against the dense int8 peak; msd times include the "
                    "activation decomposition; msd2_fixed uses s2 = s1/254 and combines the two int32 "
                    "products in integers; msd2_fixed_fused computes only s1 in a pre-pass and forms both "
                    "slices inside the product's K loop (same y bits); mxfp4_J: MXFP4 weights (the same distribution, own draw), the "
                    "activations split into J MXFP4 slices, J block-scaled fp4 products per useful "
                    "multiply-add against the dense fp4 peak, decomposition included",
            "paths": res}


def bench_mfma_ceiling(w4, torch, iters=8192):
    """The matrix-core ceiling on this part, measured (w4_mfma_rate): one
    workgroup of 8 waves per CU, each wave issuing iters x 8 independent
    16 x 16 products, fp16 (16x16x32) and int8 (16x16x64); the clock comes
    from the waves' shader-clock and 100 MHz ticks.  The same launch with V
    independent fp32 FMAs per product shows how many VALU instructions run
    beside a product without slowing it (the last V within 3 % of V = 0)."""
    wgs = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(wgs * 512, dtype=torch.float32, device="cuda")
    ticks = torch.zeros(wgs * 16, dtype=torch.int64, device="cuda")
    st = torch.cuda.Stream()
    res = {}
    for kind, name, ops, peak in ((0, "fp16_16x16x32", 16384, FP16_MFMA_PEAK_TFLOPS),
                                  (1, "int8_16x16x64", 32768, INT8_MFMA_PEAK_TOPS)):
        sweep = {}
        clock = None
        with torch.cuda.stream(st):
            for valu in (0, 1, 2, 3, 4, 6, 8):
                w4.mfma_rate(kind, valu, wgs, iters, sink, ticks, stream=st)
                st.synchronize()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(st)
                for _ in range(3):
                    w4.mfma_rate(kind, valu, wgs, iters, sink, ticks, stream=st)
                b.record(st)
                st.synchronize()
                sweep[valu] = a.elapsed_time(b) * 1e3 / 3
                if valu == 0:
                    t = ticks.cpu().double().reshape(-1, 2)
                    clock = float((t[:, 0] / (t[:, 1] / 100e6)).mean() / 1e9)
        rate = wgs * 8 * iters * 8 * ops / (sweep[0] * 1e-6) / 1e12
        free = max(v for v in sweep if sweep[v] <= 1.03 * sweep[0])
        res[name] = {"us_per_launch": round(sweep[0], 1), "rate": round(rate, 1), "peak": peak,
                     "frac_of_peak": round(rate / peak, 4), "clock_ghz": round(clock, 3),
                     "free_valu_per_product": free,
                     "us_by_valu_per_product": {str(v): round(us, 1) for v, us in sweep.items()}}
    return {"workload": "independent matrix-core products, 8 waves per CU", "iters_per_wave": iters * 8,
            "unit": "TFLOP/s (fp16), TOP/s (int8)", "kinds": res}


def bench_library_f16_gemm(torch, reps=10):
    """hipBLASLt's fp16 GEMM (torch.matmul) at the prefill shape, on fp16
    weights: no unpacking, the library's own tiling; a comparison point."""
    M, K, N = 2048, 5120, 25600
    gen = torch.Generator(device="cuda")
    gen.manual_seed(41000)
    x = torch.randn((M, K), generator=gen, device="cuda", dtype=torch.float32).half()
    w = (torch.randn((K, N), generator=gen, device="cuda", dtype=torch.float32) * 0.02).half()
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        for _ in range(3):
            y = torch.matmul(x, w)
        st.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        for _ in range(reps):
            y = torch.matmul(x, w)
        b.record(st)
        st.synchronize()
    del y
    us = a.elapsed_time(b) * 1e3 / reps
    tf = 2.0 * M * N * K / (us * 1e-6) / 1e12
    return {"workload": "fp16 GEMM M=2048 K=5120 N=25600 (torch.matmul, hipBLASLt)", "us_per_call": round(us, 1),
            "tflops": round(tf, 1), "frac": round(tf / FP16_MFMA_PEAK_TFLOPS, 4)}


def prefill_paths(w4, torch):
    """The prefill product M = 2048, K = 5120, N = 25600 (INT4 g128; MXFP4 for
    the mxfp4 paths): a dict of name -> (thunk, MFMA products per useful
    multiply-add, dense peak of that product's type)."""
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
    wmx = torch.randn((N, K), generator=gen, device="cuda", dtype=torch.float32) * 0.02
    mx_codes, mx_scale = w4.quantize_mx(wmx)
    mx_packed = w4.pack_mx(mx_codes)
    del wmx, mx_codes
    ws_mx = torch.empty(max(w4.workspace_bytes(w4.OP_GEMM_MX, M, K, N, 32, ns) for ns in (1, 2)), dtype=torch.uint8,
                        device="cuda")
    ws = torch.empty(max([w4.workspace_bytes(w4.OP_GEMM_DECOMP, M, K, N, G, ns) for ns in (1, 2, 3)] +
                         [w4.workspace_bytes(w4.OP_GEMM_DECOMP_FUSED, M, K, N, G, 0)]),
                     dtype=torch.uint8, device="cuda")
    ws_f16 = torch.empty(max(16, w4.workspace_bytes(w4.OP_GEMM, M, K, N, G, w4.DQ_F16)), dtype=torch.uint8,
                         device="cuda")
    return (M, K, N), {
        "dq_f16": (lambda: w4.gemm(x, packed, scale, zero, G, w4.INT4_ASYM, w4.DQ_F16, out=y, workspace=ws_f16), 1,
                   FP16_MFMA_PEAK_TFLOPS),
        "postscale": (lambda: w4.gemm(x, packed, scale, zero, G, w4.INT4_ASYM, w4.POSTSCALE, out=y,
                                      workspace=ws_f16), 1, FP16_MFMA_PEAK_TFLOPS),
        "msd2": (lambda: w4.gemm_decomp(x, packed, scale, zero, G, 2, out=y, workspace=ws), 2, INT8_MFMA_PEAK_TOPS),
        "msd2_fixed": (lambda: w4.gemm_decomp_fixed(x, packed, scale, zero, G, out=y, workspace=ws), 2,
                       INT8_MFMA_PEAK_TOPS),
        "msd2_fixed_fused": (lambda: w4.gemm_decomp_fixed_fused(x, packed, scale, zero, G, out=y, workspace=ws), 2,
                             INT8_MFMA_PEAK_TOPS),
        "msd1": (lambda: w4.gemm_decomp(x, packed, scale, zero, G, 1, out=y, workspace=ws), 1, INT8_MFMA_PEAK_TOPS),
        "msd3": (lambda: w4.gemm_decomp(x, packed, scale, zero, G, 3, out=y, workspace=ws), 3, INT8_MFMA_PEAK_TOPS),
        "mxfp4_2": (lambda: w4.gemm_mx(x, mx_packed, mx_scale, 2, out=y, workspace=ws_mx), 2, FP4_MFMA_PEAK_TFLOPS),
        "mxfp4_1": (lambda: w4.gemm_mx(x, mx_packed, mx_scale, 1, out=y, workspace=ws_mx), 1, FP4_MFMA_PEAK_TFLOPS),
    }


def rotation_sets(per_set_bytes):
    """Weight sets per rotation: more than 512 MB, twice the Infinity Cache."""
    return max(2, -(-(2 * 256 * 2 ** 20) // per_set_bytes) + 1)


def bench_single_gemv(w4, torch, stream, replays=4):
    """The single small GEMV: M = 1, K = N = 1024, G = 64, INT4 (scale +
    zero) and NF4 (absmax), activations without outliers.  Per launch: a
    HIP graph of one launch per weight set of a > 512 MB rotation (about
    900 sets of 0.59 MB), replayed back to back.  At 0.59 MB per launch the
    HBM time at peak is about 74 ns, so the launch itself bounds it."""
    import workloads as wl
    K = N = 1024
    G = 64
    res = []
    for fmt in (w4.INT4_ASYM, w4.NF4):
        b = weight_stream_bytes(fmt, K, N, G)
        n_sets = rotation_sets(b)
        sets = make_weight_sets(w4, torch, fmt, K, N, G, n_sets, 45000 + 5000 * fmt)
        x = torch.from_numpy(wl.make_activations(1, 0, 1, K, outliers=False)).cuda()
        y = torch.empty((1, N), dtype=torch.float16, device="cuda")
        ws = torch.zeros(max(16, w4.workspace_bytes(w4.OP_GEMV, 1, K, N, G, fmt)), dtype=torch.uint8, device="cuda")
        calls = [lambda p=p: w4.gemv(x, p[0], p[1], p[2], G, fmt, out=y, workspace=ws) for p in sets]
        g = graph_of(torch, stream, calls)
        time_replays(torch, stream, g, 1)
        us = time_replays(torch, stream, g, replays) * 1e3 / (replays * n_sets)
        del g, sets
        torch.cuda.empty_cache()
        gbs = b / (us * 1e-6) / 1e9
        res.append({"variant": ("int4_g64" if fmt == w4.INT4_ASYM else "nf4_b64") + "_m1", "us_per_launch": round(us, 3),
                    "weight_bytes": b, "GBps": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                    "rotation_sets": n_sets})
    return {"workload": "single_gemv_m1_k1024_n1024_g64", "note": "launch-bound: 0.59 MB is about 74 ns of HBM "
            "time at peak", "per_launch": res}


def bench_plain_read(w4, torch, stream, nbytes, replays=4):
    """The HBM read ceiling for one decode-layer weight stream: w4_stream_read
    (16-byte non-temporal loads, every byte once) over buffers of the GEMV's
    35.65 MB, rotating over > 512 MB like the GEMV's weight sets; one launch
    per buffer in a HIP graph replayed back to back."""
    n_sets = rotation_sets(nbytes)
    bufs = [torch.full((nbytes // 4,), i + 1, dtype=torch.int32, device="cuda") for i in range(n_sets)]
    acc = torch.zeros(w4.STREAM_READ_ACC_WORDS, dtype=torch.int32, device="cuda")
    g = graph_of(torch, stream, [lambda b=b: w4.stream_read(b, acc) for b in bufs])
    time_replays(torch, stream, g, 1)
    us = time_replays(torch, stream, g, replays) * 1e3 / (replays * n_sets)
    del g, bufs
    torch.cuda.empty_cache()
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"workload": "plain_read_35651584_bytes", "us_per_launch": round(us, 3), "bytes": nbytes,
            "GBps": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "rotation_sets": n_sets}


def bench_mlp_gemv(w4, torch, stream, replays=4):
    """MLP-shaped decode products, M = 1, 8 and 32: up/gate (K = 8192,
    N = 28672) and down (K = 28672, N = 8192), INT4 g128 and NF4 b64.  Per
    launch: a HIP graph of one launch per weight set of a > 512 MB rotation,
    replayed back to back between events on its stream."""
    import workloads as wl
    shapes = (("up_gate", 8192, 28672), ("down", 28672, 8192))
    res = []
    for si, (name, K, N) in enumerate(shapes):
        for fmt, G in ((w4.INT4_ASYM, 128), (w4.NF4, 64)):
            b = weight_stream_bytes(fmt, K, N, G)
            n_sets = rotation_sets(b)
            sets = make_weight_sets(w4, torch, fmt, K, N, G, n_sets, 50000 + 1000 * si + 100 * fmt)
            for M in (1, 8, 32):
                x = torch.from_numpy(wl.make_activations(3, si, M, K)).cuda()
                y = torch.empty((M, N), dtype=torch.float16, device="cuda")
                ws = torch.zeros(max(16, w4.workspace_bytes(w4.OP_GEMV, M, K, N, G, fmt)), dtype=torch.uint8,
                                 device="cuda")
                calls = [lambda p=p: w4.gemv(x, p[0], p[1], p[2], G, fmt, out=y, workspace=ws) for p in sets]
                g = graph_of(torch, stream, calls)
                time_replays(torch, stream, g, 1)
                us = time_replays(torch, stream, g, replays) * 1e3 / (replays * n_sets)
                res.append({"matrix": name, "K": K, "N": N, "variant": variant_name(fmt, M),
                            "us_per_launch": round(us, 3), "weight_bytes": b,
                            "GBps": round(b / (us * 1e-6) / 1e9, 1),
                            "hbm_frac": round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)})
                del g
            del sets
            torch.cuda.empty_cache()
    return {"workload": "mlp_gemv_up_gate_k8192_n28672_down_k28672_n8192", "rotation": "> 512 MB per variant",
            "per_launch": res}


DECODER_LAYER = (("q", 8192, 8192), ("k", 8192, 1024), ("v", 8192, 1024), ("o", 8192, 8192),
                 ("gate", 8192, 28672), ("up", 8192, 28672), ("down", 28672, 8192))
# The same layer with the products that share an input stored as one matrix
# (q, k, v and gate, up concatenated along N): four products instead of seven.
DECODER_LAYER_FUSED = (("qkv", 8192, 10240, ("q", "k", "v")), ("o", 8192, 8192, ("o",)),
                       ("gate_up", 8192, 57344, ("gate", "up")), ("down", 28672, 8192, ("down",)))


def bench_decoder_layer(w4, torch, stream, replays=4):
    """A 70B-style decoder layer's seven products (q, k, v, o, gate, up,
    down) back to back, at M = 1 (GEMV) and M = 256 (the matrix-core paths),
    INT4 g128 and NF4 b64; two weight sets per format (> 512 MB).  Timed as
    HIP graphs of whole layers replayed between events on their stream."""
    import workloads as wl
    out = []
    flops_256 = sum(2.0 * 256 * K * N for _, K, N in DECODER_LAYER)
    for fmt, G in ((w4.INT4_ASYM, 128), (w4.NF4, 64)):
        layer_bytes = sum(weight_stream_bytes(fmt, K, N, G) for _, K, N in DECODER_LAYER)
        n_sets = rotation_sets(layer_bytes)
        sep = [{name: make_weight_sets(w4, torch, fmt, K, N, G, 1, 60000 + 1000 * s + 10 * i + 100 * fmt)[0]
                for i, (name, K, N) in enumerate(DECODER_LAYER)} for s in range(n_sets)]
        # the fused layer holds the same weights: packed rows, scales and zero
        # points concatenated along N (the packed tiles are stored row block
        # by row block, so the bytes concatenate)
        fused = [{name: tuple(None if sep[s][parts[0]][a] is None else
                              torch.cat([sep[s][pn][a] for pn in parts]) for a in range(3))
                  for name, _, _, parts in DECODER_LAYER_FUSED} for s in range(n_sets)]
        paths = [("gemv", 1)]
        paths += [("dq_f16", 256), ("postscale", 256)]
        if fmt == w4.INT4_ASYM:
            paths += [("msd2", 256), ("msd2_fixed", 256), ("msd2_fixed_fused", 256)]
        for layout, mats, sets in (("separate", DECODER_LAYER, sep),
                                   ("fused", tuple(m[:3] for m in DECODER_LAYER_FUSED), fused)):
            for path, M in paths:
                xs = {K: torch.from_numpy(wl.make_activations(5, 0 if K == 8192 else 6, M, K)).cuda()
                      for K in {K for _, K, _ in mats}}
                ys = {name: torch.empty((M, N), dtype=torch.float16, device="cuda") for name, _, N in mats}
                calls = []
                for s in range(n_sets):
                    for name, K, N in mats:
                        p, sc, z = sets[s][name]
                        x, y = xs[K], ys[name]
                        if path == "gemv":
                            ws = torch.zeros(max(16, w4.workspace_bytes(w4.OP_GEMV, M, K, N, G, fmt)),
                                             dtype=torch.uint8, device="cuda")
                            calls.append(lambda p=p, sc=sc, z=z, x=x, y=y, ws=ws, K=K: w4.gemv(
                                x, p, sc, z, G, fmt, out=y, workspace=ws))
                        elif path in ("dq_f16", "postscale"):
                            mode = w4.DQ_F16 if path == "dq_f16" else w4.POSTSCALE
                            ws = torch.empty(max(16, w4.workspace_bytes(w4.OP_GEMM, M, K, N, G, mode)),
                                             dtype=torch.uint8, device="cuda")
                            calls.append(lambda p=p, sc=sc, z=z, x=x, y=y, ws=ws, mode=mode: w4.gemm(
                                x, p, sc, z, G, fmt, mode, out=y, workspace=ws))
                        elif path == "msd2_fixed_fused":
                            ws = torch.empty(w4.workspace_bytes(w4.OP_GEMM_DECOMP_FUSED, M, K, N, G, 0),
                                             dtype=torch.uint8, device="cuda")
                            calls.append(lambda p=p, sc=sc, z=z, x=x, y=y, ws=ws: w4.gemm_decomp_fixed_fused(
                                x, p, sc, z, G, out=y, workspace=ws))
                        else:
                            ws = torch.empty(w4.workspace_bytes(w4.OP_GEMM_DECOMP, M, K, N, G, 2), dtype=torch.uint8,
                                             device="cuda")
                            fn = w4.gemm_decomp_fixed if path == "msd2_fixed" else (
                                lambda *a, **k: w4.gemm_decomp(*a[:5], 2, **k))
                            calls.append(lambda p=p, sc=sc, z=z, x=x, y=y, ws=ws, fn=fn: fn(x, p, sc, z, G, out=y,
                                                                                             workspace=ws))
                g = graph_of(torch, stream, calls)
                time_replays(torch, stream, g, 1)
                us = time_replays(torch, stream, g, replays) * 1e3 / (replays * n_sets)
                row = {"format": "int4_asym_g128" if fmt == w4.INT4_ASYM else "nf4_b64", "layout": layout,
                       "path": path, "M": M, "us_per_layer": round(us, 1), "weight_bytes": layer_bytes}
                if M == 1:
                    gbs = layer_bytes / (us * 1e-6) / 1e9
                    row.update({"GBps": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)})
                else:
                    tf = flops_256 / (us * 1e-6) / 1e12
                    mult, peak = (2, INT8_MFMA_PEAK_TOPS) if path.startswith("msd") else (1, FP16_MFMA_PEAK_TFLOPS)
                    row.update({"tflops_useful": round(tf, 1), "mfma_frac": round(tf * mult / peak, 4)})
                out.append(row)
                del g, calls
        del sep, fused, sets
        torch.cuda.empty_cache()
    return {"workload": "decoder_layer_hidden8192_inter28672_q64_kv8", "matrices": [list(m) for m in DECODER_LAYER],
            "fused_matrices": [[m[0], m[1], m[2]] for m in DECODER_LAYER_FUSED],
            "note": "M=256 msd paths include the activation decomposition of every product and are measured "
                    "against the dense int8 peak with two int8 products per useful multiply-add; layout "
                    "'separate' runs the seven products, 'fused' the same weights as four (q|k|v and gate|up "
                    "concatenated along N, as inference engines store them)",
            "rows": out}


HOST_LINK_PEAK_GBS = 64.0  # PCIe 5.0 x16, one direction


def bench_residual(w4, torch, stream, gemv_launch, n_sets, gemv_us, K, N, ks, reps=64):
    """Residual compensation on the decode layer (K = N = 8192, M = 1, INT4
    g128): salient-channel selection and the correction that reads the picked
    residual rows from pinned host memory (device memory for comparison), each
    timed as HIP-graph replays on the launch stream, and the whole step (GEMV,
    selection, correction) against the GEMV alone.  The residual is seeded
    noise of the residual's size and place: the kernels' time does not depend
    on its values (their parity is tested elsewhere)."""
    import workloads as wl
    x = torch.from_numpy(wl.make_activations(2, 0, 1, K)).cuda()
    y = torch.zeros((1, N), dtype=torch.float16, device="cuda")
    gen = torch.Generator().manual_seed(50000)
    r_host = torch.empty((K, N), dtype=torch.float16, pin_memory=True)
    r_host.copy_((torch.randn((K, N), generator=gen) * 1e-3).half())
    r_dev = r_host.cuda()
    res = []
    for k in ks:
        idx = torch.empty((k,), dtype=torch.int32, device="cuda")
        timed = {}
        for name, call, count in (
                ("select_us", lambda: w4.salient_select(x, k, out=idx), reps),
                ("correct_host_us", lambda: w4.residual_correct(x, r_host, idx, y), reps),
                ("correct_device_us", lambda: w4.residual_correct(x, r_dev, idx, y), reps),
                ("select_correct_host_us", lambda: w4.salient_correct(x, r_host, k, y, idx=idx), reps)):
            g = graph_of(torch, stream, [call] * count)
            time_replays(torch, stream, g, 1)
            timed[name] = round(time_replays(torch, stream, g, 4) * 1e3 / (4 * count), 2)
            del g

        def chain(i):
            gemv_launch(i)
            w4.salient_select(x, k, out=idx)
            w4.residual_correct(x, r_host, idx, y)

        def fused(i):  # selection and correction in one launch
            gemv_launch(i)
            w4.salient_correct(x, r_host, k, y, idx=idx)

        # the selection depends only on x: it runs on a second stream (same
        # priority) beside the GEMV, and the correction waits for both
        side = torch.cuda.Stream()

        def forked(i):
            cur = torch.cuda.current_stream()
            side.wait_stream(cur)
            with torch.cuda.stream(side):
                w4.salient_select(x, k, out=idx)
            gemv_launch(i)
            cur.wait_stream(side)
            w4.residual_correct(x, r_host, idx, y)
        # the selection and the fp32 correction (which does not read y) on a
        # second stream beside the GEMV; the correction is added to y after both
        c = torch.empty((1, N), dtype=torch.float32, device="cuda")

        def overlapped(i):
            cur = torch.cuda.current_stream()
            side.wait_stream(cur)
            with torch.cuda.stream(side):
                w4.salient_select(x, k, out=idx)
                w4.residual_correct_f32(x, r_host, idx, c)
            gemv_launch(i)
            cur.wait_stream(side)
            w4.residual_apply(c, y)
        g = graph_of(torch, stream, [lambda i=i: chain(i) for i in range(n_sets)])
        time_replays(torch, stream, g, 1)
        serial_us = time_replays(torch, stream, g, 4) * 1e3 / (4 * n_sets)
        del g
        g = graph_of(torch, stream, [lambda i=i: overlapped(i) for i in range(n_sets)])
        time_replays(torch, stream, g, 1)
        overlapped_us = time_replays(torch, stream, g, 4) * 1e3 / (4 * n_sets)
        del g

        def overlapped_one(i):  # the same with selection and correction in one launch
            cur = torch.cuda.current_stream()
            side.wait_stream(cur)
            with torch.cuda.stream(side):
                w4.salient_correct_f32(x, r_host, k, c, idx=idx)
            gemv_launch(i)
            cur.wait_stream(side)
            w4.residual_apply(c, y)
        g = graph_of(torch, stream, [lambda i=i: overlapped_one(i) for i in range(n_sets)])
        time_replays(torch, stream, g, 1)
        overlapped_one_us = time_replays(torch, stream, g, 4) * 1e3 / (4 * n_sets)
        del g
        g = graph_of(torch, stream, [lambda i=i: forked(i) for i in range(n_sets)])
        time_replays(torch, stream, g, 1)
        forked_us = time_replays(torch, stream, g, 4) * 1e3 / (4 * n_sets)
        del g
        g = graph_of(torch, stream, [lambda i=i: fused(i) for i in range(n_sets)])
        time_replays(torch, stream, g, 1)
        fused_us = time_replays(torch, stream, g, 4) * 1e3 / (4 * n_sets)
        del g
        steps = {"serial": serial_us, "forked": forked_us, "fused": fused_us, "overlapped": overlapped_us,
                 "overlapped_one_launch": overlapped_one_us}
        schedule = min(steps, key=steps.get)
        step_us = steps[schedule]
        link = k * N * 2 / (timed["correct_host_us"] * 1e-6) / 1e9
        res.append({"k": k, **timed, "gemv_us": round(gemv_us, 2), "step_serial_us": round(serial_us, 2),
                    "step_forked_us": round(forked_us, 2), "step_fused_us": round(fused_us, 2),
                    "step_overlapped_us": round(overlapped_us, 2),
                    "step_overlapped_one_launch_us": round(overlapped_one_us, 2),
                    "step_us": round(step_us, 2), "schedule": schedule,
                    "overhead_frac": round((step_us - gemv_us) / gemv_us, 3),
                    "residual_bytes": k * N * 2, "host_link_GBps": round(link, 2),
                    "host_link_frac": round(link / HOST_LINK_PEAK_GBS, 3)})
    return {"workload": "decode_gemv_k8192_n8192_m1_int4_g128 + residual of k salient channels",
            "residual": "fp16 [K][N] in pinned host memory, read by the kernel over the host link",
            "step": "step_serial_us: GEMV, selection and correction one after the other on one stream; "
                    "step_forked_us: the selection on a second stream beside the GEMV, the correction after "
                    "both; step_fused_us: GEMV, then selection and correction in one launch "
                    "(w4_salient_correct); step_overlapped_us: the selection and the fp32 correction "
                    "(w4_residual_correct_f32) on a second stream beside the GEMV, then w4_residual_apply; "
                    "step_overlapped_one_launch_us: the same with w4_salient_correct_f32 on the second stream; "
                    "step_us: the fastest (schedule names it)",
            "host_link_peak_GBps": HOST_LINK_PEAK_GBS, "per_k": res}


def attention_call(w4, torch):
    """The decode-attention workload: batch 8, 64 query heads over 8 key/value
    heads of dimension 128, 8192 cached positions, INT4 caches quantized on the
    GPU (w4_quantize per token, w4_pack; V transposed first).  Returns (thunk,
    shape)."""
    B, Hq, Hkv, L, D = 8, 64, 8, 8192, 128
    gen = torch.Generator(device="cuda")
    gen.manual_seed(60000)
    rows = B * Hkv * L
    k = torch.randn((rows, D), generator=gen, device="cuda")
    kc, ks, kz = w4.quantize(k, D, w4.INT4_ASYM)
    kp = w4.pack(kc)
    del k, kc
    v = torch.randn((rows, D), generator=gen, device="cuda")
    vc, vs, vz = w4.quantize(v, D, w4.INT4_ASYM)
    del v
    vt = vc.view(B * Hkv, L, D).transpose(1, 2).contiguous().view(B * Hkv * D, L)
    vp = w4.pack(vt)
    del vc, vt
    q = torch.randn((B, Hq, D), generator=gen, device="cuda").half()
    out = torch.empty_like(q)
    ws = torch.empty(w4.workspace_bytes(w4.OP_ATTN_MSD, B, Hq, L, 0, 0), dtype=torch.uint8, device="cuda")
    ks, kz, vs, vz = (t.view(B, Hkv, L) for t in (ks, kz, vs, vz))
    return (lambda: w4.attn_decode_msd(q, kp, ks, kz, vp, vs, vz, Hkv, out=out, workspace=ws)), (B, Hq, Hkv, L, D)


def bench_attention(w4, torch, stream, reps=20):
    """Decode attention over an INT4 KV cache with Multi-Scale Dequant on both
    products, for a 70B-shaped layer (see attention_call).  Timed as HIP-graph
    replays on the launch stream; rate = cache bytes read (packed K and V plus
    their fp16 scales and zero points) per second, against the 8 TB/s HBM
    peak; the fp16 cache of the same layer would be the bytes of
    `fp16_cache_bytes`."""
    call, (B, Hq, Hkv, L, D) = attention_call(w4, torch)
    g = graph_of(torch, stream, [call] * reps)
    time_replays(torch, stream, g, 1)
    us = time_replays(torch, stream, g, 4) * 1e3 / (4 * reps)
    del g
    cache = B * Hkv * L * (D // 2 * 2 + 4 * 2)  # packed K and V, fp16 scale and zero of each
    fp16 = B * Hkv * L * D * 2 * 2
    rate = cache / (us * 1e-6) / 1e9
    return {"workload": "decode_attention_b8_hq64_hkv8_d128_l8192_int4_kv",
            "us_per_call": round(us, 2), "cache_bytes": cache, "fp16_cache_bytes": fp16,
            "traffic_ratio_vs_fp16": round(fp16 / cache, 2), "GBps": round(rate, 1),
            "hbm_frac": round(rate / HBM_PEAK_GBS, 4),
            "note": "time includes the query decomposition and the chunk combination"}


GEMV_SOURCE = os.path.join(ROOT, "bit_weight_quantized_amd", "csrc", "gemv.hip")
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "gemv_decode_k8192_n8192_hbm_traffic.md")
COPY_BYTES = 256 * 2 ** 20  # the plain copy the --pmc counters are calibrated on


def source_sha256(path=None, text=None):
    """SHA-256 of a C++ source's code: comments removed and whitespace runs
    collapsed, so that a comment edit does not count as a kernel change."""
    import hashlib
    import re
    if text is None:
        with open(path) as f:
            text = f.read()
    code = re.sub(r"//[^\n]*|/\*.*?\*/", " ", text, flags=re.S)
    code = " ".join(code.split())
    return hashlib.sha256(code.encode()).hexdigest()


def read_traffic_profile():
    """Per-launch HBM bytes of the GEMV variants from the committed --pmc
    summary, or None when it is missing or was taken on another version of
    the kernel source.  Rows: | variant | ... | traffic bytes per launch |."""
    if not os.path.exists(TRAFFIC_PROFILE):
        return None
    sha, rows = None, {}
    with open(TRAFFIC_PROFILE) as f:
        for line in f:
            if line.startswith("kernel code sha256:"):
                sha = line.split(":", 1)[1].strip()
            cells = [c.strip() for c in line.strip().strip("|").split("|")]
            if len(cells) >= 3 and cells[0].startswith(("int4", "nf4")):
                try:
                    rows[cells[0]] = float(cells[-1])
                except ValueError:
                    pass
    if sha != source_sha256(GEMV_SOURCE) or not rows:
        return None
    return rows


def variant_name(fmt, M):
    return ("int4_g128" if fmt == 0 else "nf4_b64") + f"_m{M}"


def graph_of(torch, stream, calls):
    """Captures `calls` (a list of thunks) into one HIP graph on `stream`."""
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for c in calls[:2]:  # eager first launches (code objects load outside the capture)
            c()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for c in calls:
            c()
    torch.cuda.synchronize()
    return g


def time_replays(torch, stream, graph, replays):
    """Milliseconds of `replays` back-to-back replays, from HIP events
    recorded on the stream the graph runs on."""
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        start.record(stream)
        for _ in range(replays):
            graph.replay()
        end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end)


def summarize(paths, pattern=None):
    """Markdown tables from rocprofv3 CSV files: kernel statistics, or counter
    values averaged per dispatch and grouped by kernel and launch geometry;
    with `pattern`, only kernels whose name matches that regular expression."""
    import csv
    import collections
    import re
    keep = (lambda name: re.search(pattern, name) is not None) if pattern else (lambda name: True)
    for path in paths:
        with open(path, newline="") as f:
            rows = list(csv.DictReader(f))
        if not rows:
            continue
        cols = {c.lower(): c for c in rows[0]}
        print(f"\n`{os.path.basename(path)}`\n")
        if "averagens" in cols:
            print("| kernel | calls | average (us) | min (us) | max (us) |")
            print("|---|---|---|---|---|")
            for r in rows:
                if not keep(r[cols["name"]]):
                    continue
                print(f"| `{short_kernel(r[cols['name']])}` | {r[cols['calls']]} | "
                      f"{float(r[cols['averagens']]) / 1e3:.2f} | {float(r[cols['minns']]) / 1e3:.2f} | "
                      f"{float(r[cols['maxns']]) / 1e3:.2f} |")
        elif "start_timestamp" in cols and "grid_size_x" in cols:  # kernel trace: per launch geometry
            agg = collections.defaultdict(list)
            for r in rows:
                if not keep(r[cols["kernel_name"]]):
                    continue
                grid = "x".join(str(int(r[cols[f"grid_size_{a}"]]) // int(r[cols[f"workgroup_size_{a}"]]))
                                for a in "xy")
                key = (short_kernel(r[cols["kernel_name"]]), grid, r[cols["workgroup_size_x"]])
                agg[key].append((int(r[cols["end_timestamp"]]) - int(r[cols["start_timestamp"]])) / 1e3)
            print("| kernel | workgroups (x by y) | workgroup size | dispatches | average (us) | min (us) | max (us) |")
            print("|---|---|---|---|---|---|---|")
            for (k, g, wg), v in agg.items():
                print(f"| `{k}` | {g} | {wg} | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f} |")
        elif "counter_name" in cols:
            agg = collections.defaultdict(list)
            for r in rows:
                if not keep(r[cols["kernel_name"]]):
                    continue
                key = (short_kernel(r[cols["kernel_name"]]), r[cols["grid_size"]], r[cols["workgroup_size"]],
                       r[cols["counter_name"]])
                agg[key].append(float(r[cols["counter_value"]]))
            print("| kernel | grid | workgroup | counter | dispatches | mean per dispatch |")
            print("|---|---|---|---|---|---|")
            for (k, g, wg, c), v in agg.items():
                print(f"| `{k}` | {g} | {wg} | {c} | {len(v)} | {sum(v) / len(v):.1f} |")


def traffic_summary(fetch_csv, write_csv):
    """Per-launch HBM bytes of each GEMV variant: FETCH_SIZE and WRITE_SIZE
    (KiB per dispatch) scaled by what each counter reads for the plain copy
    of COPY_BYTES, whose true reads and writes are COPY_BYTES each.  The
    profile pass launches the variants in bench order, --profile-launches
    each, so the i-th run of gemv dispatches is the i-th variant."""
    import csv
    def per_dispatch(path, counter):
        with open(path, newline="") as f:
            rows = [r for r in csv.DictReader(f) if r["Counter_Name"] == counter]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        gemv = [float(r["Counter_Value"]) for r in rows
                if "gemv_kernel" in r["Kernel_Name"] or "gemv_direct_kernel" in r["Kernel_Name"]]
        copy = [float(r["Counter_Value"]) for r in rows
                if "copyBuffer" in r["Kernel_Name"] and int(r["Grid_Size"]) >= 65536]
        return gemv, copy
    names = [variant_name(f, m) for f in (0, 1) for m in (1, 4, 16)]
    fg, fc = per_dispatch(fetch_csv, "FETCH_SIZE")
    wg, wc = per_dispatch(write_csv, "WRITE_SIZE")
    n = len(fg) // len(names)
    assert n > 0 and len(fg) == n * len(names) == len(wg), (len(fg), len(wg))
    fscale = COPY_BYTES / (sum(fc) / len(fc) * 1024)
    wscale = COPY_BYTES / (sum(wc) / len(wc) * 1024)
    print(f"kernel code sha256: {source_sha256(GEMV_SOURCE)}")
    print(f"copy reference: {len(fc)} copies of {COPY_BYTES} bytes; FETCH_SIZE reads "
          f"{sum(fc) / len(fc):.1f} KiB per copy (scale {fscale:.4f}), WRITE_SIZE {sum(wc) / len(wc):.1f} KiB "
          f"(scale {wscale:.4f})\n")
    print("| variant | launches | FETCH_SIZE KiB | WRITE_SIZE KiB | algorithmic bytes | traffic / algorithmic "
          "| traffic bytes per launch |")
    print("|---|---|---|---|---|---|---|")
    for i, name in enumerate(names):
        f = sum(fg[i * n:(i + 1) * n]) / n
        w = sum(wg[i * n:(i + 1) * n]) / n
        t = f * 1024 * fscale + w * 1024 * wscale
        alg = weight_stream_bytes(0 if name.startswith("int4") else 1, 8192, 8192, 128 if name.startswith("int4") else 64)
        print(f"| {name} | {n} | {f:.1f} | {w:.1f} | {alg} | {t / alg:.3f} | {t:.0f} |")


def counter_summary(paths, pattern=None):
    """One row per kernel (and launch geometry) over several --pmc passes:
    each counter's mean per dispatch, then derived figures.
    * MfmaUtil: rocprofv3's derived matrix-core busy percentage
      (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE times the SIMD count);
    * clock: GRBM_GUI_ACTIVE (summed over the 8 XCDs) / 8 over the dispatch
      duration of the same pass;
    * VALU / MFMA: SQ_INSTS_VALU over SQ_INSTS_MFMA (issued instructions);
    * MFMA co-exec: SQ_VALU_MFMA_COEXEC_CYCLES over SQ_VALU_MFMA_BUSY_CYCLES
      is not derivable from one pass, so the raw counts are listed;
    * LDS conflict: SQ_LDS_BANK_CONFLICT over SQ_LDS_IDX_ACTIVE;
    * HBM bytes: FETCH_SIZE and WRITE_SIZE (KiB) scaled by what they read for
      the plain copies of COPY_BYTES at the end of the profiled command."""
    import csv
    import collections
    import re
    keep = (lambda name: re.search(pattern, name) is not None) if pattern else (lambda name: True)
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    durs = collections.defaultdict(lambda: collections.defaultdict(list))
    copies = collections.defaultdict(list)
    order = []
    for path in paths:
        with open(path, newline="") as f:
            rows = list(csv.DictReader(f))
        for r in rows:
            name = r["Kernel_Name"]
            counter = r["Counter_Name"]
            if "copyBuffer" in name and int(r["Grid_Size"]) >= 65536:
                copies[counter].append(float(r["Counter_Value"]))
                continue
            if not keep(name):
                continue
            key = (short_kernel(name), r["Grid_Size"], r["Workgroup_Size"])
            if key not in vals:
                order.append(key)
            vals[key][counter].append(float(r["Counter_Value"]))
            if "Start_Timestamp" in r and r["Start_Timestamp"]:
                durs[key][counter].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    scale = {c: COPY_BYTES / (sum(v) / len(v) * 1024) for c, v in copies.items()
             if c in ("FETCH_SIZE", "WRITE_SIZE") and v and sum(v) > 0}
    if scale:
        print("copy reference: " + ", ".join(
            f"{c} reads {sum(copies[c]) / len(copies[c]):.1f} KiB per {COPY_BYTES}-byte copy (scale {scale[c]:.4f})"
            for c in sorted(scale)) + "\n")
    counters = sorted({c for k in order for c in vals[k]})
    print("| kernel | grid | workgroup | " + " | ".join(counters) + " | derived |")
    print("|---|---|---|" + "---|" * len(counters) + "---|")
    for key in order:
        v = {c: sum(x) / len(x) for c, x in vals[key].items()}
        cells = [f"{v[c]:.4g}" if c in v else "" for c in counters]
        d = []
        if "MfmaUtil" in v:
            d.append(f"MFMA busy {v['MfmaUtil']:.1f} %")
        if "GRBM_GUI_ACTIVE" in v and durs[key].get("GRBM_GUI_ACTIVE"):
            us = sum(durs[key]["GRBM_GUI_ACTIVE"]) / len(durs[key]["GRBM_GUI_ACTIVE"])
            d.append(f"{us:.1f} us, clock {v['GRBM_GUI_ACTIVE'] / 8 / (us * 1e3):.2f} GHz")
        if "SQ_INSTS_VALU" in v and v.get("SQ_INSTS_MFMA"):
            d.append(f"VALU/MFMA {v['SQ_INSTS_VALU'] / v['SQ_INSTS_MFMA']:.2f}")
        if "SQ_LDS_BANK_CONFLICT" in v and v.get("SQ_LDS_IDX_ACTIVE"):
            d.append(f"LDS conflict {100 * v['SQ_LDS_BANK_CONFLICT'] / v['SQ_LDS_IDX_ACTIVE']:.1f} %")
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            if c in v and c in scale:
                d.append(f"{c.split('_')[0].lower()} {v[c] * 1024 * scale[c] / 1e6:.1f} MB")
        print(f"| `{key[0]}` | {key[1]} | {key[2]} | " + " | ".join(cells) + " | " + "; ".join(d) + " |")


def short_kernel(name):
    name = name.replace("w4::(anonymous namespace)::", "")
    return name.split("(")[0] if "(" in name else name


def main():
    args = parse()
    if args.summarize:
        summarize(args.summarize, args.kernels)
        return
    if args.traffic:
        traffic_summary(*args.traffic)
        return
    if args.counters:
        counter_summary(args.counters, args.kernels)
        return
    if args.steps < 1 or args.warmup < 0:
        print("bench.py: --steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        sys.exit(2)
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
    # split-K partials (written before they are read: no initial contents needed)
    wss = {(fmt, M): torch.zeros(max(16, w4.workspace_bytes(w4.OP_GEMV, M, K, N, G, fmt)), dtype=torch.uint8,
                                 device="cuda") for fmt, M, G in variants}

    def launch(fmt, M, G, i):
        packed, scale, zero = sets[fmt][i % n_sets]
        w4.gemv(xs[M], packed, scale, zero, G, fmt, out=ys[M], workspace=wss[(fmt, M)])

    stream = torch.cuda.Stream()
    if args.profile_gemm:
        _, paths = prefill_paths(w4, torch)
        with torch.cuda.stream(stream):
            for name, (fn, _, _) in paths.items():
                for _ in range(args.profile_launches):
                    fn()
                torch.cuda.synchronize()
                print(f"profile gemm: {args.profile_launches} calls of {name}", flush=True)
            src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
            dst = torch.empty_like(src)
            for _ in range(4):
                dst.copy_(src)
            torch.cuda.synchronize()
        print(f"profile gemm: 4 copies of {COPY_BYTES} bytes (reads {COPY_BYTES}, writes {COPY_BYTES})", flush=True)
        return
    if args.profile_attention:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        call, _ = attention_call(w4, torch)
        with torch.cuda.stream(stream):
            for _ in range(args.profile_launches):
                call()
            torch.cuda.synchronize()
            print(f"profile attention: {args.profile_launches} calls", flush=True)
            for _ in range(4):
                dst.copy_(src)
            torch.cuda.synchronize()
        print(f"profile attention: 4 copies of {COPY_BYTES} bytes (reads {COPY_BYTES}, writes {COPY_BYTES})",
              flush=True)
        return
    if args.profile_pass:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        with torch.cuda.stream(stream):
            for fmt, M, G in variants:
                for i in range(args.profile_launches):
                    launch(fmt, M, G, i)
                torch.cuda.synchronize()
                print(f"profile pass: {args.profile_launches} launches of {variant_name(fmt, M)}", flush=True)
            for _ in range(4):
                dst.copy_(src)
            torch.cuda.synchronize()
        print(f"profile pass: 4 copies of {COPY_BYTES} bytes (reads {COPY_BYTES}, writes {COPY_BYTES})",
              flush=True)
        return

    # ---- the timed region: exactly --steps steps after exactly --warmup
    # steps, as HIP graph replays: a graph of n_sets whole steps (one pass
    # over the weight rotation) replayed as often as it fits, then a graph of
    # the remaining steps
    def step_calls(i):
        return [lambda fmt=fmt, M=M, G=G: launch(fmt, M, G, i * len(Ms) + Ms.index(M)) for fmt, M, G in variants]

    steps_per_graph = n_sets
    graphs = {}

    def steps_graph(n):
        if n not in graphs:
            graphs[n] = graph_of(torch, stream, [c for i in range(n) for c in step_calls(i)])
        return graphs[n]

    def run_steps(n):
        """Replays of exactly n steps on `stream` (no synchronization)."""
        for _ in range(n // steps_per_graph):
            steps_graph(steps_per_graph).replay()
        if n % steps_per_graph:
            steps_graph(n % steps_per_graph).replay()

    for n in {steps_per_graph, args.steps % steps_per_graph, args.warmup % steps_per_graph} - {0}:
        steps_graph(n)  # captured before the timed region
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        run_steps(args.warmup)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        start.record(stream)
        run_steps(args.steps)
        end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    steps_timed = args.steps
    ms_per_step = total_ms / steps_timed
    step_bytes = sum(weight_stream_bytes(fmt, K, N, G) for fmt, M, G in variants)
    value = step_bytes * steps_timed / (total_ms * 1e-3) / 1e9
    graphs.clear()

    # ---- live per-launch timing of each variant: a graph of one launch per
    # weight set, replayed back to back between events on its stream
    per = []
    for fmt, M, G in variants:
        g = graph_of(torch, stream, [lambda fmt=fmt, M=M, G=G, i=i: launch(fmt, M, G, i) for i in range(n_sets)])
        time_replays(torch, stream, g, 1)
        ms = time_replays(torch, stream, g, args.kernel_replays)
        us = ms * 1e3 / (args.kernel_replays * n_sets)
        b = weight_stream_bytes(fmt, K, N, G)
        per.append({"variant": variant_name(fmt, M), "us_per_launch": round(us, 3), "weight_bytes": b,
                    "GBps": round(b / (us * 1e-6) / 1e9, 1), "launches": args.kernel_replays * n_sets})
        del g
    sum_bytes = sum(p["weight_bytes"] for p in per)
    sum_us = sum(p["us_per_launch"] for p in per)
    achieved = sum_bytes / (sum_us * 1e-6) / 1e9

    traffic_rows = read_traffic_profile()
    traffic = None
    if traffic_rows and all(p["variant"] in traffic_rows for p in per):
        traffic = round(sum(traffic_rows[p["variant"]] for p in per) / len(per))

    plain = None
    try:
        plain = bench_plain_read(w4, torch, stream, per_set)
    except Exception as e:  # reported, never fatal to the headline line
        plain = {"error": f"{type(e).__name__}: {e}"}
    gemm = bench_gemm_prefill(w4, torch, args.gemm_reps) if args.gemm_reps > 0 else None
    if gemm is not None:
        for key, fn in (("mfma_ceiling", lambda: bench_mfma_ceiling(w4, torch)),
                        ("library_f16_gemm", lambda: bench_library_f16_gemm(torch))):
            try:
                gemm[key] = fn()
            except Exception as e:  # reported, never fatal to the headline line
                gemm[key] = {"error": f"{type(e).__name__}: {e}"}
    single = None
    try:
        single = bench_single_gemv(w4, torch, stream)
    except Exception as e:  # reported, never fatal to the headline line
        single = {"error": f"{type(e).__name__}: {e}"}
    mlp = layer = None
    if args.layers:
        try:
            mlp = bench_mlp_gemv(w4, torch, stream)
            layer = bench_decoder_layer(w4, torch, stream)
        except Exception as e:  # reported, never fatal to the headline line
            layer = {"error": f"{type(e).__name__}: {e}"}
    attn = None
    if args.attention:
        try:
            attn = bench_attention(w4, torch, stream)
        except Exception as e:  # reported, never fatal to the headline line
            attn = {"error": f"{type(e).__name__}: {e}"}
    resid = None
    if args.residual:
        m1 = next(p for p in per if p["variant"] == variant_name(w4.INT4_ASYM, 1))
        try:
            resid = bench_residual(w4, torch, stream, lambda i: launch(w4.INT4_ASYM, 1, 128, i), n_sets,
                                   m1["us_per_launch"], K, N, ks=(16, 82, 256))
        except Exception as e:  # reported, never fatal to the headline line
            resid = {"error": f"{type(e).__name__}: {e}"}

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
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic: weights N(0,0.02^2) fp32 quantized on the GPU, activations N(0,1) fp16 with 1%% x20 "
                "outlier channels; weights rotate over %d sets per format (%.0f MB)" % (n_sets, n_sets * per_set / 1e6),
        "config": {"workload": "decode_gemv_k8192_n8192", "M": list(Ms), "K": K, "N": N,
                   "formats": ["int4_asym_g128", "nf4_b64"], "launches_per_step": len(variants),
                   "timed": "HIP graph replays (graphs of %d steps and of the remainder), exactly the "
                            "requested steps after exactly the requested warmup" % steps_per_graph},
        "roofline": {"bound": "hbm", "kernel": "the 6 GEMV launches of a step (gemv_kernel at M = 1 and 4, gemv_direct_kernel at M = 16)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "bytes_per_launch": "packed N*K/2 + fp16 scales (+ zeros) = %d" % per_set,
                     "launch_average_us": round(sum_us / len(per), 3),
                     "plain_read_frac": plain.get("hbm_frac") if isinstance(plain, dict) else None},
        "per_launch": per,
        "plain_read": plain,
        "gemm_prefill": gemm,
        "single_gemv": single,
        "mlp_gemv": mlp,
        "decoder_layer": layer,
        "residual_compensation": resid,
        "attention_kv_msd": attn,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
