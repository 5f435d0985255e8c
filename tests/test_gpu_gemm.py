"""GPU parity: w4_gemm (dequantize-to-fp16 and post-scaled modes) against the
fp64 oracle.

Small shapes use oracle-quantized, oracle-packed weights and compare every
output; they span several 128 x 128 tiles, ragged M and N tails and both group
sizes.  The full prefill shape (M = 2048, K = 5120, N = 25600) runs the whole
GPU pipeline and compares sampled output columns whose weight rows the oracle
quantizes itself."""
import numpy as np
import pytest
import torch

import bit_weight_quantized_amd as w4
import oracle as o
import workloads as wl
from gpu_helpers import (TOL_ROW_REL_L2, announce, dev, host, oracle_weights, require_gpu,
                         row_rel_l2, upload_weights)

pytestmark = pytest.mark.gpu

FMTS = [(o.FMT_INT4_ASYM, 128), (o.FMT_INT4_ASYM, 64), (o.FMT_NF4, 64), (o.FMT_NF4, 128)]
MODES = [w4.DQ_F16, w4.POSTSCALE]


def reference(mode, fmt, x, codes, scale, zero, G):
    if mode == w4.POSTSCALE:
        return o.postscale_ref(fmt, x, codes, scale, zero, G)
    return o.matmul_ref(x, o.dequant(fmt, codes, scale, zero, G))


@pytest.mark.parametrize("fmt,G", FMTS)
@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("M,K,N", [(1, 128, 16), (5, 640, 48), (130, 1024, 272), (257, 512, 144),
                                   (64, 2048, 256), (384, 256, 400)])
def test_gemm_small(fmt, G, mode, M, K, N):
    if K % G:
        pytest.skip("K not a multiple of G")
    require_gpu()
    w = wl.make_weight(200 + M, 0, N, K)
    x = wl.make_activations(200 + M, 0, M, K)
    codes, scale, zero = oracle_weights(fmt, w, G)
    packed, sc, zc = upload_weights(codes, scale, zero)
    announce("gemm", dict(fmt=fmt, G=G, mode=mode, M=M, K=K, N=N))
    y = host(w4.gemm(dev(x), packed, sc, zc, G, fmt, mode))
    assert y.shape == (M, N)
    err = row_rel_l2(y, reference(mode, fmt, x, codes, scale, zero, G))
    assert err <= TOL_ROW_REL_L2, err


@pytest.mark.parametrize("S", [2, 3, 5])
@pytest.mark.parametrize("M,K,N", [(130, 1024, 272), (257, 768, 144)])
def test_gemm_split_k(monkeypatch, S, M, K, N):
    """K split over S workgroup slices (fp32 partials added by a second
    kernel): within tolerance of the oracle for both modes and formats,
    repeatable, and independent of the workspace's previous contents (NaN
    bytes here)."""
    require_gpu()
    monkeypatch.setenv("W4_GEMM_S", str(S))
    w = wl.make_weight(300 + S, 0, N, K)
    x = wl.make_activations(300 + S, 0, M, K)
    for fmt, G in FMTS[:3]:
        codes, scale, zero = oracle_weights(fmt, w, G)
        packed, sc, zc = upload_weights(codes, scale, zero)
        for mode in MODES:
            n_ws = w4.workspace_bytes(w4.OP_GEMM, M, K, N, G, mode)
            assert n_ws == min(S, K // 128) * M * N * 4
            ws = torch.full((n_ws,), 0xFF, dtype=torch.uint8, device="cuda")
            announce("gemm split", dict(S=S, fmt=fmt, G=G, mode=mode, M=M, K=K, N=N))
            y1 = host(w4.gemm(dev(x), packed, sc, zc, G, fmt, mode, workspace=ws))
            y2 = host(w4.gemm(dev(x), packed, sc, zc, G, fmt, mode, workspace=ws))
            assert row_rel_l2(y1, reference(mode, fmt, x, codes, scale, zero, G)) <= TOL_ROW_REL_L2
            assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))


def test_gemm_without_workspace_runs_unsplit():
    """A shape that would split (M = 256, N = 1024: 8 output tiles) computes
    the same product unsplit when the caller passes no room for partials."""
    require_gpu()
    M, K, N, G, fmt = 256, 2048, 1024, 128, o.FMT_INT4_ASYM
    assert w4.workspace_bytes(w4.OP_GEMM, M, K, N, G, w4.POSTSCALE) > 0
    w = wl.make_weight(13, 0, N, K)
    x = wl.make_activations(13, 0, M, K)
    codes, scale, zero = oracle_weights(fmt, w, G)
    packed, sc, zc = upload_weights(codes, scale, zero)
    tiny = torch.zeros(16, dtype=torch.uint8, device="cuda")
    announce("gemm unsplit", dict(M=M, K=K, N=N))
    y = host(w4.gemm(dev(x), packed, sc, zc, G, fmt, w4.POSTSCALE, workspace=tiny))
    assert row_rel_l2(y, reference(w4.POSTSCALE, fmt, x, codes, scale, zero, G)) <= TOL_ROW_REL_L2


def test_gemm_zero_rows_and_columns():
    """All-zero weight rows give exactly zero outputs; an all-zero token row
    gives an exactly zero output row."""
    require_gpu()
    K, N, M = 256, 160, 140
    w = np.zeros((N, K), np.float32)
    w[::2] = wl.make_weight(11, 0, N // 2, K)
    x = wl.make_activations(11, 0, M, K)
    x[7] = 0
    for fmt, G in FMTS[:3]:
        codes, scale, zero = oracle_weights(fmt, w, G)
        packed, sc, zc = upload_weights(codes, scale, zero)
        for mode in MODES:
            announce("gemm zeros", fmt, G, mode)
            y = host(w4.gemm(dev(x), packed, sc, zc, G, fmt, mode))
            assert np.all(y[:, 1::2] == 0)
            assert np.all(y[7] == 0)
            ref = reference(mode, fmt, x, codes, scale, zero, G)
            keep = np.arange(M) != 7
            assert row_rel_l2(y[keep], ref[keep]) <= TOL_ROW_REL_L2


def test_gemm_repeatable_and_matches_gemv():
    """Two calls give bit-identical outputs; for M <= 32 the tiled product
    agrees with the GEMV within the tolerance (both against the oracle)."""
    require_gpu()
    K, N, M = 1024, 320, 16
    w = wl.make_weight(12, 0, N, K)
    x = wl.make_activations(12, 0, M, K)
    for fmt, G in FMTS[::2]:
        codes, scale, zero = oracle_weights(fmt, w, G)
        packed, sc, zc = upload_weights(codes, scale, zero)
        xd = dev(x)
        announce("gemm repeat", fmt, G)
        a = host(w4.gemm(xd, packed, sc, zc, G, fmt, w4.POSTSCALE))
        b = host(w4.gemm(xd, packed, sc, zc, G, fmt, w4.POSTSCALE))
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
        v = host(w4.gemv(xd, packed, sc, zc, G, fmt))
        ref = o.matmul_ref(x, o.dequant(fmt, codes, scale, zero, G))
        assert row_rel_l2(a, ref) <= TOL_ROW_REL_L2
        assert row_rel_l2(v, ref) <= TOL_ROW_REL_L2


def full_size_columns(fmt, G, M, K, N, cfg, mat, n_sample):
    """Quantizes and packs seeded weights on the GPU; returns (x, codes, scale,
    zero, packed, sampled rows, the oracle's quantization of those rows)."""
    w = wl.make_weight(cfg, mat, N, K)
    x = wl.make_activations(cfg, mat, M, K)
    announce("gemm full quantize", dict(fmt=fmt, G=G, K=K, N=N))
    codes, scale, zero = w4.quantize(dev(w), G, fmt)
    packed = w4.pack(codes)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(cfg + mat).choice(N, n_sample,
                                                                                         replace=False)]))
    rc, rs, rz = oracle_weights(fmt, w[rows], G)
    assert np.array_equal(host(codes[rows]), rc)  # the sampled weights are the oracle's
    return x, codes, scale, zero, packed, rows, (rc, rs, rz)


@pytest.mark.parametrize("mode", MODES)
def test_gemm_prefill_m2048_k5120_n25600(mode):
    M, K, N, G, fmt = 2048, 5120, 25600, 128, o.FMT_INT4_ASYM
    x, codes, scale, zero, packed, rows, (rc, rs, rz) = full_size_columns(fmt, G, M, K, N, 4, 0, 96)
    announce("gemm prefill", dict(mode=mode, M=M, K=K, N=N))
    y = host(w4.gemm(dev(x), packed, scale, zero, G, fmt, mode))
    ref = reference(mode, fmt, x, rc, rs, rz, G)
    assert row_rel_l2(y[:, rows], ref) <= TOL_ROW_REL_L2


@pytest.mark.parametrize("fmt,G", [(o.FMT_NF4, 64), (o.FMT_INT4_ASYM, 128)])
@pytest.mark.parametrize("mat", [0, 1, 4, 6])
def test_gemm_layer_m256(fmt, G, mat):
    """The 70B-style decoder layer's matrices (q, k, gate, down; v and o share
    the shapes of k and q) at M = 256."""
    M = 256
    K, N = wl.WORKLOADS[5].mats[mat].K, wl.WORKLOADS[5].mats[mat].N
    x, codes, scale, zero, packed, rows, (rc, rs, rz) = full_size_columns(fmt, G, M, K, N, 5, mat, 48)
    for mode in MODES:
        announce("gemm layer", dict(fmt=fmt, mode=mode, M=M, K=K, N=N))
        y = host(w4.gemm(dev(x), packed, scale, zero, G, fmt, mode))
        assert row_rel_l2(y[:, rows], reference(mode, fmt, x, rc, rs, rz, G)) <= TOL_ROW_REL_L2
