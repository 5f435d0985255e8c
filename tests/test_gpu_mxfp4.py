"""GPU parity: the MXFP4 path (MXFP4 weights, activations split into MXFP4
slices, block-scaled fp4 matrix cores) against the fp64 oracle.

Codes, E8M0 scales, packed bytes and the activation slices are integer results
and must be bit-exact; the fp16 output is compared with the oracle's exact
product of the same decomposed operands within the row-relative tolerance."""
import numpy as np
import pytest
import torch

import bit_weight_quantized_amd as w4
import oracle as o
import workloads as wl
from gpu_helpers import TOL_ROW_REL_L2, announce, dev, host, require_gpu, row_rel_l2

pytestmark = pytest.mark.gpu


def pack_rows(codes):
    """Codes [..., K] -> bytes [..., K/2], low nibble first (the slice layout)."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def e8m0(e):
    return (np.asarray(e, dtype=np.int64) + 127).astype(np.uint8)


def special_weights(seed, N, K):
    w = wl.make_weight(seed, 0, N, K)
    w[0, :32] = 0.0                                   # an all-zero block
    w[1, :32] = np.float32(-0.0)
    w[2, 32:64] = np.float32(6.0 * 2.0 ** -7) * np.array(
        [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] * 4, np.float32)  # every tie of the grid
    w[3, 64:96] = np.float32(3e4)                     # large block
    w[4, 96:128] = np.float32(1e-30)                  # tiny block
    return w


@pytest.mark.parametrize("N,K", [(16, 128), (48, 1024), (272, 512)])
def test_quantize_and_pack_mx_bit_exact(N, K):
    require_gpu()
    w = special_weights(700 + N, N, K)
    announce("quantize_mx", dict(N=N, K=K))
    codes, scale = w4.quantize_mx(dev(w))
    rc, re = o.quantize_mxfp4(w)
    assert np.array_equal(host(codes), rc)
    assert np.array_equal(host(scale), e8m0(re))
    packed = w4.pack_mx(codes)
    assert np.array_equal(host(packed), o.pack_mx(rc))


def mx_case(seed, M, K, N, outliers=True):
    w = wl.make_weight(seed, 0, N, K)
    x = wl.make_activations(seed, 0, M, K, outliers=outliers)
    wc, we = o.quantize_mxfp4(w)
    return x, wc, we


def run_mx(x, wc, we, nslices):
    M, K = x.shape
    packed = dev(o.pack_mx(wc))
    sc = dev(e8m0(we))
    sl = torch.empty((nslices, M, K // 2), dtype=torch.uint8, device="cuda")
    ss = torch.empty((nslices, M, K // 32), dtype=torch.uint8, device="cuda")
    y, _, _ = w4.gemm_mx(dev(x), packed, sc, nslices, slices_out=sl, scales_out=ss)
    return host(y), host(sl), host(ss)


@pytest.mark.parametrize("nslices", [2, 1])
@pytest.mark.parametrize("M,K,N", [(1, 128, 16), (5, 640, 48), (130, 1024, 272), (257, 512, 144),
                                   (64, 2048, 256), (300, 256, 528)])
def test_gemm_mx_small(nslices, M, K, N):
    require_gpu()
    x, wc, we = mx_case(710 + M, M, K, N)
    announce("gemm_mx", dict(nslices=nslices, M=M, K=K, N=N))
    y, sl, ss = run_mx(x, wc, we, nslices)
    C, E = o.decompose_mxfp4(x, nslices)
    assert np.array_equal(sl, pack_rows(C))
    assert np.array_equal(ss, e8m0(E))
    ref = o.mx_matmul(C, E, wc, we)
    assert row_rel_l2(y, ref) <= TOL_ROW_REL_L2


def test_gemm_mx_degenerate_rows():
    """A zero row (output exactly 0), a row with one huge value, a row of
    values on the E2M1 grid (second slice zero), negative zeros."""
    require_gpu()
    M, K, N = 5, 256, 64
    x, wc, we = mx_case(720, M, K, N)
    x[0] = 0
    x[1] = 0
    x[1, 17] = 30000
    x[2] = np.float16(np.resize([0.5, -1.0, 1.5, -2.0, 3.0, -4.0, 6.0, 0.0], K))
    x[3, :40] = np.float16(-0.0)
    announce("gemm_mx degenerate")
    y, sl, ss = run_mx(x, wc, we, 2)
    C, E = o.decompose_mxfp4(x, 2)
    assert np.array_equal(sl, pack_rows(C))
    assert np.array_equal(ss, e8m0(E))
    assert np.all(C[1, 2] == 0)
    assert np.all(y[0] == 0)
    ref = o.mx_matmul(C, E, wc, we)
    assert row_rel_l2(y[1:], ref[1:]) <= TOL_ROW_REL_L2


def test_gemm_mx_repeatable_and_workspace_only():
    require_gpu()
    M, K, N = 200, 1024, 192
    x, wc, we = mx_case(721, M, K, N)
    packed, sc = dev(o.pack_mx(wc)), dev(e8m0(we))
    ws = torch.empty(w4.workspace_bytes(w4.OP_GEMM_MX, M, K, N, 32, 2), dtype=torch.uint8, device="cuda")
    announce("gemm_mx repeat")
    a = host(w4.gemm_mx(dev(x), packed, sc, 2, workspace=ws))
    b = host(w4.gemm_mx(dev(x), packed, sc, 2, workspace=ws))
    c, _, _ = run_mx(x, wc, we, 2)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    assert np.array_equal(a.view(np.uint16), c.view(np.uint16))


@pytest.mark.parametrize("nslices", [2, 1])
def test_gemm_mx_prefill_m2048_k5120_n25600(nslices):
    """Full prefill shape with GPU-quantized weights: sampled weight rows'
    codes and scales bit-exact, slices and scales bit-exact over the whole
    input, outputs compared on the sampled columns."""
    M, K, N = 2048, 5120, 25600
    w = wl.make_weight(4, 0, N, K)
    x = wl.make_activations(4, 0, M, K)
    announce("gemm_mx full quantize")
    codes, scale = w4.quantize_mx(dev(w))
    packed = w4.pack_mx(codes)
    sl = torch.empty((nslices, M, K // 2), dtype=torch.uint8, device="cuda")
    ss = torch.empty((nslices, M, K // 32), dtype=torch.uint8, device="cuda")
    announce("gemm_mx prefill", dict(nslices=nslices, M=M, K=K, N=N))
    y, _, _ = w4.gemm_mx(dev(x), packed, scale, nslices, slices_out=sl, scales_out=ss)
    y = host(y)
    C, E = o.decompose_mxfp4(x, nslices)
    assert np.array_equal(host(sl), pack_rows(C))
    assert np.array_equal(host(ss), e8m0(E))
    rows = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(43).choice(N, 48, replace=False)]))
    rc, re = o.quantize_mxfp4(w[rows])
    assert np.array_equal(host(codes[rows]), rc)
    assert np.array_equal(host(scale[rows]), e8m0(re))
    ref = o.mx_matmul(C, E, rc, re)
    assert row_rel_l2(y[:, rows], ref) <= TOL_ROW_REL_L2
