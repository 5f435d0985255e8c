"""GPU parity: quantize and pack are bit-exact against the oracle."""
import numpy as np
import pytest
import torch

import bit_weight_quantized_amd as w4
import oracle as o
import workloads as wl
from gpu_helpers import announce, dev, host, oracle_weights, require_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt", [o.FMT_INT4_ASYM, o.FMT_NF4])
@pytest.mark.parametrize("N,K,G", [(16, 64, 64), (48, 384, 128), (64, 1024, 64), (32, 2048, 128)])
def test_quantize_bit_exact_small(fmt, N, K, G):
    require_gpu()
    w = wl.make_weight(11, fmt, N, K)
    announce("quantize", fmt, N, K, G)
    codes, scale, zero = w4.quantize(dev(w), G, fmt)
    torch.cuda.synchronize()
    rc, rs, rz = oracle_weights(fmt, w, G)
    assert np.array_equal(host(codes), rc)
    assert np.array_equal(host(scale).view(np.uint16), rs.view(np.uint16))
    if fmt == o.FMT_INT4_ASYM:
        assert np.array_equal(host(zero).view(np.uint16), rz.view(np.uint16))


def test_quantize_special_groups():
    """All-zero groups, all-positive groups, grid-aligned groups, ties."""
    require_gpu()
    rng = np.random.default_rng(4)
    w = np.zeros((32, 256), np.float32)
    w[1, :64] = np.linspace(0.001, 0.2, 64, dtype=np.float32)       # all positive
    w[2, :64] = -np.linspace(0.001, 0.2, 64, dtype=np.float32)      # all negative
    w[3] = (2.0 ** -6 * (rng.integers(0, 16, 256) - 7)).astype(np.float32)  # on a grid
    w[4, :64] = 1.0                                                  # constant
    w[5, 64:128] = np.float32(1e-30)                                 # underflowing scale
    c = o.nf4_codebook()
    w[6] = c[rng.integers(0, 16, 256)] * np.float32(0.5)             # exact NF4 levels
    w[7, :] = 0.5 * (c[8] + c[9]) * np.float32(1.0)                  # midpoint ties
    w[7, 0] = 1.0
    w[8:] = wl.make_weight(12, 0, 24, 256)
    for fmt in (o.FMT_INT4_ASYM, o.FMT_NF4):
        for G in (64, 128):
            announce("quantize special", fmt, G)
            codes, scale, zero = w4.quantize(dev(w), G, fmt)
            torch.cuda.synchronize()
            rc, rs, rz = oracle_weights(fmt, w, G)
            assert np.array_equal(host(codes), rc), (fmt, G)
            assert np.array_equal(host(scale).view(np.uint16), rs.view(np.uint16)), (fmt, G)
            if fmt == o.FMT_INT4_ASYM:
                assert np.array_equal(host(zero).view(np.uint16), rz.view(np.uint16))


@pytest.mark.parametrize("N,K", [(16, 128), (48, 384), (256, 8192), (32, 28672)])
def test_pack_bit_exact(N, K):
    """The packed bytes in the tile layout equal the oracle's, byte for byte."""
    require_gpu()
    codes = np.random.default_rng(N + K).integers(0, 16, size=(N, K)).astype(np.uint8)
    announce("pack", N, K)
    packed = w4.pack(dev(codes))
    torch.cuda.synchronize()
    assert np.array_equal(host(packed), o.pack_w4(codes))


@pytest.mark.parametrize("fmt,G", [(o.FMT_INT4_ASYM, 128), (o.FMT_NF4, 64)])
def test_quantize_full_size_sampled_rows(fmt, G):
    """8192 x 8192 (the decode GEMV layer): the GPU quantizes every row, the
    oracle re-derives a sample of rows from the same seeded weights."""
    require_gpu()
    N = K = 8192
    w = wl.make_weight(2, 0, N, K)
    announce("quantize full", fmt, N, K, G)
    codes, scale, zero = w4.quantize(dev(w), G, fmt)
    packed = w4.pack(codes)
    torch.cuda.synchronize()
    # whole 16-row tiles, so the packed bytes can be compared tile for tile
    tiles = np.unique(np.concatenate([[0, N // 16 - 1], np.random.default_rng(1).choice(N // 16, 6, replace=False)]))
    rows = (tiles[:, None] * 16 + np.arange(16)[None, :]).reshape(-1)
    rc, rs, rz = oracle_weights(fmt, w[rows], G)
    assert np.array_equal(host(codes[rows]), rc)
    assert np.array_equal(host(scale[rows]).view(np.uint16), rs.view(np.uint16))
    if fmt == o.FMT_INT4_ASYM:
        assert np.array_equal(host(zero[rows]).view(np.uint16), rz.view(np.uint16))
    assert np.array_equal(host(packed[rows]), o.pack_w4(rc))
