"""GPU check of w4_mfma_rate, the matrix-core rate probe: every product is
issued (the accumulators equal iters times one product, computed on the host
from the documented lane layout of the 16x16x32 fp16 and 16x16x64 int8
products) and every wave reports its elapsed ticks."""
import numpy as np
import pytest
import torch

import bit_weight_quantized_amd as w4
from gpu_helpers import announce, require_gpu

pytestmark = pytest.mark.gpu

WG, ITERS = 3, 8


def product(kind):
    """D[m][n] of one product of the probe's operands (lane l holds A row
    l % 16 and B column l % 16 for the k block l / 16)."""
    lanes = np.arange(64)
    if kind == 0:  # 8 fp16 values per lane: words base ^ w (A) and base ^ (w + 4) (B), low half then high
        def vals(l, off):
            out = []
            for w in range(4):
                out += [1.0 + (((l & 7) ^ (w + off)) * 2.0 ** -10), 1.0]
            return out
        kb = 8
        A = np.zeros((16, 32))
        B = np.zeros((32, 16))
        for l in lanes:
            A[l % 16, kb * (l // 16):kb * (l // 16) + kb] = vals(l, 0)
            B[kb * (l // 16):kb * (l // 16) + kb, l % 16] = vals(l, 4)
    else:  # 16 int8 values per lane, the same register as A and B
        def vals(l):
            words = [0x01010101 * (l & 3), 0x01020304, 0x02010201, 0x01000100]
            return [(wd >> (8 * i)) & 0xFF for wd in words for i in range(4)]
        kb = 16
        A = np.zeros((16, 64), dtype=np.int64)
        B = np.zeros((64, 16), dtype=np.int64)
        for l in lanes:
            A[l % 16, kb * (l // 16):kb * (l // 16) + kb] = vals(l)
            B[kb * (l // 16):kb * (l // 16) + kb, l % 16] = vals(l)
    return A @ B


@pytest.mark.parametrize("kind", [0, 1])
def test_mfma_rate_products(kind):
    require_gpu()
    D = product(kind)
    lanes = np.arange(64)
    # lane l holds D[4 (l / 16) + r][l % 16], r = 0..3; the sink adds the 8 accumulators' 4 values
    per_lane = np.array([sum(float(D[4 * (l // 16) + r, l % 16]) for r in range(4)) for l in lanes]) * 8 * ITERS
    sink = torch.full((WG * 512,), float("nan"), device="cuda")
    ticks = torch.zeros(WG * 16, dtype=torch.int64, device="cuda")
    announce("mfma rate", dict(kind=kind, workgroups=WG, iters=ITERS))
    w4.mfma_rate(kind, 0, WG, ITERS, sink, ticks)
    got = sink.cpu().numpy().reshape(WG * 8, 64)
    want = np.broadcast_to(per_lane, got.shape)
    if kind == 1:
        assert np.array_equal(got, want)
    else:
        np.testing.assert_allclose(got, want, rtol=1e-6)
    t = ticks.cpu().numpy().reshape(-1, 2)
    assert np.all(t > 0)


def test_mfma_rate_with_valu():
    require_gpu()
    sink = torch.full((2 * 512,), float("nan"), device="cuda")
    for valu in (1, 2, 3, 4, 6, 8):
        w4.mfma_rate(1, valu, 2, 4, sink)
        assert torch.isfinite(sink).all()
