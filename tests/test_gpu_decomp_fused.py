"""GPU parity: w4_gemm_decomp_fixed_fused (the fixed-ratio Multi-Scale Dequant
product with the decomposition inside the product's K loop).

Its slices exist only in LDS, so the checks are: the token scales bit-exact
against the fp64 oracle; y bit-identical to w4_gemm_decomp_fixed's y on every
element (that path's slices are bit-exact against the oracle and its products
are accumulated in the same order, so any differing code shows up in y); and
y within the tolerance of the oracle's own result."""
import numpy as np
import pytest
import torch

import bit_weight_quantized_amd as w4
import oracle as o
import workloads as wl
from gpu_helpers import (TOL_ROW_REL_L2, announce, assert_elementwise, dev, host, require_gpu, row_rel_l2,
                         upload_weights)

pytestmark = pytest.mark.gpu


def run_both(x, packed, sc, zc, G):
    """(fused y, fused scales, pre-pass y, pre-pass slices, pre-pass scales)."""
    M, K = x.shape
    xd = dev(x) if isinstance(x, np.ndarray) else x
    ts_f = torch.empty((2, M), dtype=torch.float32, device="cuda")
    y_f, _ = w4.gemm_decomp_fixed_fused(xd, packed, sc, zc, G, tok_scale_out=ts_f)
    sl = torch.empty((2, M, K), dtype=torch.int8, device="cuda")
    ts = torch.empty((2, M), dtype=torch.float32, device="cuda")
    y, _, _, _ = w4.gemm_decomp_fixed(xd, packed, sc, zc, G, slices_out=sl, tok_scale_out=ts)
    return host(y_f), host(ts_f), host(y), host(sl), host(ts)


def check_against_prepass_and_oracle(x, y_f, ts_f, y, sl, ts):
    A, S = o.decompose_fixed_ratio(x)
    assert np.array_equal(ts_f.view(np.uint32), S.view(np.uint32))
    assert np.array_equal(ts.view(np.uint32), S.view(np.uint32))
    assert np.array_equal(sl, A)
    assert np.array_equal(y_f.view(np.uint16), y.view(np.uint16))
    return A, S


@pytest.mark.parametrize("G", [128, 64])
@pytest.mark.parametrize("M,K,N", [(1, 128, 16), (5, 640, 48), (130, 1024, 272), (257, 512, 144),
                                   (64, 2048, 256), (300, 384, 528)])
def test_fused_small(G, M, K, N):
    """Several token tiles and weight-column tiles with ragged edges (M, N not
    multiples of the 128/64 x 256 tile), one to sixteen K steps."""
    if K % G:
        pytest.skip("K not a multiple of G")
    require_gpu()
    w = wl.make_weight(360 + M, 0, N, K)
    x = wl.make_activations(360 + M, 0, M, K, outliers=True)
    codes, scale, zero = o.quantize_int4_asym(w, G)
    packed, sc, zc = upload_weights(codes, scale, zero)
    announce("fused small", dict(G=G, M=M, K=K, N=N))
    y_f, ts_f, y, sl, ts = run_both(x, packed, sc, zc, G)
    A, S = check_against_prepass_and_oracle(x, y_f, ts_f, y, sl, ts)
    ref = o.msd_fixed_result(S[0], o.msd_accumulators(A, codes, zero, G), scale)
    assert row_rel_l2(y_f, ref) <= TOL_ROW_REL_L2
    assert_elementwise(y_f, ref)


def tie_rows(K):
    """Rows whose quotients sit exactly on, or one fp16 ulp beside, the
    half-integers of the first slice (s_1 = 1, 2^-3, 2^5) and of the second
    (x = s_1 (q + h / 254) for half-integers h)."""
    ks = np.arange(-127, 127, dtype=np.float64)
    rows = []
    for scale_ in (1.0, 0.125, 32.0):
        base = np.resize((ks + 0.5) * scale_, K)
        base[0] = 127 * scale_
        rows.append(base)
        near = base.astype(np.float16)
        rows.append(np.nextafter(near, np.float16(np.inf)).astype(np.float64))
        rows.append(np.nextafter(near, np.float16(-np.inf)).astype(np.float64))
    rng = np.random.default_rng(361)
    for scale_ in (1.0, 0.25):
        q = rng.integers(-60, 60, K)
        h = rng.integers(-126, 126, K) + 0.5
        base = scale_ * (q + h / 254.0)
        base[0] = 127 * scale_
        rows.append(base)
        near = base.astype(np.float16)
        rows.append(np.nextafter(near, np.float16(np.inf)).astype(np.float64))
    return np.array(rows, dtype=np.float16)


def test_fused_half_integer_quotients():
    """The rare exact decisions: quotients on or next to half-integers in
    either slice give the fp64 decomposition's codes."""
    require_gpu()
    K, N, G = 512, 256, 128
    x = tie_rows(K)
    codes, scale, zero = o.quantize_int4_asym(wl.make_weight(362, 0, N, K), G)
    packed, sc, zc = upload_weights(codes, scale, zero)
    announce("fused ties", dict(M=x.shape[0], K=K, N=N))
    y_f, ts_f, y, sl, ts = run_both(x, packed, sc, zc, G)
    A, S = check_against_prepass_and_oracle(x, y_f, ts_f, y, sl, ts)
    assert S[0, 0] == 1.0 and S[0, 3] == 0.125 and S[0, 6] == 32.0
    ref = o.msd_fixed_result(S[0], o.msd_accumulators(A, codes, zero, G), scale)
    assert row_rel_l2(y_f, ref) <= TOL_ROW_REL_L2


def test_fused_degenerate_rows_and_repeat():
    """Zero row (output exactly 0), an integer row on the first grid, a single
    non-zero entry, a huge outlier; two calls give the same bits."""
    require_gpu()
    M, K, N, G = 6, 512, 64, 64
    x = wl.make_activations(363, 0, M, K)
    x[0] = 0
    x[1] = np.float16(np.random.default_rng(363).integers(-127, 128, K))
    x[1, 5] = 127
    x[2] = 0
    x[2, 77] = -3.5
    x[3, 100] = 30000
    codes, scale, zero = o.quantize_int4_asym(wl.make_weight(363, 0, N, K), G)
    packed, sc, zc = upload_weights(codes, scale, zero)
    announce("fused degenerate")
    y_f, ts_f, y, sl, ts = run_both(x, packed, sc, zc, G)
    check_against_prepass_and_oracle(x, y_f, ts_f, y, sl, ts)
    assert np.all(y_f[0] == 0)
    ws = torch.empty(w4.workspace_bytes(w4.OP_GEMM_DECOMP_FUSED, M, K, N, G, 0), dtype=torch.uint8, device="cuda")
    a = host(w4.gemm_decomp_fixed_fused(dev(x), packed, sc, zc, G, workspace=ws))
    b = host(w4.gemm_decomp_fixed_fused(dev(x), packed, sc, zc, G, workspace=ws))
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    assert np.array_equal(a.view(np.uint16), y_f.view(np.uint16))


def test_fused_rejects_nf4():
    require_gpu()
    K, N, G = 256, 32, 64
    codes, absmax = o.quantize_nf4(wl.make_weight(364, 0, N, K), G)
    packed, sc, _ = upload_weights(codes, absmax, None)
    with pytest.raises(w4.W4Error) as e:
        w4.gemm_decomp_fixed_fused(dev(wl.make_activations(364, 0, 2, K)), packed, sc, None, G)
    assert e.value.status == -2


def test_fused_prefill_m2048_k5120_n25600():
    """The full prefill shape: y bit-identical to the pre-pass path on every
    element, token scales bit-exact, sampled columns against the oracle."""
    M, K, N, G = 2048, 5120, 25600, 128
    w = wl.make_weight(4, 0, N, K)
    x = wl.make_activations(4, 0, M, K)
    announce("fused full quantize")
    codes, scale, zero = w4.quantize(dev(w), G, w4.INT4_ASYM)
    packed = w4.pack(codes)
    announce("fused prefill", dict(M=M, K=K, N=N))
    y_f, ts_f, y, sl, ts = run_both(x, packed, scale, zero, G)
    A, S = check_against_prepass_and_oracle(x, y_f, ts_f, y, sl, ts)
    rows = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(44).choice(N, 48, replace=False)]))
    rc, rs, rz = o.quantize_int4_asym(w[rows], G)
    ref = o.msd_fixed_result(S[0], o.msd_accumulators(A, rc, rz, G), rs)
    assert row_rel_l2(y_f[:, rows], ref) <= TOL_ROW_REL_L2
    assert_elementwise(y_f[:, rows], ref)


LAYER_INDEX = {"q": 0, "k": 1, "v": 2, "o": 3, "gate": 4, "up": 5, "down": 6}


@pytest.mark.parametrize("name,K,N", [("q", 8192, 8192), ("k", 8192, 1024), ("gate", 8192, 28672),
                                      ("down", 28672, 8192)])
def test_fused_decoder_layer_m256(name, K, N):
    """Decoder-layer products at M = 256 (their plans split the left-over
    tiles over K): y bit-identical to the pre-pass path."""
    M, G = 256, 128
    w = wl.make_weight(5, LAYER_INDEX[name], N, K)
    x = wl.make_activations(5, 0 if K == 8192 else 6, M, K)
    announce("fused layer quantize", dict(name=name, K=K, N=N))
    codes, scale, zero = w4.quantize(dev(w), G, w4.INT4_ASYM)
    packed = w4.pack(codes)
    announce("fused layer", dict(name=name, M=M, K=K, N=N))
    y_f, ts_f, y, sl, ts = run_both(x, packed, scale, zero, G)
    A, S = check_against_prepass_and_oracle(x, y_f, ts_f, y, sl, ts)
    rows = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(45).choice(N, 32, replace=False)]))
    rc, rs, rz = o.quantize_int4_asym(w[rows], G)
    ref = o.msd_fixed_result(S[0], o.msd_accumulators(A, rc, rz, G), rs)
    assert_elementwise(y_f[:, rows], ref)
