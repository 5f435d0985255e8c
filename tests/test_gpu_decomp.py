"""GPU parity: w4_gemm_decomp (Multi-Scale Dequant) against the fp64 oracle.

The int8 slices, the per-token scales and the per-group int32 accumulators are
integer (or fp32 decision) results and must be bit-exact; the fp16 output is
compared with the oracle's recombination of its own accumulators within the
row-relative tolerance."""
import numpy as np
import pytest
import torch

import bit_weight_quantized_amd as w4
import oracle as o
import workloads as wl
from gpu_helpers import (TOL_ROW_REL_L2, announce, assert_elementwise, dev, host, oracle_weights,
                         require_gpu, row_rel_l2, upload_weights)

pytestmark = pytest.mark.gpu


def run_decomp(x, codes, scale, zero, G, nslices, with_acc=True):
    M, K = x.shape
    N = codes.shape[0]
    packed, sc, zc = upload_weights(codes, scale, zero)
    sl = torch.empty((nslices, M, K), dtype=torch.int8, device="cuda")
    ts = torch.empty((nslices, M), dtype=torch.float32, device="cuda")
    acc = torch.empty((nslices, M, K // G, N), dtype=torch.int32, device="cuda") if with_acc else None
    y, _, _, _ = w4.gemm_decomp(dev(x), packed, sc, zc, G, nslices, slices_out=sl, tok_scale_out=ts,
                                acc_out=acc)
    return host(y), host(sl), host(ts), (host(acc) if with_acc else None)


@pytest.mark.parametrize("G", [128, 64])
@pytest.mark.parametrize("nslices", [2, 1, 3])
@pytest.mark.parametrize("M,K,N", [(1, 128, 16), (5, 640, 48), (130, 1024, 272), (257, 512, 144),
                                   (64, 2048, 256)])
def test_decomp_small(G, nslices, M, K, N):
    if K % G:
        pytest.skip("K not a multiple of G")
    require_gpu()
    w = wl.make_weight(300 + M, 0, N, K)
    x = wl.make_activations(300 + M, 0, M, K)
    codes, scale, zero = o.quantize_int4_asym(w, G)
    announce("decomp", dict(G=G, nslices=nslices, M=M, K=K, N=N))
    y, sl, ts, acc = run_decomp(x, codes, scale, zero, G, nslices)
    A, S = o.decompose_activations(x, nslices)
    assert np.array_equal(sl, A)
    assert np.array_equal(ts.view(np.uint32), S.view(np.uint32))
    D = o.msd_accumulators(A, codes, zero, G)
    assert np.array_equal(acc.astype(np.int64), D)
    assert row_rel_l2(y, o.msd_result(S, D, scale)) <= TOL_ROW_REL_L2


def test_decomp_degenerate_rows():
    """A zero token row (both scales 0, output exactly 0); a row of integers
    with max |x| = 127 (first scale exactly 1, residual 0, second slice all
    zero); a row with one non-zero entry; a single huge outlier."""
    require_gpu()
    M, K, N, G = 6, 256, 64, 128
    x = wl.make_activations(13, 0, M, K)
    x[0] = 0
    x[1] = np.float16(np.random.default_rng(13).integers(-127, 128, K))
    x[1, 5] = 127
    x[2] = 0
    x[2, 77] = -3.5
    x[3, 100] = 30000
    w = wl.make_weight(13, 0, N, K)
    codes, scale, zero = o.quantize_int4_asym(w, G)
    announce("decomp degenerate")
    y, sl, ts, acc = run_decomp(x, codes, scale, zero, G, 2)
    A, S = o.decompose_activations(x, 2)
    assert S[0, 1] == 1.0 and S[1, 1] == 0.0 and S[0, 0] == 0.0
    assert np.array_equal(sl, A)
    assert np.array_equal(ts.view(np.uint32), S.view(np.uint32))
    D = o.msd_accumulators(A, codes, zero, G)
    assert np.array_equal(acc.astype(np.int64), D)
    assert np.all(y[0] == 0)
    ref = o.msd_result(S, D, scale)
    assert row_rel_l2(y[1:], ref[1:]) <= TOL_ROW_REL_L2


def test_decomp_repeatable_without_optional_outputs():
    """The workspace-only call (no optional outputs) gives the same bits as
    the call that returns slices and accumulators, twice."""
    require_gpu()
    M, K, N, G = 200, 1024, 192, 128
    x = wl.make_activations(14, 0, M, K)
    codes, scale, zero = o.quantize_int4_asym(wl.make_weight(14, 0, N, K), G)
    packed, sc, zc = upload_weights(codes, scale, zero)
    xd = dev(x)
    ws = torch.empty(w4.workspace_bytes(w4.OP_GEMM_DECOMP, M, K, N, G, 2), dtype=torch.uint8, device="cuda")
    announce("decomp repeat")
    a = host(w4.gemm_decomp(xd, packed, sc, zc, G, 2, workspace=ws))
    b = host(w4.gemm_decomp(xd, packed, sc, zc, G, 2, workspace=ws))
    c, _, _, _ = run_decomp(x, codes, scale, zero, G, 2)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    assert np.array_equal(a.view(np.uint16), c.view(np.uint16))


def test_decomp_rejects_nf4():
    require_gpu()
    K, N, G = 256, 32, 64
    codes, absmax = o.quantize_nf4(wl.make_weight(15, 0, N, K), G)
    packed, sc, _ = upload_weights(codes, absmax, None)
    x = dev(wl.make_activations(15, 0, 2, K))
    with pytest.raises(w4.W4Error) as e:
        w4.gemm_decomp(x, packed, sc, None, G, 2)
    assert e.value.status == -2


@pytest.mark.parametrize("nslices", [2, 1, 3])
def test_decomp_prefill_m2048_k5120_n25600(nslices):
    """Full prefill shape: slices and scales bit-exact over the whole input;
    outputs compared on sampled columns."""
    M, K, N, G = 2048, 5120, 25600, 128
    w = wl.make_weight(4, 0, N, K)
    x = wl.make_activations(4, 0, M, K)
    announce("decomp full quantize")
    codes, scale, zero = w4.quantize(dev(w), G, w4.INT4_ASYM)
    packed = w4.pack(codes)
    sl = torch.empty((nslices, M, K), dtype=torch.int8, device="cuda")
    ts = torch.empty((nslices, M), dtype=torch.float32, device="cuda")
    announce("decomp prefill", dict(nslices=nslices, M=M, K=K, N=N))
    y, _, _, _ = w4.gemm_decomp(dev(x), packed, scale, zero, G, nslices, slices_out=sl, tok_scale_out=ts)
    y = host(y)
    A, S = o.decompose_activations(x, nslices)
    assert np.array_equal(host(sl), A)
    assert np.array_equal(host(ts).view(np.uint32), S.view(np.uint32))
    rows = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(41).choice(N, 64, replace=False)]))
    rc, rs, rz = o.quantize_int4_asym(w[rows], G)
    assert np.array_equal(host(codes[rows]), rc)
    ref = o.msd_result(S, o.msd_accumulators(A, rc, rz, G), rs)
    assert row_rel_l2(y[:, rows], ref) <= TOL_ROW_REL_L2


# ------------------------------------------------------------ fixed ratio
def run_fixed(x, codes, scale, zero, G, with_acc=True, workspace=None):
    M, K = x.shape
    N = codes.shape[0]
    packed, sc, zc = upload_weights(codes, scale, zero)
    sl = torch.empty((2, M, K), dtype=torch.int8, device="cuda")
    ts = torch.empty((2, M), dtype=torch.float32, device="cuda")
    acc = torch.empty((2, M, K // G, N), dtype=torch.int32, device="cuda") if with_acc else None
    y, _, _, _ = w4.gemm_decomp_fixed(dev(x), packed, sc, zc, G, slices_out=sl, tok_scale_out=ts, acc_out=acc,
                                      workspace=workspace)
    return host(y), host(sl), host(ts), (host(acc) if with_acc else None)


@pytest.mark.parametrize("G", [128, 64])
@pytest.mark.parametrize("M,K,N", [(1, 128, 16), (5, 640, 48), (130, 1024, 272), (257, 512, 144),
                                   (64, 2048, 256)])
def test_decomp_fixed_small(G, M, K, N):
    if K % G:
        pytest.skip("K not a multiple of G")
    require_gpu()
    w = wl.make_weight(310 + M, 0, N, K)
    x = wl.make_activations(310 + M, 0, M, K, outliers=True)
    codes, scale, zero = o.quantize_int4_asym(w, G)
    announce("decomp fixed", dict(G=G, M=M, K=K, N=N))
    y, sl, ts, acc = run_fixed(x, codes, scale, zero, G)
    A, S = o.decompose_fixed_ratio(x)
    assert np.array_equal(sl, A)
    assert np.array_equal(ts.view(np.uint32), S.view(np.uint32))
    D = o.msd_accumulators(A, codes, zero, G)
    assert np.array_equal(acc.astype(np.int64), D)
    assert row_rel_l2(y, o.msd_fixed_result(S[0], D, scale)) <= TOL_ROW_REL_L2


def test_decomp_fixed_degenerate_rows_and_repeat():
    """Zero row (output exactly 0), integer row on the first grid (second
    slice zero), one non-zero entry, a huge outlier; the workspace-only call
    gives the same bits as the call with every optional output."""
    require_gpu()
    M, K, N, G = 6, 512, 64, 64
    x = wl.make_activations(16, 0, M, K)
    x[0] = 0
    x[1] = np.float16(np.random.default_rng(16).integers(-127, 128, K))
    x[1, 5] = 127
    x[2] = 0
    x[2, 77] = -3.5
    x[3, 100] = 30000
    codes, scale, zero = o.quantize_int4_asym(wl.make_weight(16, 0, N, K), G)
    announce("decomp fixed degenerate")
    y, sl, ts, acc = run_fixed(x, codes, scale, zero, G)
    A, S = o.decompose_fixed_ratio(x)
    assert S[0, 1] == 1.0 and np.all(A[1, 1] == 0) and S[0, 0] == 0.0
    assert np.array_equal(sl, A)
    assert np.array_equal(ts.view(np.uint32), S.view(np.uint32))
    D = o.msd_accumulators(A, codes, zero, G)
    assert np.array_equal(acc.astype(np.int64), D)
    assert np.all(y[0] == 0)
    assert row_rel_l2(y[1:], o.msd_fixed_result(S[0], D, scale)[1:]) <= TOL_ROW_REL_L2
    packed, sc, zc = upload_weights(codes, scale, zero)
    ws = torch.empty(w4.workspace_bytes(w4.OP_GEMM_DECOMP, M, K, N, G, 2), dtype=torch.uint8, device="cuda")
    a = host(w4.gemm_decomp_fixed(dev(x), packed, sc, zc, G, workspace=ws))
    b = host(w4.gemm_decomp_fixed(dev(x), packed, sc, zc, G, workspace=ws))
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    assert np.array_equal(a.view(np.uint16), y.view(np.uint16))


def test_decomp_fixed_rejects_nf4():
    require_gpu()
    K, N, G = 256, 32, 64
    codes, absmax = o.quantize_nf4(wl.make_weight(17, 0, N, K), G)
    packed, sc, _ = upload_weights(codes, absmax, None)
    with pytest.raises(w4.W4Error) as e:
        w4.gemm_decomp_fixed(dev(wl.make_activations(17, 0, 2, K)), packed, sc, None, G)
    assert e.value.status == -2


def test_decomp_fixed_prefill_m2048_k5120_n25600():
    """Full prefill shape: slices and scales bit-exact over the whole input;
    outputs compared on sampled columns."""
    M, K, N, G = 2048, 5120, 25600, 128
    w = wl.make_weight(4, 0, N, K)
    x = wl.make_activations(4, 0, M, K)
    announce("decomp fixed full quantize")
    codes, scale, zero = w4.quantize(dev(w), G, w4.INT4_ASYM)
    packed = w4.pack(codes)
    sl = torch.empty((2, M, K), dtype=torch.int8, device="cuda")
    ts = torch.empty((2, M), dtype=torch.float32, device="cuda")
    announce("decomp fixed prefill", dict(M=M, K=K, N=N))
    y, _, _, _ = w4.gemm_decomp_fixed(dev(x), packed, scale, zero, G, slices_out=sl, tok_scale_out=ts)
    y = host(y)
    A, S = o.decompose_fixed_ratio(x)
    assert np.array_equal(host(sl), A)
    assert np.array_equal(host(ts).view(np.uint32), S.view(np.uint32))
    rows = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(42).choice(N, 64, replace=False)]))
    rc, rs, rz = o.quantize_int4_asym(w[rows], G)
    assert np.array_equal(host(codes[rows]), rc)
    ref = o.msd_fixed_result(S[0], o.msd_accumulators(A, rc, rz, G), rs)
    assert row_rel_l2(y[:, rows], ref) <= TOL_ROW_REL_L2



# ------------------------------------------------- decoder layer at M = 256
# The 70B-style layer's products (hidden 8192, intermediate 28672, 8 KV heads
# of 128): index in the layer order q, k, v, o, gate, up, down.
LAYER_INDEX = {"q": 0, "k": 1, "v": 2, "o": 3, "gate": 4, "up": 5, "down": 6}


@pytest.mark.parametrize("fixed", [False, True], ids=["adaptive", "fixed"])
@pytest.mark.parametrize("name,K,N", [("q", 8192, 8192), ("k", 8192, 1024), ("gate", 8192, 28672),
                                      ("down", 28672, 8192)])
def test_decomp_decoder_layer_m256(name, K, N, fixed):
    """Two-slice MSD (adaptive and fixed-ratio scales) on decoder-layer
    products at M = 256: the slices and token scales bit-exact over the whole
    input (these shapes take the 1024-thread decomposition, which holds rows
    of up to 32768 positions in registers), the output on sampled columns
    (including the split-K tail's, when the plan has one)."""
    M, G = 256, 128
    w = wl.make_weight(5, LAYER_INDEX[name], N, K)
    x = wl.make_activations(5, 0 if K == 8192 else 6, M, K)
    announce("decomp layer quantize", dict(name=name, K=K, N=N))
    codes, scale, zero = w4.quantize(dev(w), G, w4.INT4_ASYM)
    packed = w4.pack(codes)
    sl = torch.empty((2, M, K), dtype=torch.int8, device="cuda")
    ts = torch.empty((2, M), dtype=torch.float32, device="cuda")
    announce("decomp layer", dict(name=name, M=M, K=K, N=N, fixed=fixed))
    if fixed:
        y, _, _, _ = w4.gemm_decomp_fixed(dev(x), packed, scale, zero, G, slices_out=sl, tok_scale_out=ts)
        A, S = o.decompose_fixed_ratio(x)
    else:
        y, _, _, _ = w4.gemm_decomp(dev(x), packed, scale, zero, G, 2, slices_out=sl, tok_scale_out=ts)
        A, S = o.decompose_activations(x, 2)
    y = host(y)
    assert np.array_equal(host(sl), A)
    assert np.array_equal(host(ts).view(np.uint32), S.view(np.uint32))
    rows = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(43).choice(N, 48, replace=False)]))
    rc, rs, rz = o.quantize_int4_asym(w[rows], G)
    assert np.array_equal(host(codes[rows]), rc)
    D = o.msd_accumulators(A, rc, rz, G)
    ref = o.msd_fixed_result(S[0], D, rs) if fixed else o.msd_result(S, D, rs)
    assert row_rel_l2(y[:, rows], ref) <= TOL_ROW_REL_L2
    assert_elementwise(y[:, rows], ref)


@pytest.mark.parametrize("nslices", [1, 3])
@pytest.mark.parametrize("K", [8192, 28672])
def test_decomp_slices_m256_long_rows(nslices, K):
    """One and three slices at M = 256 on the decoder layer's row lengths:
    slices and scales bit-exact, every output within tolerance."""
    M, N, G = 256, 256, 128
    x = wl.make_activations(5, 0 if K == 8192 else 6, M, K)
    codes, scale, zero = o.quantize_int4_asym(wl.make_weight(320, 0, N, K), G)
    announce("decomp long rows", dict(nslices=nslices, M=M, K=K, N=N))
    y, sl, ts, _ = run_decomp(x, codes, scale, zero, G, nslices, with_acc=False)
    A, S = o.decompose_activations(x, nslices)
    assert np.array_equal(sl, A)
    assert np.array_equal(ts.view(np.uint32), S.view(np.uint32))
    ref = o.msd_result(S, o.msd_accumulators(A, codes, zero, G), scale)
    assert row_rel_l2(y, ref) <= TOL_ROW_REL_L2
    assert_elementwise(y, ref)


@pytest.mark.parametrize("fixed", [False, True], ids=["adaptive", "fixed"])
def test_decomp_exact_half_integer_quotients(fixed):
    """Quotients x / s that are exact half-integers take the division itself
    (round half to even); quotients a few ulps from one do not round
    differently.  Rows: s = 1 (max |x| = 127) with x = k + 1/2; s = 2^-3 with
    x = (k + 1/2) / 8; s = 2^5 with x = 32 (k + 1/2); and rows whose values
    sit one fp16 ulp beside those ties.  Slices and scales bit-exact against
    the oracle's fp64 division."""
    require_gpu()
    K, N, G = 512, 64, 128
    ks = np.arange(-127, 127, dtype=np.float64)
    rows = []
    for scale_ in (1.0, 0.125, 32.0):
        base = np.resize((ks + 0.5) * scale_, K)
        base[0] = 127 * scale_  # the row maximum fixes s = scale_
        rows.append(base)
        near = base.astype(np.float16)
        rows.append(np.nextafter(near, np.float16(np.inf)).astype(np.float64))
        rows.append(np.nextafter(near, np.float16(-np.inf)).astype(np.float64))
    x = np.array(rows, dtype=np.float16)
    M = x.shape[0]
    w = wl.make_weight(340, 0, N, K)
    codes, scale, zero = o.quantize_int4_asym(w, G)
    announce("decomp ties", dict(fixed=fixed, M=M, K=K))
    if fixed:
        y, sl, ts, _ = run_fixed(x, codes, scale, zero, G, with_acc=False)
        A, S = o.decompose_fixed_ratio(x)
    else:
        y, sl, ts, _ = run_decomp(x, codes, scale, zero, G, 2, with_acc=False)
        A, S = o.decompose_activations(x, 2)
    assert np.array_equal(sl, A)
    assert np.array_equal(ts.view(np.uint32), S.view(np.uint32))
    assert S[0, 0] == 1.0 and S[0, 3] == 0.125 and S[0, 6] == 32.0
