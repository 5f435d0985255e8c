"""GPU parity: salient-channel selection and residual compensation against the
oracle (the DecDEC page's residual fetch for the channels with activation
outliers).

Selection is an index result and must be bit-exact (its order is unique).  The
correction is compared with the oracle's fp64 correction within the
row-relative tolerance, with the residual in pinned host memory (read by the
GPU over the host link) and in device memory."""
import numpy as np
import pytest
import torch

import bit_weight_quantized_amd as w4
import oracle as o
import workloads as wl
from gpu_helpers import TOL_ROW_REL_L2, announce, dev, host, require_gpu, row_rel_l2, upload_weights

pytestmark = pytest.mark.gpu


def pinned(a):
    t = torch.empty(a.shape, dtype=torch.float16, pin_memory=True)
    t.copy_(torch.from_numpy(np.ascontiguousarray(a)))
    return t


def residual_case(seed, M, K, N, G=128):
    w = wl.make_weight(seed, 0, N, K)
    x = wl.make_activations(seed, 0, M, K, outliers=True)
    codes, scale, zero = o.quantize_int4_asym(w, G)
    wd = o.dequant_int4_asym(codes, scale, zero, G)
    return x, codes, scale, zero, wd, o.residual_fp16(w, wd)


@pytest.mark.parametrize("M,K,k", [(1, 1, 1), (1, 8192, 64), (4, 8192, 82), (16, 1000, 1000), (32, 28672, 1024),
                                   (1, 28672, 287), (2, 32768, 5), (8, 4096, 0)])
def test_salient_select_matches_oracle(M, K, k):
    require_gpu()
    x = wl.make_activations(600 + K % 97, 0, M, K, outliers=True)
    announce("salient select", dict(M=M, K=K, k=k))
    got = host(w4.salient_select(dev(x), k))
    assert np.array_equal(got, o.salient_channels(x, k))


def test_salient_select_ties_and_zeros():
    """Integer activations with many equal scores, a zero channel block and
    negative zeros: the order among ties is by channel."""
    require_gpu()
    rng = np.random.default_rng(61)
    M, K = 3, 3000
    x = rng.integers(-6, 7, size=(M, K)).astype(np.float16)
    x[:, 100:400] = 0
    x[1, 500:510] = -0.0
    announce("salient select ties")
    for k in (1, 7, 513, 1024):
        got = host(w4.salient_select(dev(x), k))
        assert np.array_equal(got, o.salient_channels(x, k)), k
    # one score shared by every channel of the widest row: the ties fill
    # all 32 channel chunks and the picks are the lowest channels
    x = np.where(rng.integers(0, 2, size=(2, 32768)) == 1, 0.5, -0.5).astype(np.float16)
    for k in (1, 1000, 1024):
        got = host(w4.salient_select(dev(x), k))
        assert np.array_equal(got, o.salient_channels(x, k)), k


@pytest.mark.parametrize("where", ["pinned", "device"])
@pytest.mark.parametrize("M,K,N,k", [(1, 1024, 256, 11), (5, 2048, 1040, 40), (8, 512, 8, 512),
                                     (9, 1024, 520, 33), (32, 2048, 2048, 100)])
def test_residual_correction_matches_oracle(where, M, K, N, k):
    require_gpu()
    x, _, _, _, _, R = residual_case(610 + M, M, K, N)
    idx = o.salient_channels(x, k)
    ref = o.residual_correction(x, R, idx)
    r = pinned(R) if where == "pinned" else dev(R)
    y = torch.zeros((M, N), dtype=torch.float16, device="cuda")
    announce("residual correct", dict(where=where, M=M, K=K, N=N, k=k))
    w4.residual_correct(dev(x), r, dev(idx), y)
    torch.cuda.synchronize()
    assert row_rel_l2(host(y), ref) <= TOL_ROW_REL_L2


def test_residual_correction_skips_out_of_range_and_k0():
    require_gpu()
    M, K, N = 2, 256, 64
    x, _, _, _, _, R = residual_case(620, M, K, N)
    y0 = torch.randn((M, N), device="cuda").half()
    y = y0.clone()
    r = pinned(R)
    announce("residual correct k=0 and bad indices")
    w4.residual_correct(dev(x), r, torch.empty((0,), dtype=torch.int32, device="cuda"), y)
    torch.cuda.synchronize()
    assert torch.equal(y, y0)
    idx = np.array([5, -1, K, 7, 1 << 30], dtype=np.int32)
    w4.residual_correct(dev(x), r, dev(idx), y)
    ref = host(y0).astype(np.float64) + o.residual_correction(x, R, np.array([5, 7]))
    assert row_rel_l2(host(y), ref) <= TOL_ROW_REL_L2


def test_residual_correction_rejects_pageable_host_memory():
    require_gpu()
    M, K, N = 1, 128, 16
    x, _, _, _, _, R = residual_case(621, M, K, N)
    y = torch.zeros((M, N), dtype=torch.float16, device="cuda")
    r = torch.from_numpy(np.ascontiguousarray(R))  # pageable
    idx = dev(np.array([0, 1], dtype=np.int32))
    with pytest.raises(ValueError):
        w4.residual_correct(dev(x), r, idx, y)
    st = w4.lib().w4_residual_correct(w4._ptr(dev(x)), M, K, N, w4._ptr(r), w4._ptr(idx), 2, w4._ptr(y), None)
    assert st == -1
    torch.cuda.synchronize()  # nothing left behind on the stream


@pytest.mark.parametrize("M,K,N,k", [(1, 8192, 8192, 82), (16, 8192, 8192, 82), (1, 28672, 8192, 287)])
def test_gemv_then_correction_decode_layer(M, K, N, k):
    """The decode step as a whole: GEMV of the quantized layer, selection of the
    step's salient channels, correction from pinned host memory; against the
    oracle's quantized product plus its correction.  Full-size layers, output
    compared on sampled columns (the oracle quantizes only those rows)."""
    require_gpu()
    G = 128
    seed = 630 + M
    w = wl.make_weight(seed, 0, N, K)
    x = wl.make_activations(seed, 0, M, K, outliers=True)
    announce("decode + residual", dict(M=M, K=K, N=N, k=k))
    codes_d, scale_d, zero_d = w4.quantize(dev(w), G, w4.INT4_ASYM)
    packed = w4.pack(codes_d)
    cols = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(seed).choice(N, 96, replace=False)]))
    rc, rs, rz = o.quantize_int4_asym(w[cols], G)
    assert np.array_equal(host(codes_d[cols]), rc)
    wd = o.dequant_int4_asym(rc, rs, rz, G)
    R_cols = o.residual_fp16(w[cols], wd)  # [K][len(cols)]
    # the device's residual: the oracle's for the sampled columns; elsewhere
    # seeded values of the same size (those columns are not checked, and a full
    # fp64 quantization of the layer would take most of the test's time)
    R = (np.random.default_rng(seed + 1).standard_normal((K, N), dtype=np.float32) * 1e-3).astype(np.float16)
    R[:, cols] = R_cols
    xd = dev(x)
    y = w4.gemv(xd, packed, scale_d, zero_d, G, w4.INT4_ASYM)
    idx = w4.salient_select(xd, k)
    w4.residual_correct(xd, pinned(R), idx, y)
    torch.cuda.synchronize()
    idx_ref = o.salient_channels(x, k)
    assert np.array_equal(host(idx), idx_ref)
    ref = o.matmul_ref(x, wd) + o.residual_correction(x, R_cols, idx_ref)
    assert row_rel_l2(host(y)[:, cols], ref) <= TOL_ROW_REL_L2
    # the compensated product is closer to the unquantized one than the GEMV alone
    y_full = x.astype(np.float64) @ w[cols].astype(np.float64).T
    y_q = o.matmul_ref(x, wd)
    assert np.linalg.norm(host(y)[:, cols] - y_full) < np.linalg.norm(y_q - y_full)


@pytest.mark.parametrize("where", ["pinned", "device"])
@pytest.mark.parametrize("M,K,N,k", [(1, 1024, 256, 11), (5, 2048, 1040, 40), (8, 512, 8, 512),
                                     (9, 1024, 520, 33), (32, 2048, 2048, 100), (1, 8192, 8192, 82),
                                     (2, 32768, 1024, 1024), (3, 128, 8, 1), (4, 128, 64, 0)])
def test_salient_correct_equals_select_then_correct(where, M, K, N, k):
    """The one-launch step picks the same channels (in the same order) and
    leaves the same y bits as the two calls; y also matches the oracle."""
    require_gpu()
    x, _, _, _, _, R = residual_case(640 + M, M, K, N)
    r = pinned(R) if where == "pinned" else dev(R)
    xd = dev(x)
    y0 = torch.randn((M, N), device="cuda").half()
    y_two, y_one = y0.clone(), y0.clone()
    announce("salient correct", dict(where=where, M=M, K=K, N=N, k=k))
    idx_two = w4.salient_select(xd, k)
    w4.residual_correct(xd, r, idx_two, y_two)
    idx_one = torch.full((k,), -7, dtype=torch.int32, device="cuda")
    w4.salient_correct(xd, r, k, y_one, idx=idx_one)
    torch.cuda.synchronize()
    assert torch.equal(idx_one, idx_two)
    assert torch.equal(y_one, y_two)
    idx_ref = o.salient_channels(x, k)
    assert np.array_equal(host(idx_one), idx_ref)
    ref = host(y0).astype(np.float64) + o.residual_correction(x, R, idx_ref)
    assert row_rel_l2(host(y_one), ref) <= TOL_ROW_REL_L2


@pytest.mark.parametrize("where", ["pinned", "device"])
@pytest.mark.parametrize("M,K,N,k", [(1, 1024, 256, 11), (5, 2048, 1040, 40), (9, 1024, 520, 33),
                                     (32, 2048, 2048, 100), (1, 8192, 8192, 82), (2, 256, 64, 0)])
def test_correction_f32_then_apply_equals_correction(where, M, K, N, k):
    """The correction stored in fp32 matches the oracle (every element
    written: c starts as NaN; k = 0 gives zeros), and adding it to y leaves
    the same bits as the correction that adds to y itself."""
    require_gpu()
    x, _, _, _, _, R = residual_case(660 + M, M, K, N)
    idx = o.salient_channels(x, k)
    r = pinned(R) if where == "pinned" else dev(R)
    xd, idxd = dev(x), dev(idx)
    y0 = torch.randn((M, N), device="cuda").half()
    y_one, y_two = y0.clone(), y0.clone()
    c = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    announce("residual correct f32 + apply", dict(where=where, M=M, K=K, N=N, k=k))
    w4.residual_correct(xd, r, idxd, y_one)
    w4.residual_correct_f32(xd, r, idxd, c)
    w4.residual_apply(c, y_two)
    torch.cuda.synchronize()
    ref = o.residual_correction(x, R, idx)
    if k == 0:
        assert torch.count_nonzero(c).item() == 0
    else:
        assert row_rel_l2(host(c), ref) <= TOL_ROW_REL_L2
    assert torch.equal(y_two, y_one)


@pytest.mark.parametrize("where", ["pinned", "device"])
@pytest.mark.parametrize("M,K,N,k", [(1, 1024, 256, 11), (9, 1024, 520, 33), (32, 2048, 2048, 100),
                                     (1, 8192, 8192, 82), (2, 32768, 1024, 1024), (3, 128, 8, 1), (4, 128, 64, 0)])
def test_salient_correct_f32_equals_select_then_correct_f32(where, M, K, N, k):
    """The one-launch selection with the fp32 correction picks the same
    channels and stores the same c bits as the two calls (k = 0: zeros)."""
    require_gpu()
    x, _, _, _, _, R = residual_case(680 + M, M, K, N)
    r = pinned(R) if where == "pinned" else dev(R)
    xd = dev(x)
    announce("salient correct f32", dict(where=where, M=M, K=K, N=N, k=k))
    idx_two = w4.salient_select(xd, k)
    c_two = w4.residual_correct_f32(xd, r, idx_two, N=N)
    idx_one = torch.full((k,), -7, dtype=torch.int32, device="cuda")
    c_one = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    w4.salient_correct_f32(xd, r, k, c_one, idx=idx_one)
    torch.cuda.synchronize()
    assert torch.equal(idx_one, idx_two)
    assert torch.equal(c_one, c_two)
    assert np.array_equal(host(idx_one), o.salient_channels(x, k))
    if k == 0:
        assert torch.count_nonzero(c_one).item() == 0


@pytest.mark.parametrize("side_launches", [2, 1])
def test_overlapped_step_equals_serial_step(side_launches):
    """The decode step with the residual work beside the GEMV (selection and
    fp32 correction on a second stream, as two launches or one, then the
    apply after both) gives the serial step's picks and output bits: eagerly,
    and over graph replays of the forked schedule."""
    require_gpu()
    M, K, N, k, G = 1, 8192, 8192, 82, 128
    w = wl.make_weight(670, 0, N, K)
    x = wl.make_activations(670, 0, M, K, outliers=True)
    R = (np.random.default_rng(671).standard_normal((K, N), dtype=np.float32) * 1e-3).astype(np.float16)
    announce("overlapped residual step", dict(M=M, K=K, N=N, k=k, side_launches=side_launches))
    codes, scale, zero = w4.quantize(dev(w), G, w4.INT4_ASYM)
    packed = w4.pack(codes)
    xd, r = dev(x), pinned(R)
    y_ser = torch.empty((M, N), dtype=torch.float16, device="cuda")
    idx_ser = torch.empty((k,), dtype=torch.int32, device="cuda")
    w4.gemv(xd, packed, scale, zero, G, w4.INT4_ASYM, out=y_ser)
    w4.salient_select(xd, k, out=idx_ser)
    w4.residual_correct(xd, r, idx_ser, y_ser)
    torch.cuda.synchronize()

    y_ovl = torch.empty_like(y_ser)
    idx_ovl = torch.empty_like(idx_ser)
    c = torch.empty((M, N), dtype=torch.float32, device="cuda")
    main, side = torch.cuda.Stream(), torch.cuda.Stream()

    def step():
        side.wait_stream(main)
        with torch.cuda.stream(side):
            if side_launches == 2:
                w4.salient_select(xd, k, out=idx_ovl, stream=side)
                w4.residual_correct_f32(xd, r, idx_ovl, c, stream=side)
            else:
                w4.salient_correct_f32(xd, r, k, c, idx=idx_ovl, stream=side)
        w4.gemv(xd, packed, scale, zero, G, w4.INT4_ASYM, out=y_ovl, stream=main)
        main.wait_stream(side)
        w4.residual_apply(c, y_ovl, stream=main)

    with torch.cuda.stream(main):
        step()
    torch.cuda.synchronize()
    assert torch.equal(idx_ovl, idx_ser)
    assert torch.equal(y_ovl, y_ser)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=main):
        step()
    torch.cuda.synchronize()
    for _ in range(3):
        y_ovl.zero_()
        idx_ovl.zero_()
        c.zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(main):
            g.replay()
        main.synchronize()
        assert torch.equal(idx_ovl, idx_ser)
        assert torch.equal(y_ovl, y_ser)
