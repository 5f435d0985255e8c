"""GPU parity: w4_gemv against the fp64 oracle.

Small shapes use oracle-quantized, oracle-packed weights uploaded as is, and
compare every output.  Full-size shapes (the decode and MLP layers) run the
whole GPU pipeline and compare a sample of output columns whose weight rows
the oracle quantizes itself from the same seeded weights."""
import numpy as np
import pytest
import torch

import bit_weight_quantized_amd as w4
import oracle as o
import workloads as wl
from gpu_helpers import (TOL_ROW_REL_L2, announce, assert_elementwise, dev, host, oracle_weights, require_gpu,
                         row_rel_l2, upload_weights)

pytestmark = pytest.mark.gpu

FMTS = [(o.FMT_INT4_ASYM, 128), (o.FMT_INT4_ASYM, 64), (o.FMT_NF4, 64), (o.FMT_NF4, 128)]


def run_small(fmt, G, M, K, N, seed, outliers=True):
    w = wl.make_weight(seed, 0, N, K)
    x = wl.make_activations(seed, 0, M, K, outliers=outliers)
    codes, scale, zero = oracle_weights(fmt, w, G)
    packed, sc, zc = upload_weights(codes, scale, zero)
    announce("gemv", dict(fmt=fmt, G=G, M=M, K=K, N=N, seed=seed))
    y = w4.gemv(dev(x), packed, sc, zc, G, fmt)
    torch.cuda.synchronize()
    y_ref = o.matmul_ref(x, o.dequant(fmt, codes, scale, zero, G))
    return host(y), y_ref


@pytest.mark.parametrize("fmt,G", FMTS)
@pytest.mark.parametrize("M", [1, 2, 4, 5, 16, 17, 32])
@pytest.mark.parametrize("K,N", [(128, 16), (640, 48), (1024, 1040), (2048, 256)])
def test_gemv_small(fmt, G, M, K, N):
    if K % G:
        pytest.skip("K not a multiple of G")
    y, y_ref = run_small(fmt, G, M, K, N, seed=100 + M)
    assert y.shape == (M, N)
    err = row_rel_l2(y, y_ref)
    assert err <= TOL_ROW_REL_L2, err
    assert_elementwise(y, y_ref)


@pytest.mark.parametrize("nwr,nwk,s", [(1, 1, 1), (1, 4, 1), (2, 3, 1), (4, 2, 1), (1, 8, 1), (1, 2, 3),
                                       (2, 2, 5), (1, 1, 12), (8, 1, 2), (4, 1, 4), (1, 5, 3), (2, 4, 2),
                                       (1, 6, 1), (2, 1, 7)])
def test_gemv_launch_variants_agree(monkeypatch, nwr, nwk, s):
    """Every work split (row waves, K waves, K slices over workgroups) stays
    within tolerance of the oracle, and two calls sharing one
    workspace give bit-identical results (the split-K partials are added in a
    fixed order).  The workspace starts as NaN bytes: a partial read before it
    is written would show.  K = 1536 is 12 weight tiles, so some splits leave
    waves without tiles."""
    require_gpu()
    monkeypatch.setenv("W4_GEMV_KIND", "0")  # the staged variant, whatever M
    monkeypatch.setenv("W4_GEMV_NWR", str(nwr))
    monkeypatch.setenv("W4_GEMV_NWK", str(nwk))
    monkeypatch.setenv("W4_GEMV_S", str(s))
    K, N = 1536, 208
    w = wl.make_weight(7, 0, N, K)
    for fmt, G in FMTS[:3]:
        codes, scale, zero = oracle_weights(fmt, w, G)
        packed, sc, zc = upload_weights(codes, scale, zero)
        for M in (1, 3, 17):
            x = wl.make_activations(7, 0, M, K)
            xd = dev(x)
            ws_n = w4.workspace_bytes(w4.OP_GEMV, M, K, N, G, fmt)
            ws = torch.full((max(ws_n, 16),), 0xFF, dtype=torch.uint8, device="cuda")  # fp32 NaNs
            announce("gemv variant", dict(nwr=nwr, nwk=nwk, s=s, fmt=fmt, G=G, M=M, ws=ws_n))
            y1 = host(w4.gemv(xd, packed, sc, zc, G, fmt, workspace=ws))
            y2 = host(w4.gemv(xd, packed, sc, zc, G, fmt, workspace=ws))
            y_ref = o.matmul_ref(x, o.dequant(fmt, codes, scale, zero, G))
            assert row_rel_l2(y1, y_ref) <= TOL_ROW_REL_L2, (fmt, G, M)
            assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))


@pytest.mark.parametrize("M", [5, 8, 16, 17, 32])
@pytest.mark.parametrize("cols,nwk,K", [(2, 8, 1536), (4, 8, 8192), (1, 4, 8192), (2, 2, 1536)])
def test_direct_activation_paths_agree(monkeypatch, M, cols, nwk, K):
    """The direct kernel's two activation paths (operand-order loads, and
    whole rows reordered through LDS): within tolerance of the oracle and
    bit-identical to each other (same products, same order), for one and two
    token tiles, ragged M, runs shorter and longer than the operand ring."""
    require_gpu()
    monkeypatch.setenv("W4_GEMV_KIND", "1")
    monkeypatch.setenv("W4_GEMV_C", str(cols))
    monkeypatch.setenv("W4_GEMV_NWK", str(nwk))
    N = 208
    w = wl.make_weight(10, 1, N, K)
    x = wl.make_activations(10, 1, M, K)
    xd = dev(x)
    for fmt, G in FMTS[:3]:
        codes, scale, zero = oracle_weights(fmt, w, G)
        packed, sc, zc = upload_weights(codes, scale, zero)
        ws_n = w4.workspace_bytes(w4.OP_GEMV, M, K, N, G, fmt)
        ws = torch.full((max(ws_n, 16),), 0xFF, dtype=torch.uint8, device="cuda")  # fp32 NaNs
        ys = {}
        for xl in ("0", "1"):
            monkeypatch.setenv("W4_GEMV_XL", xl)
            plan = w4.gemv_plan(M, K, N, G, fmt)
            assert plan["kernel"] == 1 and plan["act_lds"] == int(xl), plan
            announce("gemv direct activations", dict(xl=xl, cols=cols, nwk=nwk, K=K, fmt=fmt, G=G, M=M))
            ys[xl] = host(w4.gemv(xd, packed, sc, zc, G, fmt, workspace=ws))
        y_ref = o.matmul_ref(x, o.dequant(fmt, codes, scale, zero, G))
        assert row_rel_l2(ys["1"], y_ref) <= TOL_ROW_REL_L2, (fmt, G, M)
        assert_elementwise(ys["1"], y_ref)
        assert np.array_equal(ys["0"].view(np.uint16), ys["1"].view(np.uint16)), (fmt, G, M)


@pytest.mark.parametrize("ring", [8, 16])
@pytest.mark.parametrize("nwr,nwk,s,K", [(1, 4, 1, 1536), (2, 4, 1, 1536), (1, 1, 1, 1536), (1, 8, 2, 1536),
                                         (2, 4, 1, 8192), (1, 4, 1, 8192), (1, 2, 1, 8192)])
def test_gemv_ring_depths_agree(monkeypatch, ring, nwr, nwk, s, K):
    """The staged kernel with 8 or 16 weight tiles in flight per wave: runs
    shorter than, equal to and longer than the ring (K = 1536 is 12 tiles
    per column, K = 8192 64), within tolerance of the oracle, bit-identical
    to the default 4-deep ring (same products, same order) and repeatable."""
    require_gpu()
    monkeypatch.setenv("W4_GEMV_KIND", "0")
    monkeypatch.setenv("W4_GEMV_NWR", str(nwr))
    monkeypatch.setenv("W4_GEMV_NWK", str(nwk))
    monkeypatch.setenv("W4_GEMV_S", str(s))
    N = 208
    w = wl.make_weight(9, 1, N, K)
    for fmt, G in FMTS[:3]:
        codes, scale, zero = oracle_weights(fmt, w, G)
        packed, sc, zc = upload_weights(codes, scale, zero)
        for M in (1, 3):
            x = wl.make_activations(9, 1, M, K)
            xd = dev(x)
            ws_n = w4.workspace_bytes(w4.OP_GEMV, M, K, N, G, fmt)
            ws = torch.full((max(ws_n, 16),), 0xFF, dtype=torch.uint8, device="cuda")  # fp32 NaNs
            monkeypatch.setenv("W4_GEMV_RING", str(ring))
            assert w4.gemv_plan(M, K, N, G, fmt)["ring"] == ring
            announce("gemv ring", dict(ring=ring, nwr=nwr, nwk=nwk, s=s, K=K, fmt=fmt, G=G, M=M))
            y1 = host(w4.gemv(xd, packed, sc, zc, G, fmt, workspace=ws))
            y2 = host(w4.gemv(xd, packed, sc, zc, G, fmt, workspace=ws))
            monkeypatch.setenv("W4_GEMV_RING", "4")
            y4 = host(w4.gemv(xd, packed, sc, zc, G, fmt, workspace=ws))
            y_ref = o.matmul_ref(x, o.dequant(fmt, codes, scale, zero, G))
            assert row_rel_l2(y1, y_ref) <= TOL_ROW_REL_L2, (fmt, G, M)
            assert_elementwise(y1, y_ref)
            assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))
            assert np.array_equal(y1.view(np.uint16), y4.view(np.uint16))


@pytest.mark.parametrize("cols,nwk,s", [(1, 8, 1), (2, 8, 1), (4, 8, 1), (2, 4, 1), (2, 3, 2), (4, 1, 3),
                                        (2, 8, 5), (1, 2, 1)])
def test_gemv_direct_variants_agree(monkeypatch, cols, nwk, s):
    """The direct variant (activations read straight into matrix-core
    operands, `cols` tile columns per wave) for each work split: within
    tolerance of the oracle and repeatable.  N = 208 is 13 tile columns, so
    the last column group is partial for cols = 2 and 4."""
    require_gpu()
    monkeypatch.setenv("W4_GEMV_KIND", "1")
    monkeypatch.setenv("W4_GEMV_C", str(cols))
    monkeypatch.setenv("W4_GEMV_NWK", str(nwk))
    monkeypatch.setenv("W4_GEMV_S", str(s))
    K, N = 1536, 208
    w = wl.make_weight(8, 0, N, K)
    for fmt, G in FMTS:
        codes, scale, zero = oracle_weights(fmt, w, G)
        packed, sc, zc = upload_weights(codes, scale, zero)
        for M in (1, 5, 16, 17, 32):
            x = wl.make_activations(8, 0, M, K)
            xd = dev(x)
            ws_n = w4.workspace_bytes(w4.OP_GEMV, M, K, N, G, fmt)
            ws = torch.full((max(ws_n, 16),), 0xFF, dtype=torch.uint8, device="cuda")  # fp32 NaNs
            announce("gemv direct", dict(cols=cols, nwk=nwk, s=s, fmt=fmt, G=G, M=M, ws=ws_n))
            y1 = host(w4.gemv(xd, packed, sc, zc, G, fmt, workspace=ws))
            y2 = host(w4.gemv(xd, packed, sc, zc, G, fmt, workspace=ws))
            y_ref = o.matmul_ref(x, o.dequant(fmt, codes, scale, zero, G))
            assert row_rel_l2(y1, y_ref) <= TOL_ROW_REL_L2, (fmt, G, M)
            assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))


def test_gemv_cfg1_both_formats():
    """1024 x 1024, G = 64, M = 1, no outliers (the single-GEMV workload)."""
    for fmt in (o.FMT_INT4_ASYM, o.FMT_NF4):
        y, y_ref = run_small(fmt, 64, 1, 1024, 1024, seed=1, outliers=False)
        assert row_rel_l2(y, y_ref) <= TOL_ROW_REL_L2


def test_gemv_zero_activations_and_weights():
    require_gpu()
    K, N = 256, 32
    w = np.zeros((N, K), np.float32)
    w[: N // 2] = wl.make_weight(5, 0, N // 2, K)
    for fmt, G in FMTS[:3]:
        codes, scale, zero = oracle_weights(fmt, w, G)
        packed, sc, zc = upload_weights(codes, scale, zero)
        x = np.zeros((2, K), np.float16)
        x[1] = wl.make_activations(5, 0, 1, K)[0]
        announce("gemv zeros", fmt, G)
        y = host(w4.gemv(dev(x), packed, sc, zc, G, fmt))
        assert np.all(y[0] == 0)
        assert np.all(y[1, N // 2:] == 0)
        y_ref = o.matmul_ref(x, o.dequant(fmt, codes, scale, zero, G))
        assert o.max_row_rel_l2(y[1:], y_ref[1:]) <= TOL_ROW_REL_L2


def test_gemv_repeatable():
    """Two runs give bit-identical outputs (deterministic reduction order)."""
    require_gpu()
    w = wl.make_weight(9, 0, 512, 4096)
    x = wl.make_activations(9, 0, 4, 4096)
    codes, scale, zero = oracle_weights(o.FMT_INT4_ASYM, w, 128)
    packed, sc, zc = upload_weights(codes, scale, zero)
    xd = dev(x)
    announce("gemv repeat")
    a = host(w4.gemv(xd, packed, sc, zc, 128, 0))
    b = host(w4.gemv(xd, packed, sc, zc, 128, 0))
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


def full_size_case(fmt, G, M, K, N, cfg, mat, n_sample=160):
    w = wl.make_weight(cfg, mat, N, K)
    x = wl.make_activations(cfg, mat, M, K)
    announce("gemv full", dict(fmt=fmt, G=G, M=M, K=K, N=N))
    codes, scale, zero = w4.quantize(dev(w), G, fmt)
    packed = w4.pack(codes)
    y = host(w4.gemv(dev(x), packed, scale, zero, G, fmt))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(cfg).choice(N, n_sample, replace=False)]))
    rc, rs, rz = oracle_weights(fmt, w[rows], G)
    assert np.array_equal(host(codes[rows]), rc)  # the sampled weights are the oracle's
    y_ref = o.matmul_ref(x, o.dequant(fmt, rc, rs, rz, G))
    return y[:, rows], y_ref


@pytest.mark.parametrize("fmt,G", [(o.FMT_INT4_ASYM, 128), (o.FMT_NF4, 64)])
@pytest.mark.parametrize("M", [1, 4, 16])
def test_gemv_decode_layer_8192(fmt, G, M):
    y, y_ref = full_size_case(fmt, G, M, 8192, 8192, cfg=2, mat=0)
    assert row_rel_l2(y, y_ref) <= TOL_ROW_REL_L2
    assert_elementwise(y, y_ref)


# Every (M, matrix) point of the MLP-shaped workload: up/gate K=8192, N=28672
# and down K=28672, N=8192 at M = 1, 8, 32 (plus M = 4, a staged-kernel plan).
@pytest.mark.parametrize("fmt,G", [(o.FMT_INT4_ASYM, 128), (o.FMT_NF4, 64)])
@pytest.mark.parametrize("M,K,N", [(1, 8192, 28672), (4, 8192, 28672), (8, 8192, 28672), (32, 8192, 28672),
                                   (1, 28672, 8192), (4, 28672, 8192), (8, 28672, 8192), (32, 28672, 8192)])
def test_gemv_mlp_layers(fmt, G, M, K, N):
    y, y_ref = full_size_case(fmt, G, M, K, N, cfg=3, mat=0 if N == 28672 else 1, n_sample=96)
    assert row_rel_l2(y, y_ref) <= TOL_ROW_REL_L2
    assert_elementwise(y, y_ref)


# The decoder layer's products at M = 1 not covered above: k and v
# (K = 8192, N = 1024, which split K over workgroups).
@pytest.mark.parametrize("fmt,G", [(o.FMT_INT4_ASYM, 128), (o.FMT_NF4, 64)])
def test_gemv_decoder_layer_kv_m1(fmt, G):
    p = w4.gemv_plan(1, 8192, 1024, G, fmt)
    assert p["k_slices"] > 1, p  # the case exercises the split-K reduction
    y, y_ref = full_size_case(fmt, G, 1, 8192, 1024, cfg=5, mat=1, n_sample=128)
    assert row_rel_l2(y, y_ref) <= TOL_ROW_REL_L2
    assert_elementwise(y, y_ref)


@pytest.mark.parametrize("G", [64, 128])
@pytest.mark.parametrize("M", [1, 3, 4, 16])
def test_nf4_table_copies_agree(monkeypatch, G, M):
    """NF4 with the 64-copy level table (addresses formed by v_perm_b32,
    chosen where the plan runs one workgroup per CU) and with the 16-copy
    table (W4_GEMV_LUT=16): bit-identical outputs (the same levels, products
    and order), within tolerance of the oracle."""
    require_gpu()
    K, N = 8192, 4096
    assert w4.gemv_plan(M, K, N, G, w4.NF4)["static_lds"] == 256 * 64 * 4  # the wide table is the default here
    w = wl.make_weight(11, 0, N, K)
    x = wl.make_activations(11, 0, M, K)
    codes, scale, zero = oracle_weights(o.FMT_NF4, w, G)
    packed, sc, zc = upload_weights(codes, scale, zero)
    announce("gemv nf4 table", dict(G=G, M=M, K=K, N=N))
    y64 = host(w4.gemv(dev(x), packed, sc, zc, G, w4.NF4))
    monkeypatch.setenv("W4_GEMV_LUT", "16")
    assert w4.gemv_plan(M, K, N, G, w4.NF4)["static_lds"] == 256 * 16 * 4
    y16 = host(w4.gemv(dev(x), packed, sc, zc, G, w4.NF4))
    y_ref = o.matmul_ref(x, o.dequant(o.FMT_NF4, codes, scale, zero, G))
    assert row_rel_l2(y64, y_ref) <= TOL_ROW_REL_L2
    assert_elementwise(y64, y_ref)
    assert np.array_equal(y64.view(np.uint16), y16.view(np.uint16))
