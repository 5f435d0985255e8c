"""GPU parity of the split-K tail of the matrix-core GEMMs.

The GEMMs run one workgroup per CU.  When the tiles leave a partial last
round, the tiles of that round run as a second launch with each tile's K
steps split over several workgroups (fp32 partials, then a reduction kernel).
Each product here is shaped so that this happens: 13 x 20 = 260 output tiles
on 256 CUs leave 4.  It is compared with the oracle on every output row of
the tail's tiles and of sampled other tiles, with the tail on, with it off
(W4_GEMM_TAIL=0), and with a workspace too small for the tail's partials
(one launch: bit-identical to the tail-off result)."""
import numpy as np
import pytest
import torch

import bit_weight_quantized_amd as w4
import oracle as o
import workloads as wl
from gpu_helpers import (TOL_ROW_REL_L2, announce, dev, host, oracle_weights, require_gpu,
                         row_rel_l2, upload_weights)

pytestmark = pytest.mark.gpu

BN = 256  # output columns per tile in every matrix-core kernel


def walk(tiles_m, tiles_n, gm, places):
    """(row block, column block) of places in the kernels' tile walk: groups
    of gm row blocks, column block by column block."""
    out = []
    for p in places:
        group = p // (gm * tiles_n)
        first = group * gm
        g = min(tiles_m - first, gm)
        i = p - group * gm * tiles_n
        out.append((first + i % g, i // g))
    return out


def tail_rows_cols(M, N, bm, seed):
    """Rows and columns covering the tail's tiles, plus sampled others."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tiles_m, tiles_n = -(-M // bm), -(-N // BN)
    tiles = tiles_m * tiles_n
    r = tiles % cus
    assert tiles > cus and 0 < r <= cus // 2, (tiles, cus)
    tail = walk(tiles_m, tiles_n, 4, range(tiles - r, tiles))
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(M, 48, replace=False).tolist())
    cols = set(rng.choice(N, 48, replace=False).tolist())
    for mb, nb in tail:
        rows.update(range(mb * bm, min(M, (mb + 1) * bm)))
        cols.update(range(nb * BN, min(N, (nb + 1) * BN)))
    return np.array(sorted(rows)), np.array(sorted(cols))


@pytest.fixture
def group_rows(monkeypatch):
    monkeypatch.delenv("W4_GEMM_GM", raising=False)  # the walk above assumes the default of 4


@pytest.mark.parametrize("mode", [w4.DQ_F16, w4.POSTSCALE])
def test_tail_gemm_f16(monkeypatch, group_rows, mode):
    M, K, N, G, fmt = 1664, 4096, 5120, 128, o.FMT_INT4_ASYM
    rows, cols = tail_rows_cols(M, N, 128, 70)
    w = wl.make_weight(70, 0, N, K)
    x = wl.make_activations(70, 0, M, K)
    codes, scale, zero = oracle_weights(fmt, w, G)
    packed, sc, zc = upload_weights(codes, scale, zero)
    assert w4.workspace_bytes(w4.OP_GEMM, M, K, N, G, mode) > 0  # room for the tail's partials
    if mode == w4.POSTSCALE:
        ref = o.postscale_ref(fmt, x, codes[cols], scale[cols], zero[cols], G)
    else:
        ref = o.matmul_ref(x, o.dequant(fmt, codes[cols], scale[cols], zero[cols], G))
    announce("gemm tail", dict(mode=mode, M=M, K=K, N=N))
    y_tail = host(w4.gemm(dev(x), packed, sc, zc, G, fmt, mode))
    assert row_rel_l2(y_tail[:, cols], ref) <= TOL_ROW_REL_L2
    monkeypatch.setenv("W4_GEMM_TAIL", "0")
    announce("gemm tail off", dict(mode=mode))
    y_off = host(w4.gemm(dev(x), packed, sc, zc, G, fmt, mode))
    assert row_rel_l2(y_off[:, cols], ref) <= TOL_ROW_REL_L2
    monkeypatch.delenv("W4_GEMM_TAIL")
    announce("gemm tail, workspace too small", dict(mode=mode))
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    y_small = host(w4.gemm(dev(x), packed, sc, zc, G, fmt, mode, workspace=small))
    assert np.array_equal(y_small.view(np.uint16), y_off.view(np.uint16))
    # the tail moved only the tail's tiles' summation order
    assert row_rel_l2(y_tail, y_off.astype(np.float64)) <= TOL_ROW_REL_L2


@pytest.mark.parametrize("variant", ["msd2", "msd1", "fixed"])
def test_tail_gemm_decomp(monkeypatch, group_rows, variant):
    M, K, N, G = 1664, 4096, 5120, 128
    ns = 1 if variant == "msd1" else 2
    rows, cols = tail_rows_cols(M, N, 128, 71)
    w = wl.make_weight(71, 0, N, K)
    x = wl.make_activations(71, 0, M, K)
    codes, scale, zero = o.quantize_int4_asym(w, G)
    packed, sc, zc = upload_weights(codes, scale, zero)
    base = w4.workspace_bytes(w4.OP_GEMM_DECOMP, M, K, 0, G, ns)
    full = w4.workspace_bytes(w4.OP_GEMM_DECOMP, M, K, N, G, ns)
    assert full > base
    if variant == "fixed":
        A, S = o.decompose_fixed_ratio(x[rows])
        ref = o.msd_fixed_result(S[0], o.msd_accumulators(A, codes[cols], zero[cols], G), scale[cols])
        call = lambda ws: w4.gemm_decomp_fixed(dev(x), packed, sc, zc, G, workspace=ws)
    else:
        A, S = o.decompose_activations(x[rows], ns)
        ref = o.msd_result(S, o.msd_accumulators(A, codes[cols], zero[cols], G), scale[cols])
        call = lambda ws: w4.gemm_decomp(dev(x), packed, sc, zc, G, ns, workspace=ws)
    announce("decomp tail", dict(variant=variant, M=M, K=K, N=N))
    y_tail = host(call(torch.empty(full, dtype=torch.uint8, device="cuda")))
    assert row_rel_l2(y_tail[np.ix_(rows, cols)], ref) <= TOL_ROW_REL_L2
    announce("decomp tail, workspace without room for it", dict(variant=variant))
    y_small = host(call(torch.empty(base, dtype=torch.uint8, device="cuda")))
    assert row_rel_l2(y_small[np.ix_(rows, cols)], ref) <= TOL_ROW_REL_L2
    monkeypatch.setenv("W4_GEMM_TAIL", "0")
    announce("decomp tail off", dict(variant=variant))
    y_off = host(call(torch.empty(full, dtype=torch.uint8, device="cuda")))
    assert np.array_equal(y_small.view(np.uint16), y_off.view(np.uint16))
    assert row_rel_l2(y_tail, y_off.astype(np.float64)) <= TOL_ROW_REL_L2


@pytest.mark.parametrize("nslices", [1, 2])
def test_tail_gemm_mx(monkeypatch, group_rows, nslices):
    monkeypatch.delenv("W4_MX_WM", raising=False)  # 256-token tiles
    M, K, N = 3328, 2048, 5120
    rows, cols = tail_rows_cols(M, N, 256, 72)
    w = wl.make_weight(72, 0, N, K)
    x = wl.make_activations(72, 0, M, K)
    wc, we = o.quantize_mxfp4(w[cols])
    announce("mx tail quantize", dict(M=M, K=K, N=N))
    codes, scale = w4.quantize_mx(dev(w))
    assert np.array_equal(host(codes[cols]), wc)
    packed = w4.pack_mx(codes)
    base = w4.workspace_bytes(w4.OP_GEMM_MX, M, K, 0, 32, nslices)
    full = w4.workspace_bytes(w4.OP_GEMM_MX, M, K, N, 32, nslices)
    assert full > base
    C, E = o.decompose_mxfp4(x[rows], nslices)
    ref = o.mx_matmul(C, E, wc, we)
    call = lambda ws: host(w4.gemm_mx(dev(x), packed, scale, nslices, workspace=ws))
    announce("mx tail", dict(nslices=nslices))
    y_tail = call(torch.empty(full, dtype=torch.uint8, device="cuda"))
    assert row_rel_l2(y_tail[np.ix_(rows, cols)], ref) <= TOL_ROW_REL_L2
    announce("mx tail, workspace without room for it", dict(nslices=nslices))
    y_small = call(torch.empty(base, dtype=torch.uint8, device="cuda"))
    assert row_rel_l2(y_small[np.ix_(rows, cols)], ref) <= TOL_ROW_REL_L2
    monkeypatch.setenv("W4_GEMM_TAIL", "0")
    announce("mx tail off", dict(nslices=nslices))
    y_off = call(torch.empty(full, dtype=torch.uint8, device="cuda"))
    assert np.array_equal(y_small.view(np.uint16), y_off.view(np.uint16))
    assert row_rel_l2(y_tail, y_off.astype(np.float64)) <= TOL_ROW_REL_L2


@pytest.mark.parametrize("variant", ["msd1", "msd2", "msd3", "fixed"])
def test_tail_only_small_m_decomp(monkeypatch, group_rows, variant):
    """M = 256: the 16 output tiles fill a sixteenth of the CUs, so every tile
    runs with K split over workgroups (no full-round launch).  Every output
    against the oracle, and against the unsplit product (W4_GEMM_TAIL=0)."""
    M, K, N, G = 256, 2048, 2048, 128
    ns = {"msd1": 1, "msd2": 2, "msd3": 3, "fixed": 2}[variant]
    w = wl.make_weight(73, 0, N, K)
    x = wl.make_activations(73, 0, M, K)
    codes, scale, zero = o.quantize_int4_asym(w, G)
    packed, sc, zc = upload_weights(codes, scale, zero)
    full = w4.workspace_bytes(w4.OP_GEMM_DECOMP, M, K, N, G, ns)
    assert full > w4.workspace_bytes(w4.OP_GEMM_DECOMP, M, K, 0, G, ns)
    if variant == "fixed":
        A, S = o.decompose_fixed_ratio(x)
        ref = o.msd_fixed_result(S[0], o.msd_accumulators(A, codes, zero, G), scale)
        call = lambda: w4.gemm_decomp_fixed(dev(x), packed, sc, zc, G,
                                            workspace=torch.empty(full, dtype=torch.uint8, device="cuda"))
    else:
        A, S = o.decompose_activations(x, ns)
        ref = o.msd_result(S, o.msd_accumulators(A, codes, zero, G), scale)
        call = lambda: w4.gemm_decomp(dev(x), packed, sc, zc, G, ns,
                                      workspace=torch.empty(full, dtype=torch.uint8, device="cuda"))
    announce("decomp tail only", dict(variant=variant, M=M, K=K, N=N))
    y_tail = host(call())
    assert row_rel_l2(y_tail, ref) <= TOL_ROW_REL_L2
    monkeypatch.setenv("W4_GEMM_TAIL", "0")
    announce("decomp unsplit", dict(variant=variant))
    y_off = host(call())
    assert row_rel_l2(y_off, ref) <= TOL_ROW_REL_L2
    assert row_rel_l2(y_tail, y_off.astype(np.float64)) <= TOL_ROW_REL_L2
