"""Host-only checks of the GEMV launch planner through w4_gemv_plan (no GPU).

Every plan the library can choose -- default or forced through the
W4_GEMV_* sweep overrides -- must fit the kernels it launches: at most 512
threads per workgroup (the kernels' launch bound), dynamic LDS within the
budget the library reserves, and static plus dynamic LDS within the 160 KiB
of one CU.  The workspace the plan asks for must hold its split-K partials.
"""
import itertools

import pytest

import bit_weight_quantized_amd as w4

LDS_PER_CU = 160 * 1024
MAX_THREADS = 512
FMTS = [(0, 128), (0, 64), (1, 64), (1, 128)]
OVERRIDES = ("W4_GEMV_KIND", "W4_GEMV_NWR", "W4_GEMV_NWK", "W4_GEMV_C", "W4_GEMV_S", "W4_GEMV_RING", "W4_GEMV_XL")


@pytest.fixture(autouse=True)
def no_overrides(monkeypatch):
    for v in OVERRIDES:
        monkeypatch.delenv(v, raising=False)
    import os
    if not os.path.exists(w4.lib_path):
        import bit_weight_quantized_amd.build as b
        b.build()


def check(p, M, K, N):
    where = (M, K, N, p)
    assert p["ok"] == 1, where
    assert 64 <= p["threads"] <= MAX_THREADS and p["threads"] % 64 == 0, where
    assert p["threads"] == 64 * p["row_waves"] * p["k_waves"], where
    assert 0 <= p["lds_bytes"] <= p["lds_budget"], where
    assert p["lds_budget"] + p["static_lds"] <= LDS_PER_CU, where
    assert 1 <= p["k_slices"] <= K // 128, where
    assert p["token_tiles"] == (1 if M <= 16 else 2), where
    if p["k_slices"] > 1:
        assert p["workspace_bytes"] == p["k_slices"] * M * N * 4, where
    else:
        assert p["workspace_bytes"] == 0, where
    if p["kernel"] == 1:
        assert p["ring"] == (4 if M <= 16 else 2), where
        assert p["row_waves"] == 1 and p["cols"] in (1, 2, 4), where
        assert p["workgroups"] == -(-(N // 16) // p["cols"]), where
        assert p["act_lds"] in (0, 1), where
        if p["act_lds"]:  # the per-wave activation areas fit after the scale block or reduction area
            assert p["lds_bytes"] >= p["k_waves"] * p["token_tiles"] * 4096, where
    else:
        assert p["kernel"] == 0 and p["cols"] == 1 and p["act_lds"] == 0, where
        assert p["ring"] in ((4, 8, 16) if M <= 16 else (4,)), where
        assert p["workgroups"] == -(-N // (16 * p["row_waves"])), where


def test_default_plans_fit_the_kernels():
    """M = 1..32, K = 128..32768 in steps of 128, N from one tile to 57344,
    both formats and both group sizes (about 360 thousand plans)."""
    Ns = (16, 32, 48, 208, 1024, 1040, 4096, 8192, 14336, 28672, 57344)
    n = 0
    for fmt, G in FMTS:
        for M in range(1, 33):
            for K in range(128, 32768 + 1, 128):
                if K % G:
                    continue
                for N in Ns:
                    check(w4.gemv_plan(M, K, N, G, fmt), M, K, N)
                    n += 1
    assert n > 300000


def test_case_m17_k128_n16_runs_512_threads():
    """The shape that once faulted under a 1024-thread plan now gets the
    direct kernel with eight K waves (512 threads), in every format."""
    for fmt, G in FMTS:
        p = w4.gemv_plan(17, 128, 16, G, fmt)
        check(p, 17, 128, 16)
        assert p["kernel"] == 1 and p["k_waves"] == 8 and p["threads"] == 512, p


SHAPES = [(M, K, N) for M in (1, 4, 5, 17, 32) for K in (128, 1536, 8192, 28672) for N in (16, 208, 8192)]


@pytest.mark.parametrize("kind", [0, 1])
def test_forced_plans_fit_the_kernels(monkeypatch, kind):
    """Every W4_GEMV_* override combination the sweeps and tests use, and the
    out-of-range values the planner must clamp."""
    monkeypatch.setenv("W4_GEMV_KIND", str(kind))
    waves = range(0, 18)  # 0 and > 8 are out of range: the default applies
    slices = (0, 1, 2, 3, 5, 7, 12, 64, 300)
    if kind == 0:
        combos = itertools.product(waves, waves, (0,), slices)
    else:
        combos = itertools.product((0,), waves, (0, 1, 2, 3, 4, 8), slices)
    for n, (nwr, nwk, c, s) in enumerate(combos):
        monkeypatch.setenv("W4_GEMV_RING", str((0, 4, 8, 16, 5)[n % 5]))
        monkeypatch.setenv("W4_GEMV_XL", str(n % 2))
        monkeypatch.setenv("W4_GEMV_NWR", str(nwr))
        monkeypatch.setenv("W4_GEMV_NWK", str(nwk))
        monkeypatch.setenv("W4_GEMV_C", str(c))
        monkeypatch.setenv("W4_GEMV_S", str(s))
        for fmt, G in FMTS:
            for M, K, N in SHAPES:
                if K % G:
                    continue
                p = w4.gemv_plan(M, K, N, G, fmt)
                check(p, M, K, N)
                assert p["kernel"] == kind, p


def test_workspace_query_matches_plan():
    for fmt, G in FMTS:
        for M, K, N in SHAPES:
            if K % G:
                continue
            assert w4.workspace_bytes(w4.OP_GEMV, M, K, N, G, fmt) == w4.gemv_plan(M, K, N, G, fmt)[
                "workspace_bytes"]


@pytest.mark.parametrize("args", [(0, 128, 16, 128, 0), (33, 128, 16, 128, 0), (1, 200, 16, 128, 0),
                                  (1, 128, 40, 128, 0), (1, 128, 16, 32, 0), (1, 128, 16, 128, 5)])
def test_plan_query_rejects_bad_shapes(args):
    with pytest.raises(w4.W4Error):
        w4.gemv_plan(*args)
