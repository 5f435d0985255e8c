"""Pins for the CPU oracle, independent of the oracle's own formulas.

Each check below ties an oracle function to something other than itself:
an inverse relation checked with a different library routine, exact rational
arithmetic, brute force over every candidate code, hand-written bytes, closed
form error bounds, or constructed inputs whose answer is known.  The
``planted`` tests feed deliberately wrong variants of oracle steps to the same
checks and assert that they are rejected, so a dropped term, a wrong sign or a
transposed operand cannot pass unnoticed.
"""
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import ndtr  # standard normal CDF (not the quantile routine the oracle calls)

import oracle as o
import workloads as wl

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# ---------------------------------------------------------------- NF4 table
def check_nf4_table(c64, c32):
    """Construction-level checks of a 16-level NormalFloat table.

    c64: levels before fp32 rounding, c32: the fp32 table.
    """
    assert c32.shape == (16,) and c32.dtype == np.float32
    assert c32.nbytes == 64  # 16 entries x 4 bytes, the 64-byte table of the NF4 page
    assert c32[0] == -1.0 and c32[7] == 0.0 and c32[15] == 1.0
    assert np.all(np.diff(c32.astype(np.float64)) > 0)
    assert (c32 < 0).sum() == 7 and (c32 > 0).sum() == 8
    assert np.array_equal(c64.astype(np.float32), c32)
    # Undo the normalisation with t = Phi^-1(delta), checked through the CDF.
    delta = 0.5 * ((1 - 1 / 30) + (1 - 1 / 32))
    lo, hi = 0.0, 10.0
    for _ in range(200):  # bisection on the CDF for t with Phi(t) = delta
        mid = 0.5 * (lo + hi)
        lo, hi = (mid, hi) if ndtr(mid) < delta else (lo, mid)
    t = 0.5 * (lo + hi)
    pos = c64[8:] * t
    neg = -c64[:7] * t
    # positive levels sit at evenly spaced probabilities 1/2 + i*(delta-1/2)/8
    p_pos = ndtr(pos)
    want_pos = 0.5 + np.arange(1, 9) * (delta - 0.5) / 8
    assert np.allclose(p_pos, want_pos, rtol=0, atol=1e-12)
    # negative levels at 1/2 + i*(delta-1/2)/7 (mirrored), i = 1..7
    p_neg = ndtr(neg)
    want_neg = 0.5 + np.arange(7, 0, -1) * (delta - 0.5) / 7
    assert np.allclose(p_neg, want_neg, rtol=0, atol=1e-12)


def test_nf4_codebook_construction():
    check_nf4_table(o.nf4_codebook_fp64(), o.nf4_codebook())


def test_nf4_codebook_fp16_rounding_error_bound():
    c32 = o.nf4_codebook().astype(np.float64)
    c16 = o.nf4_codebook().astype(np.float16).astype(np.float64)
    nz = c32 != 0
    assert np.all(np.abs(c16 - c32)[nz] / np.abs(c32[nz]) <= 2.0 ** -11)


def test_planted_nf4_mistakes_rejected():
    good = o.nf4_codebook_fp64()
    # wrong offset: 7 and 8 level halves built from the same spacing
    bad1 = good.copy()
    bad1[8:] = np.sort(good[8:]) * 0.999
    bad1[15] = 1.0
    # missing zero level / shifted table
    bad2 = np.concatenate([good[:7], good[8:], [1.0]])
    for bad in (bad1, bad2):
        with pytest.raises(AssertionError):
            check_nf4_table(bad, bad.astype(np.float32))


# ---------------------------------------------------------- INT4 quantize
def _grid_int4(rng, N, K, G, log2s=-6):
    """Weights exactly on a 4-bit grid with power-of-two scale and integer
    zero point; every group contains codes 0 and 15."""
    ng = K // G
    s = np.float64(2.0 ** log2s)
    z = rng.integers(0, 16, size=(N, ng))
    q = rng.integers(0, 16, size=(N, ng, G))
    q[:, :, 0] = 0
    q[:, :, 1] = 15
    for n in range(N):
        for g in range(ng):
            rng.shuffle(q[n, g])
    w = (s * (q - z[..., None])).reshape(N, K).astype(np.float32)
    return w, q.reshape(N, K), s, z


@pytest.mark.parametrize("G", [64, 128])
def test_int4_round_trip_on_grid(G):
    rng = np.random.default_rng(7)
    w, q, s, z = _grid_int4(rng, 6, 4 * G, G)
    codes, scale, zero = o.quantize_int4_asym(w, G)
    assert np.all(scale.astype(np.float64) == s)
    assert np.array_equal(zero.astype(np.int64), z)
    assert np.array_equal(codes.astype(np.int64), q)
    assert np.array_equal(o.dequant_int4_asym(codes, scale, zero, G), w.astype(np.float64))


def _int4_codes_optimal(w, codes, scale, zero, G):
    """Brute force: each code is a nearest grid point among q in [0, 15]
    (exact rational comparison)."""
    N, K = w.shape
    for n in range(N):
        for k in range(K):
            g = k // G
            s = Fraction(float(scale[n, g]))
            z = Fraction(float(zero[n, g]))
            wf = Fraction(float(w[n, k]))
            errs = [abs(wf - s * (q - z)) for q in range(16)]
            if errs[int(codes[n, k])] != min(errs):
                return False
    return True


def test_int4_codes_are_nearest_grid_points():
    w = wl.make_weight(99, 0, 4, 256)
    codes, scale, zero = o.quantize_int4_asym(w, 64)
    assert _int4_codes_optimal(w, codes, scale, zero, 64)


def test_int4_grid_spans_group_range():
    """The dequant grid reaches both group extremes: every weight is within one
    step of its reconstruction, and the group's min and max within half a step
    plus the fp16 rounding of the scale."""
    w = wl.make_weight(98, 0, 32, 512)
    G = 128
    codes, scale, zero = o.quantize_int4_asym(w, G)
    wd = o.dequant_int4_asym(codes, scale, zero, G).reshape(32, 4, G)
    wg = w.astype(np.float64).reshape(32, 4, G)
    s = scale.astype(np.float64)[..., None]
    assert np.all(np.abs(wd - wg) <= 0.5 * s + 16 * s * 2.0 ** -11)
    assert np.all(s > 0)


def test_int4_special_cases():
    w = np.zeros((2, 128), np.float32)
    w[1, 64:] = np.linspace(0.01, 0.5, 64, dtype=np.float32)  # all-positive group
    codes, scale, zero = o.quantize_int4_asym(w, 64)
    assert scale[0, 0] == 0 and zero[0, 0] == 0 and np.all(codes[0] == 0)
    assert scale[1, 0] == 0 and np.all(codes[1, :64] == 0)
    assert zero[1, 1] == 0 and codes[1, 127] == 15 and codes[1, 64] >= 0


def test_planted_int4_mistakes_rejected():
    rng = np.random.default_rng(5)
    w, q, s, z = _grid_int4(rng, 4, 256, 64)
    # (a) zero point with the wrong sign, (b) code without the zero point
    bad_a = np.clip(np.rint(w.astype(np.float64).reshape(4, 4, 64) / s) - z[..., None], 0, 15)
    bad_b = np.clip(np.rint(w.astype(np.float64).reshape(4, 4, 64) / s), 0, 15)
    for bad in (bad_a, bad_b):
        assert not np.array_equal(bad.reshape(4, 256).astype(np.int64), q)


# ----------------------------------------------------------- NF4 quantize
def test_nf4_round_trip_on_levels():
    rng = np.random.default_rng(11)
    c = o.nf4_codebook()
    N, K, B = 5, 256, 64
    idx = rng.integers(0, 16, size=(N, K // B, B))
    idx[:, :, 0] = 15
    a = np.float32(2.0 ** rng.integers(-8, 2, size=(N, K // B)))
    w = (c[idx] * a[..., None]).astype(np.float32).reshape(N, K)
    codes, absmax = o.quantize_nf4(w, B)
    assert np.array_equal(absmax.astype(np.float32), a)
    assert np.array_equal(codes, idx.reshape(N, K).astype(np.uint8))
    assert np.array_equal(o.dequant_nf4(codes, absmax, B), w.astype(np.float64))


def test_nf4_codes_are_nearest_levels():
    w = wl.make_weight(97, 0, 3, 128)
    codes, absmax = o.quantize_nf4(w, 64)
    c = [Fraction(float(v)) for v in o.nf4_codebook()]
    for n in range(3):
        for k in range(128):
            a = Fraction(float(absmax[n, k // 64]))
            wf = Fraction(float(w[n, k]))
            errs = [abs(wf - ci * a) for ci in c]
            i = int(codes[n, k])
            assert errs[i] == min(errs)
            assert i == errs.index(min(errs))  # lowest index on ties


def test_nf4_zero_block():
    w = np.zeros((1, 128), np.float32)
    w[0, 64:] = 0.25
    codes, absmax = o.quantize_nf4(w, 64)
    assert absmax[0, 0] == 0 and np.all(codes[0, :64] == 7)
    assert absmax[0, 1] == np.float16(0.25) and np.all(codes[0, 64:] == 15)


# ----------------------------------------------------------------- packing
def test_pack_hand_written_bytes():
    codes = np.array([[1, 2, 3, 4, 5, 6, 7, 8], [15, 0, 0, 15, 9, 10, 11, 12]], np.uint8)
    want = np.array([[0x21, 0x43, 0x65, 0x87], [0x0F, 0xF0, 0xA9, 0xCB]], np.uint8)
    assert np.array_equal(o.pack_nibbles(codes), want)
    assert np.array_equal(o.unpack_nibbles(want), codes)


def test_pack_round_trip_and_size():
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 16, size=(16, 1024)).astype(np.uint8)
    p = o.pack_nibbles(codes)
    assert p.shape == (16, 512) and p.nbytes * 4 == codes.size * 2  # 4x smaller than fp16
    assert np.array_equal(o.unpack_nibbles(p), codes)


def test_tile_layout_matches_offset_formula():
    """Every code of a random 32 x 256 matrix sits at the byte and nibble the
    per-element formula names (brute force over all positions)."""
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 16, (32, 256)).astype(np.uint8)
    flat = o.pack_w4(codes).reshape(-1)
    for n in range(32):
        for k in range(256):
            off, nib = o.tile_offset(n, k, 256)
            assert (flat[off] >> (4 * nib)) & 15 == codes[n, k], (n, k)


def test_tile_layout_golden_and_round_trip():
    g = _golden("tile_layout_example.json")
    N, K = g["N"], g["K"]
    n = np.arange(N)[:, None]
    k = np.arange(K)[None, :]
    codes = ((n + k // 8 + 1) % 16).astype(np.uint8)
    t = o.pack_w4(codes).reshape(-1)
    for off, val in g["bytes"].items():
        assert t[int(off)] == val, off
    tb = o.pack_w4(np.broadcast_to(k % 8, (N, K)).astype(np.uint8)).reshape(-1)
    assert list(tb[:4]) == g["pattern_b_first_word"]
    assert list(tb[1020:1024]) == g["pattern_b_first_word"]
    rng = np.random.default_rng(4)
    c2 = rng.integers(0, 16, (48, 384)).astype(np.uint8)
    t2 = o.pack_w4(c2)
    assert t2.shape == (48, 192)
    assert np.array_equal(o.unpack_w4(t2), c2)
    # row tile nb holds only rows 16 nb .. 16 nb + 15
    for nb in range(3):
        assert np.array_equal(o.unpack_w4(t2[16 * nb:16 * nb + 16]), c2[16 * nb:16 * nb + 16])


def test_planted_tile_mistake_rejected():
    """Codes packed low-nibble-first in K order (the plain nibble packing,
    words placed as in the tile layout) are caught by the offset formula."""
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 16, (32, 256)).astype(np.uint8)
    p = o.pack_nibbles(codes)
    w = p.reshape(2, 16, 2, 4, 4, 4).transpose(0, 2, 4, 1, 3, 5)  # [nb][kb][j][r][t][byte]
    wrong = np.ascontiguousarray(w).reshape(-1)
    bad = 0
    for n in range(32):
        for k in range(0, 256, 3):
            off, nib = o.tile_offset(n, k, 256)
            bad += int((wrong[off] >> (4 * nib)) & 15 != codes[n, k])
    assert bad > 0


def test_planted_pack_mistake_rejected():
    codes = np.array([[1, 2, 3, 4]], np.uint8)
    swapped = (codes[:, 1::2] | (codes[:, 0::2] << 4)).astype(np.uint8)
    assert not np.array_equal(swapped, np.array([[0x21, 0x43]], np.uint8))


# -------------------------------------------------- activation decomposition
def _decomp_rows_ok(x, A, S):
    """Brute force + closed-form bound for a two-slice decomposition."""
    xd = x.astype(np.float64)
    M, K = xd.shape
    cand = np.arange(-127, 128, dtype=np.float64)
    r = xd.copy()
    for j in range(A.shape[0]):
        s = S[j].astype(np.float64)
        for m in range(M):
            if s[m] == 0:
                if np.any(A[j, m] != 0):
                    return False
                continue
            # each integer is a nearest point of the grid s * [-127, 127]
            err = np.abs(r[m][:, None] - s[m] * cand[None, :])
            chosen = np.abs(r[m] - s[m] * A[j, m].astype(np.float64))
            if np.any(chosen > err.min(axis=1)):
                return False
        r = r - s[:, None] * A[j].astype(np.float64)
    return True


def test_decompose_nearest_integers_and_bound():
    x = wl.make_activations(96, 0, 8, 512, outliers=True)
    A, S = o.decompose_activations(x, 2)
    assert A.dtype == np.int8 and S.dtype == np.float32
    assert _decomp_rows_ok(x, A, S)
    # exact reconstruction error (rational), bound amax / (127 * 508)
    for m in range(8):
        amax = Fraction(float(np.abs(x[m].astype(np.float64)).max()))
        s1, s2 = Fraction(float(S[0, m])), Fraction(float(S[1, m]))
        worst = max(abs(Fraction(float(xv)) - s1 * int(a1) - s2 * int(a2))
                    for xv, a1, a2 in zip(x[m], A[0, m], A[1, m]))
        assert worst <= s2 / 2
        assert worst <= amax / 64516 * Fraction(1 + 2 ** -21)
        # close to 16 effective bits (MSD page, Abstract)
        assert float(amax / worst if worst else 1e30) >= 2 ** 15.97


def test_decompose_exact_first_slice():
    rng = np.random.default_rng(2)
    ints = rng.integers(-127, 128, size=(3, 64))
    ints[:, 0] = 127
    x = (ints * 2.0 ** -4).astype(np.float16)
    A, S = o.decompose_activations(x, 2)
    assert np.all(S[0] == np.float32(2.0 ** -4))
    assert np.array_equal(A[0].astype(np.int64), ints)
    assert np.all(S[1] == 0) and np.all(A[1] == 0)


def test_decompose_zero_rows_and_one_slice():
    x = np.zeros((2, 32), np.float16)
    x[1, 5] = -3.0
    A, S = o.decompose_activations(x, 1)
    assert A.shape == (1, 2, 32)
    assert S[0, 0] == 0 and np.all(A[0, 0] == 0)
    assert A[0, 1, 5] == -127


def test_planted_decompose_mistake_rejected():
    x = wl.make_activations(95, 0, 4, 256)
    A, S = o.decompose_activations(x, 2)
    # second slice taken from x instead of the residual: fails the bound
    A2 = np.clip(np.rint(x.astype(np.float64) / S[1].astype(np.float64)[:, None]), -127, 127)
    bad = A.copy()
    bad[1] = A2.astype(np.int8)
    assert not _decomp_rows_ok(x, bad, S)


def test_three_slices_nearest_integers_exact_residual_and_bound():
    x = wl.make_activations(97, 0, 6, 512, outliers=True)
    A, S = o.decompose_activations(x, 3)
    assert A.shape == (3, 6, 512)
    assert _decomp_rows_ok(x, A, S)
    for m in range(6):
        r = [Fraction(float(v)) for v in x[m]]
        rf = x[m].astype(np.float64)
        for j in range(3):
            sj = Fraction(float(S[j, m]))
            r = [rv - sj * int(a) for rv, a in zip(r, A[j, m])]
            rf = rf - np.float64(S[j, m]) * A[j, m].astype(np.float64)
            # the fp64 residual the oracle carries is the exact one
            assert all(Fraction(float(a)) == b for a, b in zip(rf, r))
        worst = max(abs(v) for v in r)
        assert worst <= Fraction(float(S[2, m])) / 2
        # each pass shrinks the step by about 254: third step <= amax / 127^3 / 4
        amax = Fraction(float(np.abs(x[m].astype(np.float64)).max()))
        assert worst <= amax / (127 * 254 * 254) * Fraction(1 + 2 ** -20)


def _fixed_rows_ok(x, A, S):
    """Brute-force check of a fixed-ratio decomposition, exact rationals."""
    cand = range(-127, 128)
    for m in range(x.shape[0]):
        s1 = Fraction(float(S[0, m]))
        if s1 == 0:
            if np.any(A[:, m] != 0):
                return False
            continue
        if Fraction(float(S[1, m])) != Fraction(float(np.float32(float(s1 / 254)))):
            return False
        for xv, a1, a2 in zip(x[m], A[0, m], A[1, m]):
            xv = Fraction(float(xv))
            e1 = [abs(xv - s1 * c) for c in cand]
            if abs(xv - s1 * int(a1)) != min(e1):
                return False
            r1 = xv - s1 * int(a1)
            e2 = [abs(r1 - s1 / 254 * c) for c in cand]
            best = min(e2)
            if abs(r1 - s1 / 254 * int(a2)) != best:
                return False
            # on an exact tie the even code is taken (rint)
            if e2.count(best) > 1 and int(a2) % 2:
                return False
    return True


def test_fixed_ratio_nearest_codes_and_bound():
    x = wl.make_activations(98, 0, 5, 256, outliers=True)
    x[4, :] = 0
    A, S = o.decompose_fixed_ratio(x)
    assert A.dtype == np.int8 and S.dtype == np.float32 and A.shape == (2, 5, 256)
    assert _fixed_rows_ok(x, A, S)
    assert np.all(A[:, 4] == 0) and S[0, 4] == 0
    for m in range(4):
        s1 = Fraction(float(S[0, m]))
        worst = max(abs(Fraction(float(xv)) - s1 * int(a1) - s1 / 254 * int(a2))
                    for xv, a1, a2 in zip(x[m], A[0, m], A[1, m]))
        assert worst <= s1 / 508
        assert np.abs(A[1, m]).max() <= 127


def test_fixed_ratio_exact_first_slice_and_ties():
    # x on the first grid: the second slice is zero
    ints = np.arange(-127, 128, dtype=np.int64)
    x = (ints * 2.0 ** -6).astype(np.float16)[None, :]
    A, S = o.decompose_fixed_ratio(x)
    assert S[0, 0] == np.float32(2.0 ** -6)
    assert np.array_equal(A[0, 0].astype(np.int64), ints) and np.all(A[1] == 0)
    # residual of exactly half a second-grid step (s1 = 1, x = 1 + 0.5/254 is
    # not an fp16; use s1 = 2^-6 * 127 / 127 and a residual of 2^-14): checks
    # rounding of 254 * r / s1 = 254 * 2^-14 / 2^-6 = 0.9921875 -> 1
    x2 = np.array([[127 * 2.0 ** -6, 2.0 ** -6 + 2.0 ** -14]], np.float16)
    A2, S2 = o.decompose_fixed_ratio(x2)
    assert A2[0, 0, 1] == 1 and A2[1, 0, 1] == 1


def test_planted_fixed_ratio_mistakes_rejected():
    x = wl.make_activations(99, 0, 3, 128, outliers=True)
    A, S = o.decompose_fixed_ratio(x)
    # the residual's own scale instead of the fixed ratio
    Aa, Sa = o.decompose_activations(x, 2)
    assert not _fixed_rows_ok(x, Aa, np.stack([Sa[0], S[1]]))
    # ratio 256 instead of 254
    r1 = x.astype(np.float64) - S[0].astype(np.float64)[:, None] * A[0]
    bad = A.copy()
    bad[1] = np.clip(np.rint(256 * r1 / S[0].astype(np.float64)[:, None]), -127, 127).astype(np.int8)
    assert not _fixed_rows_ok(x, bad, S)


# ------------------------------------------------------------------ products
def _tiny_case(fmt, seed, M=3, N=4, K=256, G=64):
    w = wl.make_weight(seed, 0, N, K)
    x = wl.make_activations(seed, 0, M, K)
    if fmt == o.FMT_INT4_ASYM:
        codes, scale, zero = o.quantize_int4_asym(w, G)
    else:
        codes, scale = o.quantize_nf4(w, G)
        zero = None
    return x, codes, scale, zero


@pytest.mark.parametrize("fmt", [o.FMT_INT4_ASYM, o.FMT_NF4])
def test_matmul_matches_exact_rationals(fmt):
    x, codes, scale, zero = _tiny_case(fmt, 90 + fmt)
    wd = o.dequant(fmt, codes, scale, zero, 64)
    y = o.matmul_ref(x, wd)
    ex = o.matmul_exact(x, wd)
    absxw = np.abs(x.astype(np.float64)) @ np.abs(wd).T
    for m in range(y.shape[0]):
        for n in range(y.shape[1]):
            # standard dot-product rounding bound, K * 2^-53 * sum |x||w|
            assert abs(Fraction(float(y[m, n])) - ex[m][n]) <= Fraction(256 * 2.0 ** -53) * Fraction(float(absxw[m, n])) * 2


def test_planted_transpose_rejected():
    x, codes, scale, zero = _tiny_case(o.FMT_INT4_ASYM, 89, M=2, N=4, K=256)
    wd = o.dequant(o.FMT_INT4_ASYM, codes, scale, zero, 64)
    ex = o.matmul_exact(x, wd)
    # a plausible slip: using W' in the wrong orientation (reshape, not transpose)
    bad = x.astype(np.float64) @ wd.reshape(256, 4)
    assert not np.allclose(bad, np.array(ex, dtype=np.float64), rtol=1e-6)


@pytest.mark.parametrize("fmt", [o.FMT_INT4_ASYM, o.FMT_NF4])
def test_postscale_equals_dequant_first(fmt):
    x, codes, scale, zero = _tiny_case(fmt, 80 + fmt, M=5, N=32, K=512, G=128 if fmt == 0 else 64)
    G = 128 if fmt == 0 else 64
    y_dq = o.matmul_ref(x, o.dequant(fmt, codes, scale, zero, G))
    y_ps = o.postscale_ref(fmt, x, codes, scale, zero, G)
    assert np.allclose(y_ps, y_dq, rtol=1e-12, atol=1e-12 * np.abs(y_dq).max())


def test_msd_accumulators_brute_force():
    x, codes, scale, zero = _tiny_case(o.FMT_INT4_ASYM, 70, M=2, N=3, K=128, G=64)
    A, S = o.decompose_activations(x, 2)
    D = o.msd_accumulators(A, codes, zero, 64)
    for j in range(2):
        for m in range(2):
            for g in range(2):
                for n in range(3):
                    want = 0
                    for k in range(64 * g, 64 * g + 64):
                        want += int(A[j, m, k]) * (int(codes[n, k]) - int(zero[n, g]))
                    assert D[j, m, g, n] == want
    # int32 never overflows: |D| <= 127 * 15 * G
    assert np.abs(D).max() <= 127 * 15 * 64


def test_msd_result_exact_and_bound():
    G = 64
    x, codes, scale, zero = _tiny_case(o.FMT_INT4_ASYM, 71, M=3, N=4, K=256, G=G)
    y, A, S, D = o.msd_matmul(x, codes, scale, zero, G, 2)
    # exact rational recombination
    for m in range(3):
        for n in range(4):
            ex = sum(Fraction(float(S[j, m])) * Fraction(float(scale[n, g])) * int(D[j, m, g, n])
                     for j in range(2) for g in range(4))
            assert abs(Fraction(float(y[m, n])) - ex) <= abs(ex) * Fraction(2.0 ** -48) + Fraction(2.0 ** -80)
    # closed-form bound against the exact product: |y_msd - y| <= amax/64516 * sum|w'|
    wd = o.dequant_int4_asym(codes, scale, zero, G)
    y_exact = o.matmul_ref(x, wd)
    amax = np.abs(x.astype(np.float64)).max(axis=1)
    bound = (amax / 64516)[:, None] * np.abs(wd).sum(axis=1)[None, :] * (1 + 2 ** -20)
    assert np.all(np.abs(y - y_exact) <= bound + 1e-12)


def test_msd_fixed_result_exact_and_bound():
    G = 64
    x, codes, scale, zero = _tiny_case(o.FMT_INT4_ASYM, 72, M=3, N=4, K=256, G=G)
    y, A, S, D = o.msd_fixed_matmul(x, codes, scale, zero, G)
    wd = o.dequant_int4_asym(codes, scale, zero, G)
    # equals the exact rational product of the reconstructed activations
    for m in range(3):
        s1 = Fraction(float(S[0, m]))
        xh = [s1 * int(a1) + s1 / 254 * int(a2) for a1, a2 in zip(A[0, m], A[1, m])]
        for n in range(4):
            ex = sum(xv * Fraction(float(wv)) for xv, wv in zip(xh, wd[n]))
            assert abs(Fraction(float(y[m, n])) - ex) <= abs(ex) * Fraction(2.0 ** -46) + Fraction(2.0 ** -80)
    # integer combine, brute force
    for m in range(3):
        for g in range(4):
            for n in range(4):
                want = sum((254 * int(A[0, m, k]) + int(A[1, m, k])) * (int(codes[n, k]) - int(zero[n, g]))
                           for k in range(G * g, G * g + G))
                assert 254 * int(D[0, m, g, n]) + int(D[1, m, g, n]) == want
                assert abs(want) < 2 ** 31
    # bound against the exact product: |y - y_exact| <= s1/508 * sum|w'|
    y_exact = o.matmul_ref(x, wd)
    bound = (S[0].astype(np.float64) / 508)[:, None] * np.abs(wd).sum(axis=1)[None, :] * (1 + 2 ** -20)
    assert np.all(np.abs(y - y_exact) <= bound + 1e-12)


def test_planted_fixed_combine_rejected():
    G = 64
    x, codes, scale, zero = _tiny_case(o.FMT_INT4_ASYM, 73, M=2, N=3, K=128, G=G)
    y, A, S, D = o.msd_fixed_matmul(x, codes, scale, zero, G)
    y_exact = o.matmul_ref(x, o.dequant_int4_asym(codes, scale, zero, G))
    # dropping the second slice or weighting it twice moves the result by far
    # more than the decomposition error (which the bound test above pins)
    assert o.max_row_rel_l2(y, y_exact) < 1e-3
    assert o.max_row_rel_l2(o.msd_fixed_result(S[0], np.stack([D[0], 0 * D[1]]), scale), y) > 5e-3
    assert o.max_row_rel_l2(o.msd_fixed_result(S[0], np.stack([D[0], 2 * D[1]]), scale), y) > 5e-3


# ------------------------------------------------------------------ MXFP4
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]  # the format's magnitudes, codes 0..7


def test_e2m1_code_values():
    for c in range(16):
        want = E2M1_TABLE[c & 7] * (-1 if c & 8 else 1)
        assert o.e2m1_value(c) == want and (c < 8 or np.signbit(o.e2m1_value(c)))


def test_mx_scale_exponent_brute_force():
    rng = np.random.default_rng(7)
    amax = np.concatenate([np.abs(rng.standard_normal(200)) * 10.0 ** rng.integers(-6, 5, 200),
                           [6.0 * 2.0 ** k for k in range(-20, 20)], [6.0 * 2.0 ** k * (1 + 2 ** -20) for k in range(-5, 5)],
                           [0.0, 2.0 ** -140]])
    e = o.mx_scale_exponent(amax)
    for a, ee in zip(amax, e):
        if a == 0:
            assert ee == -127
            continue
        want = next(k for k in range(-127, 128) if a <= 6.0 * 2.0 ** k) if a <= 6.0 * 2.0 ** 127 else 127
        assert ee == want, (a, ee, want)


def test_e2m1_round_brute_force_and_ties():
    rng = np.random.default_rng(8)
    t = np.concatenate([rng.uniform(-6, 6, 500), [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -5.0, -0.0, 0.0, 6.0, -6.0]])
    codes = o.e2m1_round(t)
    for v, c in zip(t, codes):
        d = [abs(v - o.e2m1_value(k)) for k in range(16)]
        best = min(d)
        assert d[c] == best
        cands = [k for k in range(16) if d[k] == best and o.e2m1_value(k) != 0 or (d[k] == best and k == 0)]
        if len({o.e2m1_value(k) for k in cands}) > 1:  # a true tie between two values: the even mantissa wins
            assert c % 2 == 0
        if o.e2m1_value(c) == 0:
            assert c == 0  # no negative zero
    # planted: ties away from zero instead of to even
    assert o.e2m1_round(np.array([2.5]))[0] == 4 and o.e2m1_round(np.array([5.0]))[0] == 6


def test_mx_quantize_round_trip_on_grid():
    rng = np.random.default_rng(9)
    codes = rng.integers(0, 16, size=(3, 128)).astype(np.uint8)
    codes[:, ::32] = 7  # every block reaches the largest magnitude, 6
    e = rng.integers(-10, 10, size=(3, 4))
    v = o.mx_dequant(codes, e)
    c2, e2 = o.mx_quantize(v)
    assert np.array_equal(e2, e)
    assert np.array_equal(o.mx_dequant(c2, e2), v)


def _e4m3_grid():
    vals = {m / 8 * 2.0 ** -6 for m in range(8)}
    vals |= {(1 + m / 8) * 2.0 ** (e - 7) for e in range(1, 16) for m in range(8) if (1 + m / 8) * 2.0 ** (e - 7) <= 448}
    return np.array(sorted(vals))


def _rms_bits(x, err):
    return -np.log2(np.sqrt(np.mean(err ** 2)) / np.sqrt(np.mean(x ** 2)))


def test_mx_scale_rule_reproduces_the_mxfp8_figure():
    """The MSD abstract quotes 5.24 effective bits for single-pass MXFP8.  The
    same scale rule applied to E4M3 elements (largest 448) on standard normal
    data gives that figure as RMS effective bits, which fixes the reading."""
    G = _e4m3_grid()
    x = np.random.default_rng(10).standard_normal(32 * 30000).astype(np.float16).astype(np.float64)
    b = x.reshape(-1, 32)
    amax = np.abs(b).max(axis=1)
    e = np.array([next(k for k in range(-40, 40) if a <= 448 * 2.0 ** k) for a in amax])
    t = np.abs(b) / 2.0 ** e[:, None]
    i = np.clip(np.searchsorted(G, t), 1, len(G) - 1)
    lo, hi = G[i - 1], G[i]
    q = np.where(t - lo < hi - t, lo, np.where(t - lo > hi - t, hi, np.where((i - 1) % 2 == 0, lo, hi)))
    err = (b - np.sign(b) * q * 2.0 ** e[:, None]).ravel()
    assert abs(_rms_bits(x, err) - 5.24) < 0.02
    # planted: the saturating rule (largest power of two below amax, minus 8) does not
    e_sat = np.floor(np.log2(amax)) - 8
    t2 = np.minimum(np.abs(b) / 2.0 ** e_sat[:, None], 448)
    i2 = np.clip(np.searchsorted(G, t2), 1, len(G) - 1)
    q2 = np.where(t2 - G[i2 - 1] <= G[i2] - t2, G[i2 - 1], G[i2])
    err2 = (b - np.sign(b) * q2 * 2.0 ** e_sat[:, None]).ravel()
    assert abs(_rms_bits(x, err2) - 5.24) > 0.1


def test_mxfp4_two_pass_bound_and_effective_bits():
    x = wl.make_activations(11, 0, 64, 1024, outliers=False)
    C, E = o.decompose_mxfp4(x, 2)
    xd = x.astype(np.float64)
    r1 = xd - o.mx_dequant(C[0], E[0])
    r2 = r1 - o.mx_dequant(C[1], E[1])
    amax = np.abs(xd.reshape(64, 32, 32)).max(axis=2)
    worst = np.abs(r2.reshape(64, 32, 32)).max(axis=2)
    assert np.all(E[1] <= E[0] - 2)
    # the 1/64 per block of the MSD abstract: |err| <= 2^(e1 - 3) = 2^(e1 + 3) / 64, attained
    assert np.all(worst <= np.ldexp(1.0, E[0] - 3))
    assert np.any(worst == np.ldexp(1.0, E[0] - 3))
    assert np.all(worst < amax / 24)
    assert np.all(np.abs(r1.reshape(64, 32, 32)).max(axis=2) <= np.ldexp(1.0, E[0]))
    # exact residuals: the fp64 pass-2 residual equals the rational one on a sample
    for m in range(2):
        for k in range(0, 1024, 37):
            ex = Fraction(float(x[m, k])) - Fraction(float(o.mx_dequant(C[0], E[0])[m, k])) \
                - Fraction(float(o.mx_dequant(C[1], E[1])[m, k]))
            assert Fraction(float(r2[m, k])) == ex
    bits = _rms_bits(xd.ravel(), r2.ravel())
    # normal blocks: 6.1-6.2 RMS effective bits (uniform blocks give the
    # abstract's 6.6, pinned below)
    assert 6.0 < bits < 6.35
    assert _rms_bits(xd.ravel(), r1.ravel()) < 3.3  # one pass: about 3.1


def test_mxfp4_two_pass_gives_6_6_bits_on_uniform_blocks():
    """The MSD abstract's "near 6.6 effective bits" for two-pass MXFP4: the
    oracle's decomposition of uniformly distributed fp16 values (blocks of
    32 on [-1, 1]) has 6.6 RMS effective bits; the same bits definition gives
    the abstract's 5.24 for single-pass MXFP8 on normal data (above)."""
    rng = np.random.default_rng(21)
    x = rng.uniform(-1, 1, (256, 1024)).astype(np.float16)
    C, E = o.decompose_mxfp4(x, 2)
    xd = x.astype(np.float64)
    err = xd - o.mx_dequant(C[0], E[0]) - o.mx_dequant(C[1], E[1])
    assert abs(_rms_bits(xd.ravel(), err.ravel()) - 6.6) < 0.05


def test_mxfp8_closed_form_5_24_bits():
    """5.24 is also the closed form of a 3-bit-mantissa float's RMS relative
    error when mantissas are log-uniform: ulp 2^-3, rounding error uniform
    (variance ulp^2 / 12), E[1/m^2] = 3 / (8 ln 2) over m in [1, 2)."""
    bits = -0.5 * np.log2(2.0 ** -6 / 12 * 3 / (8 * np.log(2)))
    assert abs(bits - 5.2356) < 1e-4


def test_other_second_pass_rules_miss_the_1_64_bound():
    """Planted alternatives: a saturating second pass (floor(log2 amax) - 2) or
    a fixed offset e2 = e1 - 3 leave errors up to 2^(e1 + 3) / 32 -- twice
    the abstract's bound -- so they are not the reading."""
    from oracle.mx_readings import blocks, two_pass_error
    b = blocks("normal", 4000, seed=22)
    for rule2, bound in (("nosat", 1 / 64), ("ocp", 1 / 32), ("e1-3", 1 / 32)):
        r2, e1 = two_pass_error(b, "nosat", rule2)
        worst = np.max(np.abs(r2).max(axis=1) / np.ldexp(1.0, e1 + 3))
        assert abs(worst - bound) < 0.1 * bound, (rule2, worst)
    # the oracle's own decomposition is the "nosat" rule
    C, E = o.decompose_mxfp4(b.reshape(40, -1).astype(np.float16), 2)
    r2, _ = two_pass_error(b, "nosat", "nosat")
    ref = b.reshape(40, -1) - o.mx_dequant(C[0], E[0]) - o.mx_dequant(C[1], E[1])
    assert np.array_equal(ref.reshape(-1, 32), r2)


def test_mx_matmul_exact_and_pack_layout():
    rng = np.random.default_rng(12)
    x = (rng.standard_normal((2, 128)) * 3).astype(np.float16)
    w = (rng.standard_normal((16, 128)) * 0.02).astype(np.float32)
    wc, we = o.quantize_mxfp4(w)
    C, E = o.decompose_mxfp4(x, 2)
    y = o.mx_matmul(C, E, wc, we)
    for m in range(2):
        for n in range(0, 16, 5):
            ex = sum(Fraction(float(o.mx_dequant(C[j], E[j])[m, k])) * Fraction(float(o.mx_dequant(wc, we)[n, k]))
                     for j in range(2) for k in range(128))
            assert abs(Fraction(float(y[m, n])) - ex) <= abs(ex) * Fraction(2.0 ** -45) + Fraction(2.0 ** -90)
    # packed tile: bytes 16 * (16 j + r) .. + 15 are row r's positions 32 j .. 32 j + 31, low nibble first
    p = o.pack_mx(wc)
    for j in range(4):
        for r in range(16):
            for byte in range(16):
                k = 32 * j + 2 * byte
                assert p[16 * (16 * j + r) + byte] == (wc[r, k] | (wc[r, k + 1] << 4))
    assert np.array_equal(o.unpack_mx(p, 16, 128), wc)


# ------------------------------------------------------------- KV-cache MSD
def _kv_case(seed, Hq, Hkv, L, d=128):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((Hq, d)).astype(np.float16)
    k = rng.standard_normal((Hkv, L, d)).astype(np.float32)
    v = rng.standard_normal((Hkv, L, d)).astype(np.float32)
    kq = [o.quantize_int4_asym(k[h], d) for h in range(Hkv)]
    vq = [o.quantize_int4_asym(v[h], d) for h in range(Hkv)]
    kc = np.stack([a[0] for a in kq]); ks = np.stack([a[1][:, 0] for a in kq]); kz = np.stack([a[2][:, 0] for a in kq])
    vc = np.stack([a[0] for a in vq]); vs = np.stack([a[1][:, 0] for a in vq]); vz = np.stack([a[2][:, 0] for a in vq])
    kd = np.stack([o.dequant_int4_asym(kc[h], ks[h][:, None], kz[h][:, None], d) for h in range(Hkv)])
    vd = np.stack([o.dequant_int4_asym(vc[h], vs[h][:, None], vz[h][:, None], d) for h in range(Hkv)])
    return q, (kc, ks, kz), (vc, vs, vz), kd, vd


def test_attention_ref_brute_force_and_special_cases():
    q, _, _, kd, vd = _kv_case(21, 4, 2, 5, d=128)
    y = o.attention_ref(q, kd, vd, 2)
    for g in range(4):
        h = g // 2  # query heads 0, 1 -> kv head 0; 2, 3 -> kv head 1
        sc = [sum(float(q[g, i]) * kd[h, t, i] for i in range(128)) / 128 ** 0.5 for t in range(5)]
        mx = max(sc)
        e = [np.exp(x - mx) for x in sc]
        want = [sum(e[t] * vd[h, t, n] for t in range(5)) / sum(e) for n in range(128)]
        assert np.allclose(y[g], want, rtol=1e-12, atol=1e-12)
    # one position: the output is that value; equal keys: the mean of the values
    y1 = o.attention_ref(q, kd[:, :1], vd[:, :1], 2)
    assert np.allclose(y1[0], vd[0, 0]) and np.allclose(y1[3], vd[1, 0])
    k2 = np.repeat(kd[:, :1], 2, axis=1)
    y2 = o.attention_ref(q, k2, vd[:, :2], 2)
    assert np.allclose(y2[1], vd[0, :2].mean(axis=0))
    # planted: the wrong head grouping (g mod Hkv) changes the result
    bad = np.stack([o.attention_ref(q[g:g + 1], kd[g % 2:g % 2 + 1], vd[g % 2:g % 2 + 1], 1)[0] for g in range(4)])
    assert not np.allclose(bad, y, rtol=1e-6)


def test_msd_attention_integer_scores_and_error():
    q, K, V, kd, vd = _kv_case(22, 8, 2, 512)
    y = o.msd_attention(q, *K, *V, 2)
    y_ref = o.attention_ref(q, kd, vd, 2)
    # two int8 slices on both sides: ~16 effective bits each
    assert o.max_row_rel_l2(y, y_ref) < 5e-4
    # the score products are exact integers (brute force on a few entries)
    A, S = o.decompose_activations(q[:4], 2)
    kc, ks, kz = K
    for j in range(2):
        for g in (0, 3):
            for t in (0, 77, 511):
                want = sum(int(A[j, g, i]) * (int(kc[0, t, i]) - int(kz[0, t])) for i in range(128))
                got = int(np.einsum("d,d->", A[j, g].astype(np.int64), kc[0, t].astype(np.int64) - int(kz[0, t])))
                assert got == want
    # planted: dropping the value zero points is far off
    y_bad = o.msd_attention(q, *K, V[0], V[1], np.zeros_like(V[2]), 2)
    assert o.max_row_rel_l2(y_bad, y_ref) > 1e-2


def _int_query_case(seed, Hq, Hkv, L, d=128):
    """Integer queries in [-127, 127] (each head reaching 127): their own first
    int8 slice with s_1 = 1 and no residual, so the score products are exact.
    Keys ~ N(0, 0.02^2) keep the softmax spread out; values ~ N(0, 1)."""
    rng = np.random.default_rng(seed)
    q = rng.integers(-127, 128, size=(Hq, d)).astype(np.float16)
    q[:, 0] = 127
    k = (rng.standard_normal((Hkv, L, d)) * 0.02).astype(np.float32)
    v = rng.standard_normal((Hkv, L, d)).astype(np.float32)
    kq = [o.quantize_int4_asym(k[h], d) for h in range(Hkv)]
    vq = [o.quantize_int4_asym(v[h], d) for h in range(Hkv)]
    K = tuple(np.stack([a[i] if i == 0 else a[i][:, 0] for a in kq]) for i in range(3))
    V = tuple(np.stack([a[i] if i == 0 else a[i][:, 0] for a in vq]) for i in range(3))
    kd = np.stack([o.dequant_int4_asym(K[0][h], K[1][h][:, None], K[2][h][:, None], d) for h in range(Hkv)])
    vd = np.stack([o.dequant_int4_asym(V[0][h], V[1][h][:, None], V[2][h][:, None], d) for h in range(Hkv)])
    return q, K, V, kd, vd


def test_msd_attention_exact_when_its_slices_are():
    """Exact score slices (integer queries) and one position per weight block:
    each weight w is +-127 s_1 plus a second slice that takes the fp32 rounding
    of s_1, so the split is exact to about 2^-48 and the output equals plain
    attention over the dequantized cache to fp64 rounding."""
    Hq, Hkv, L = 8, 2, 40
    q, K, V, kd, vd = _int_query_case(23, Hq, Hkv, L)
    A, S = o.decompose_activations(q, 2)
    assert np.all(S[0] == 1.0) and np.all(S[1] == 0.0) and np.array_equal(A[0], q.astype(np.int8))
    y = o.msd_attention(q, *K, *V, Hkv, chunk=1)
    y_ref = o.attention_ref(q, kd, vd, Hkv)
    assert o.max_row_rel_l2(y, y_ref) < 1e-10
    # the softmax is not one-hot here: the check covers the whole weighting
    h0 = q[:2].astype(np.float64) @ kd[0].T / np.sqrt(128)
    p = np.exp(h0 - h0.max(axis=1, keepdims=True))
    assert (p / p.sum(axis=1, keepdims=True)).max() < 0.5


def test_msd_attention_value_error_within_slice_bound(monkeypatch):
    """With exact scores only the weights' two-slice split errs, and the
    decomposition leaves each weight within s_2 / 2 of its slices; so, per
    query head g and dimension n, |o - o_ref| <= sum over blocks b of
    s_2[b, g] / 2 * sum_{t in b} |qV[t, n] - zV[t]| / l[g].  Three blocks of the
    default 256 positions, the last one ragged."""
    Hq, Hkv, L, d = 8, 2, 700, 128
    q, K, V, kd, vd = _int_query_case(24, Hq, Hkv, L, d)
    y = o.msd_attention(q, *K, *V, Hkv)
    y_ref = o.attention_ref(q, kd, vd, Hkv)
    G = Hq // Hkv
    for h in range(Hkv):
        rows = slice(h * G, (h + 1) * G)
        score = q[rows].astype(np.float64) @ kd[h].T / np.sqrt(d)       # exact keys, exact queries
        p = np.exp(score - score.max(axis=1, keepdims=True))
        l = p.sum(axis=1)
        w = p * V[1][h].astype(np.float64)[None, :]                   # weights with the value scale
        qv = np.abs(V[0][h].astype(np.int64) - V[2][h].astype(np.float16).astype(np.int64)[:, None])
        bound = np.zeros((G, d))
        for c0 in range(0, L, o.ATTN_CHUNK):
            _, R = o.decompose_activations(w[:, c0:c0 + o.ATTN_CHUNK], 2)
            bound += (R[1].astype(np.float64) / 2)[:, None] * qv[c0:c0 + o.ATTN_CHUNK].sum(axis=0)[None, :]
        bound /= l[:, None]
        err = np.abs(y[rows] - y_ref[rows])
        assert np.all(err <= bound * (1 + 1e-9) + 1e-13)
        # the bound is tight enough to mean something: within 0.3 % of the
        # largest output (a wrong block scale or a dropped slice is far off)
        assert bound.max() < 3e-3 * np.abs(y_ref[rows]).max()
        assert np.abs(y[rows] - y_ref[rows]).max() > 0  # the split is not exact here
    # planted: a weight split that keeps only its first slice breaks the bound
    import oracle.w4_oracle as ow
    real = ow.decompose_activations

    def first_slice_only(x, nslices=2):
        A, S = real(x, nslices)
        A[1:] = 0
        return A, S
    monkeypatch.setattr(ow, "decompose_activations", first_slice_only)
    y_bad = o.msd_attention(q, *K, *V, Hkv)
    monkeypatch.setattr(ow, "decompose_activations", real)
    assert np.abs(y_bad - y_ref).max() > 2 * np.abs(y - y_ref).max()
    assert o.max_row_rel_l2(y_bad, y_ref) > 1e-3


# ------------------------------------------------------- residual compensation
def test_salient_channels_hand_example():
    x = np.array([[0.5, -3.0, 2.0, 3.0, 0.0, 1.0],
                  [0.25, 1.0, -2.5, 0.0, 0.0, -1.0]], np.float16)
    # scores max_m |x|: 0.5, 3, 2.5, 3, 0, 1 -> 1 and 3 tie (lower index first), then 2, 5, 0, 4
    assert o.salient_channels(x, 4).tolist() == [1, 3, 2, 5]
    assert o.salient_channels(x, 6).tolist() == [1, 3, 2, 5, 0, 4]
    assert o.salient_channels(x, 0).size == 0


def test_salient_channels_brute_force():
    rng = np.random.default_rng(5)
    for trial in range(20):
        M, K = int(rng.integers(1, 5)), int(rng.integers(1, 40))
        x = rng.integers(-4, 5, size=(M, K)).astype(np.float16)  # many ties
        k = int(rng.integers(0, K + 1))
        idx = o.salient_channels(x, k).tolist()
        score = [max(abs(float(x[m, c])) for m in range(M)) for c in range(K)]
        # selection sort by (score desc, index asc), written out
        rest, want = list(range(K)), []
        for _ in range(k):
            best = rest[0]
            for c in rest[1:]:
                if score[c] > score[best] or (score[c] == score[best] and c < best):
                    best = c
            want.append(best)
            rest.remove(best)
        assert idx == want


def test_residual_restores_weights_within_fp16_rounding():
    G = 64
    w = wl.make_weight(91, 0, 4, 256)
    codes, scale, zero = o.quantize_int4_asym(w, G)
    wd = o.dequant_int4_asym(codes, scale, zero, G)
    R = o.residual_fp16(w, wd)
    assert R.shape == (256, 4) and R.dtype == np.float16
    for n in range(4):
        for k in range(0, 256, 7):
            exact = Fraction(float(w[n, k])) - Fraction(float(wd[n, k]))
            r = Fraction(float(R[k, n]))
            # fp16 rounding of the exact residual: within half an fp16 step
            step = Fraction(2) ** (int(np.floor(np.log2(abs(float(exact))))) - 10) if exact else Fraction(0)
            assert abs(r - exact) <= max(step / 2, Fraction(2) ** -25)


def test_full_correction_equals_product_with_restored_weights():
    G = 64
    x, codes, scale, zero = _tiny_case(o.FMT_INT4_ASYM, 92, M=3, N=5, K=256, G=G)
    w = wl.make_weight(92, 0, 5, 256)
    wd = o.dequant_int4_asym(codes, scale, zero, G)
    R = o.residual_fp16(w, wd)
    idx = o.salient_channels(x, 256)
    y = o.matmul_ref(x, wd) + o.residual_correction(x, R, idx)
    # the same thing as one product with W' + R (a different evaluation order)
    w_restored = wd + R.T.astype(np.float64)
    y2 = x.astype(np.float64) @ w_restored.T
    assert np.allclose(y, y2, rtol=1e-12, atol=1e-14)
    # and it is closer to the unquantized product than W' alone
    y_full = x.astype(np.float64) @ w.astype(np.float64).T
    assert np.abs(y - y_full).max() < 1e-3 * np.abs(o.matmul_ref(x, wd) - y_full).max()
    # planted mistakes: residual with the wrong sign, or the transposed residual
    assert not np.allclose(o.matmul_ref(x, wd) - o.residual_correction(x, R, idx), y2, rtol=1e-6)
    assert not np.allclose(x.astype(np.float64)[:, idx] @ R.astype(np.float64)[::-1][idx, :] + o.matmul_ref(x, wd),
                           y2, rtol=1e-6)


def test_correction_of_outlier_channels_reduces_error():
    G = 128
    M, K, N = 2, 1024, 64
    w = wl.make_weight(93, 0, N, K)
    x = wl.make_activations(93, 0, M, K, outliers=True)
    codes, scale, zero = o.quantize_int4_asym(w, G)
    wd = o.dequant_int4_asym(codes, scale, zero, G)
    R = o.residual_fp16(w, wd)
    y_full = x.astype(np.float64) @ w.astype(np.float64).T
    y_q = o.matmul_ref(x, wd)
    n_out = int(np.ceil(0.01 * K))
    idx = o.salient_channels(x, n_out)
    # the selected channels are exactly the workload's x20 outlier channels
    assert sorted(idx.tolist()) == wl.outlier_channels(93, 0, K).tolist()
    err_q = np.linalg.norm(y_q - y_full)
    err_c = np.linalg.norm(y_q + o.residual_correction(x, R, idx) - y_full)
    assert err_c < 0.9 * err_q


def test_max_row_rel_l2_hand_example():
    y_ref = np.array([[3.0, 4.0], [1.0, 0.0]])
    y = np.array([[3.0, 4.5], [1.0, 0.01]])
    assert o.max_row_rel_l2(y, y_ref) == pytest.approx(max(0.5 / 5.0, 0.01))


# ------------------------------------------------------- hand-worked fixtures
def _golden(name):
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", name)) as f:
        return json.load(f)


def test_int4_hand_example():
    g = _golden("int4_hand_example.json")
    w = np.array([g["w"]], np.float32)
    codes, scale, zero = o.quantize_int4_asym(w, g["G"])
    assert codes[0].tolist() == g["codes"]
    assert hex(int(scale.view(np.uint16)[0, 0])) == g["scale_fp16_bits"]
    assert float(zero[0, 0]) == g["zero"]


def test_nf4_hand_example():
    g = _golden("nf4_hand_example.json")
    w = np.array([g["w"]], np.float32)
    codes, absmax = o.quantize_nf4(w, g["B"])
    assert codes[0].tolist() == g["codes"]
    assert float(absmax[0, 0]) == g["absmax"]
