"""CPU checks of the fp32 decision procedures the decomposition kernels use
(an fp32 estimate of each quotient, rounded with one addition of 1.5 * 2^23,
and an exact sign test where the estimate lies within 2^-14 of a
half-integer), emulated with numpy float32 arithmetic and exact rationals,
against the fp64 oracle's integer codes.

* ``decide127``: clamp(rint(fl64(n / s)), +-127) for an exact numerator n
  (x, a residual, 254 times one) and an fp32 scale s, the estimate
  fl32(fl32(n) * fl32(1 / s)), the sign test on n - h s in fp64;
* the fixed-ratio procedure of the product with the decomposition inside its
  K loop: A_1 from fl32(x * inv), r_1 = fl32(fma(-s_1, A_1, x)), A_2 from
  fl32(fl32(254 r_1) * inv), the exact test on 254 x - (254 A_1 + h) s_1.

Rows: Gaussian activations with outlier channels; rows built so that
quotients of every slice sit exactly on half-integers or one fp16 step away;
rows of tiny and subnormal fp16 values; and the same rows with the exact
test forced for every element (window 1/2), which checks the exact path
alone."""
from fractions import Fraction

import numpy as np
import pytest

import oracle as o
import workloads as wl

F32 = np.float32
MAGIC = F32(12582912.0)  # 1.5 * 2^23


def rint32(t):
    return (t + MAGIC).astype(F32) - MAGIC


def inv32(s):
    return np.float32(1.0 / float(s)) if s != 0 else np.float32(0.0)


def decide127(n, s, inv, window):
    """n: exact fp64 numerators (array), s: the fp32 scale (as a Python
    float), inv: fl32(1 / s)."""
    t = (n.astype(F32) * inv).astype(F32)
    q = rint32(t)
    assert np.all(np.abs(q) <= 127)  # the kernels take the fast estimate without a clamp
    # near a half-integer: |t - q| > 1/2 - window (the kernels' form; the
    # same set as ||t - q| - 1/2| < window, since |t - q| <= 1/2)
    near = np.abs((t - q).astype(F32)) > F32(0.5) - F32(window)
    assert np.array_equal(near, np.abs(np.abs((t - q).astype(F32)) - F32(0.5)) < F32(window))
    for i in np.nonzero(near)[0]:
        sg = 1.0 if t[i] >= q[i] else -1.0
        h = Fraction(float(q[i])) + Fraction(sg) / 2
        d = Fraction(float(n[i])) - h * Fraction(s)
        if d * int(sg) > 0 or (d == 0 and int(q[i]) % 2 != 0):
            q[i] = q[i] + F32(sg)
    return np.clip(q, -127, 127).astype(np.float64)


def decompose_emulated(x, nslices, fixed, window):
    """The decomposition kernel's procedure for one row x (fp16)."""
    r = x.astype(np.float64)
    codes, scales = [], []
    s = [float(F32(np.abs(r).max() / 127.0))]
    for j in range(nslices):
        if fixed and j == 1:
            q = decide127(254.0 * r, s[0], inv32(s[0]), window)
            codes.append(q)
            scales.append(float(F32(s[0] / 254.0)))
            break
        q = decide127(r, s[j], inv32(s[j]), window)
        codes.append(q)
        scales.append(s[j])
        r = r - s[j] * q  # exact in fp64
        if j + 1 < nslices:
            s.append(float(F32(np.abs(r).max() / 127.0)))
    return np.array(codes), np.array(scales, dtype=np.float32)


def fused_fixed_emulated(x, s1, window):
    """The product's in-loop procedure for one row (fixed ratio)."""
    xf = x.astype(F32)
    s1f, inv = F32(s1), inv32(s1)
    t1 = (xf * inv).astype(F32)
    q1 = rint32(t1)
    assert np.all(np.abs(q1) <= 127)
    near = np.abs((t1 - q1).astype(F32)) > F32(0.5) - F32(window)
    q1 = np.clip(q1, -127, 127).astype(F32)
    # fma(-s1, q1, x) rounded once: the fp64 sum is exact here
    r1 = (xf.astype(np.float64) - float(s1f) * q1.astype(np.float64)).astype(F32)
    t2 = ((F32(254.0) * r1).astype(F32) * inv).astype(F32)
    q2 = rint32(t2)
    assert np.all(np.abs(q2) <= 127)
    near |= np.abs((t2 - q2).astype(F32)) > F32(0.5) - F32(window)
    q2 = np.clip(q2, -127, 127).astype(F32)
    for i in np.nonzero(near)[0]:
        def exact_rint(v, c, t):
            q = float(rint32(np.array([t], F32))[0])
            sg = 1.0 if t >= q else -1.0
            h = Fraction(q) + Fraction(sg) / 2
            d = Fraction(float(v)) - (Fraction(float(c)) + h) * Fraction(float(s1f))
            return q + sg if (d * int(sg) > 0 or (d == 0 and int(q) % 2 != 0)) else q
        a1 = min(max(exact_rint(xf[i], 0.0, t1[i]), -127.0), 127.0)
        r = F32(float(xf[i]) - float(s1f) * a1)
        t = F32(F32(254.0 * float(r)) * inv)
        a2 = min(max(exact_rint(254.0 * float(xf[i]), 254.0 * a1, t), -127.0), 127.0)
        q1[i], q2[i] = a1, a2
    return np.stack([q1, q2]).astype(np.float64)


def tie_rows(K, rng):
    rows = []
    ks = np.arange(-127, 127, dtype=np.float64)
    for scale in (1.0, 0.125, 32.0, 3.0):
        base = np.resize((ks + 0.5) * scale, K)
        base[0] = 127 * scale
        rows += [base, np.nextafter(base.astype(np.float16), np.float16(np.inf)).astype(np.float64),
                 np.nextafter(base.astype(np.float16), np.float16(-np.inf)).astype(np.float64)]
        q = rng.integers(-100, 100, K)
        h = rng.integers(-126, 126, K) + 0.5
        sec = scale * (q + h / 254.0)  # second-slice ties of the fixed ratio
        sec[0] = 127 * scale
        rows.append(sec)
    return np.array(rows, dtype=np.float16)


def rows_under_test():
    rng = np.random.default_rng(2024)
    K = 384
    gauss = wl.make_activations(71, 0, 24, K, outliers=True)
    tiny = (rng.standard_normal((4, K)) * 1e-6).astype(np.float16)
    mixed = (rng.standard_normal((4, K)) * 10.0 ** rng.uniform(-3, 3, (4, 1))).astype(np.float16)
    return np.concatenate([gauss, tie_rows(K, rng), tiny, mixed])


@pytest.mark.parametrize("window", [2.0 ** -14, 0.5], ids=["kernel_window", "exact_path_everywhere"])
@pytest.mark.parametrize("nslices,fixed", [(1, False), (2, False), (3, False), (2, True)])
def test_decomposition_decisions_match_fp64(nslices, fixed, window):
    x = rows_under_test()
    A, S = o.decompose_fixed_ratio(x) if fixed else o.decompose_activations(x, nslices)
    for m in range(x.shape[0]):
        codes, scales = decompose_emulated(x[m], nslices, fixed, window)
        assert np.array_equal(codes, A[:, m].astype(np.float64)), (m, nslices, fixed)
        assert np.array_equal(scales.view(np.uint32), S[:, m].view(np.uint32)), (m, nslices, fixed)


@pytest.mark.parametrize("window", [2.0 ** -14, 0.5], ids=["kernel_window", "exact_path_everywhere"])
def test_fused_fixed_decisions_match_fp64(window):
    x = rows_under_test()
    A, S = o.decompose_fixed_ratio(x)
    for m in range(x.shape[0]):
        codes = fused_fixed_emulated(x[m], float(S[0, m]), window)
        assert np.array_equal(codes, A[:, m].astype(np.float64)), m


def test_emulation_rejects_a_plain_fp32_rounding():
    """Without the exact test (and its window), fp32 estimates misround the
    tie rows: the check above is not vacuous."""
    x = rows_under_test()
    A, _ = o.decompose_activations(x, 1)
    wrong = 0
    for m in range(x.shape[0]):
        r = x[m].astype(np.float64)
        s = float(F32(np.abs(r).max() / 127.0))
        t = (r.astype(F32) * inv32(s)).astype(F32)
        wrong += int(np.sum(np.clip(rint32(t), -127, 127) != A[0, m]))
    assert wrong > 0


def test_first_residual_is_exact_in_fp32():
    """x - s_1 A_1 (A_1 the oracle's first slice) is an fp32 value: for A_1 = 0
    it is x, otherwise x sits on a grid coarser than s_1's ulp and |r| <= s_1
    / 2.  Rows: those above, plus rows spanning 10 decades with fp16
    subnormals."""
    rng = np.random.default_rng(77)
    wide = (rng.standard_normal((64, 512)) * 10.0 ** rng.uniform(-7, 4, (64, 512))).astype(np.float16)
    for x in (rows_under_test(), wide):
        A, S = o.decompose_activations(x, 2)
        r = x.astype(np.float64) - S[0][:, None].astype(np.float64) * A[0].astype(np.float64)  # exact in fp64
        assert np.array_equal(r.astype(F32).astype(np.float64), r)
        # the fp32 fma the kernels use gives it: fl32 of the exact value
        assert np.array_equal(np.abs(r).max(axis=1).astype(F32).view(np.uint32),
                              np.abs(r.astype(F32)).max(axis=1).view(np.uint32))
    # the single rounding matters: the product rounded to fp32 first, then
    # the difference, misses the exact residual on some elements
    x = rows_under_test()
    A, S = o.decompose_activations(x, 2)
    r = x.astype(np.float64) - S[0][:, None].astype(np.float64) * A[0].astype(np.float64)
    two = (x.astype(F32) - (S[0][:, None] * A[0].astype(F32)).astype(F32)).astype(F32)
    assert not np.array_equal(two.astype(np.float64), r)
