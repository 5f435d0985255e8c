"""Plain CPU oracle for the 4-bit weight-quantized matmul path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
product path (the HIP library and its Python binding) never does, and this
module imports nothing from it: the two share no code, tables or constants.

Everything here is slow and obviously correct: floating point is fp64, integer
work is exact int64, and each function follows the step order of the passage
it cites.  NumPy primitives (min/max, rint, matmul, einsum) are used as steps;
there is no blocking or reordering beyond the definitions.

Pages cited (title, section):

* [MSD]    "Multi-Scale Dequant: Eliminating Dequantization Bottleneck via
           Activation Decomposition for Efficient LLM Inference", Abstract.
* [MixPE]  "MixPE: Quantization and Hardware Co-design for Efficient LLM
           Inference", Abstract.
* [NF4]    "Fast NF4 Dequantization Kernels for Large Language Model
           Inference", Abstract.
* OCP Microscaling (MX) format definition: the E2M1 element and E8M0 scale
           encodings of MXFP4 (a published format the [MSD] page names).
* [DecDEC] "DecDEC: A Systems Approach to Advancing Low-Bit LLM
           Quantization", Abstract (residual compensation of salient
           channels) and "Builds on" list (names QLoRA, the source of the
           NormalFloat construction used for the NF4 codebook).

Where the pages leave a step open, the reading taken is stated in the
docstring of the function that implements it (marked READING).

Pins: every function below is pinned by ``tests/test_oracle_pins.py`` against
closed forms, brute force on tiny inputs, exact rational arithmetic or
invariants; none is "parity unpinned".
"""
from __future__ import annotations

from fractions import Fraction
from statistics import NormalDist

import numpy as np

INT4_LEVELS = 15  # codes 0..15
NF4_ZERO_INDEX = 7  # index of the exact-zero NF4 level
INT8_QMAX = 127  # symmetric int8 range [-127, 127]

FMT_INT4_ASYM = 0
FMT_NF4 = 1


# --------------------------------------------------------------------------
# rounding helpers (IEEE round-to-nearest-even everywhere)
# --------------------------------------------------------------------------
def fp32_rne(v):
    """Round fp64 value(s) to fp32 (nearest-even) and return them as fp64."""
    return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)


def fp16_from_fp32(v32):
    """Round fp32 value(s) to fp16 (nearest-even)."""
    return np.asarray(v32, dtype=np.float32).astype(np.float16)


# --------------------------------------------------------------------------
# NF4 codebook  ([NF4] Abstract: the 4-bit NormalFloat format; construction per
# QLoRA, listed in [DecDEC] "Builds on")
# --------------------------------------------------------------------------
def nf4_codebook_fp64() -> np.ndarray:
    """The 16 NormalFloat levels in fp64, before rounding to fp32.

    READING: the pages name NF4 but print no codebook.  The NormalFloat
    construction of QLoRA is taken: with the offset
    delta = 1/2 * ((1 - 1/30) + (1 - 1/32)), the 8 positive levels are the
    standard-normal quantiles at the first 8 of 9 evenly spaced
    probabilities from delta down to 1/2, the 7 negative levels are the
    negated quantiles at the first 7 of 8 evenly spaced probabilities over the
    same interval, an exact zero is added, and all 16 are divided by the
    largest.  Quantiles come from ``statistics.NormalDist.inv_cdf``.
    """
    nd = NormalDist()
    delta = 0.5 * ((1.0 - 1.0 / 30.0) + (1.0 - 1.0 / 32.0))
    pos_p = np.linspace(delta, 0.5, 9)[:-1]
    neg_p = np.linspace(delta, 0.5, 8)[:-1]
    pos = [nd.inv_cdf(float(p)) for p in pos_p]
    neg = [-nd.inv_cdf(float(p)) for p in neg_p]
    levels = sorted(pos + [0.0] + neg)
    top = max(levels)
    return np.array([v / top for v in levels], dtype=np.float64)


def nf4_codebook() -> np.ndarray:
    """NF4 levels rounded to fp32 (nearest-even); shape (16,), dtype float32."""
    return nf4_codebook_fp64().astype(np.float32)


# --------------------------------------------------------------------------
# INT4 asymmetric quantization  ([MixPE] Abstract: one scale and one zero
# point per quantization group)
# --------------------------------------------------------------------------
def quantize_int4_asym(wt: np.ndarray, G: int):
    """Quantize W^T [N][K] (fp32) per (row n, group of G along K).

    Steps for each group, all in fp64 (READING: the pages give only one
    scale and one zero point per group):

    1. lo = min(0, min w), hi = max(0, max w)  (range widened to hold 0, so the
       zero point is always a valid code);
    2. s = fp16(fp32((hi - lo) / 15))  (rounding staged fp64 -> fp32 -> fp16);
    3. z = clamp(rint(-lo / s), 0, 15)  (an integer, stored as fp16, +0 for 0);
    4. q = clamp(rint(w / s) + z, 0, 15);
    5. if s == 0 the group is all zero: q = z = 0.

    ``rint`` is round-half-to-even.  Returns (codes uint8 [N][K],
    scale float16 [N][K/G], zero float16 [N][K/G]).
    """
    wt = np.asarray(wt, dtype=np.float32)
    N, K = wt.shape
    assert K % G == 0
    w = wt.astype(np.float64).reshape(N, K // G, G)
    lo = np.minimum(w.min(axis=2), 0.0)
    hi = np.maximum(w.max(axis=2), 0.0)
    s16 = fp16_from_fp32(fp32_rne((hi - lo) / float(INT4_LEVELS)))
    s = s16.astype(np.float64)
    nz = s != 0.0
    safe = np.where(nz, s, 1.0)
    # "+ 0.0" turns a -0 (from lo == +0) into +0: the zero point is the
    # integer 0, stored as the fp16 bit pattern 0x0000.
    z = np.clip(np.rint(-lo / safe), 0, INT4_LEVELS) + 0.0
    q = np.clip(np.rint(w / safe[..., None]) + z[..., None], 0, INT4_LEVELS)
    z = np.where(nz, z, 0.0)
    q = np.where(nz[..., None], q, 0.0)
    return (q.reshape(N, K).astype(np.uint8), s16, z.astype(np.float16))


def dequant_int4_asym(codes, scale, zero, G: int) -> np.ndarray:
    """W' [N][K] in fp64: w' = s * (q - z), exact in fp64."""
    codes = np.asarray(codes)
    N, K = codes.shape
    q = codes.astype(np.float64).reshape(N, K // G, G)
    s = np.asarray(scale, dtype=np.float16).astype(np.float64)[..., None]
    z = np.asarray(zero, dtype=np.float16).astype(np.float64)[..., None]
    return (s * (q - z)).reshape(N, K)


# --------------------------------------------------------------------------
# NF4 quantization  ([NF4] Abstract)
# --------------------------------------------------------------------------
def quantize_nf4(wt: np.ndarray, B: int = 64, row_chunk: int = 256):
    """Quantize W^T [N][K] (fp32) to NF4 codes with a per-block absmax.

    For each (row n, block of B along K):

    1. a = fp16(max |w|)  (the absmax is exact in fp32, then rounded once);
    2. idx = argmin_i |w - c_i * a| over the 16 fp32 levels c_i, evaluated in
       fp64 (c_i * a is exact); READING: ties go to the lowest index;
    3. if a == 0 every code is the exact-zero level, index 7.

    Returns (codes uint8 [N][K], absmax float16 [N][K/B]).
    """
    wt = np.asarray(wt, dtype=np.float32)
    N, K = wt.shape
    assert K % B == 0
    c = nf4_codebook().astype(np.float64)
    codes = np.empty((N, K), dtype=np.uint8)
    absmax = np.empty((N, K // B), dtype=np.float16)
    for r0 in range(0, N, row_chunk):
        r1 = min(N, r0 + row_chunk)
        blk = wt[r0:r1].reshape(r1 - r0, K // B, B)
        a16 = fp16_from_fp32(np.abs(blk).max(axis=2))
        a = a16.astype(np.float64)
        levels = c[None, None, :] * a[..., None]  # exact products
        d = np.abs(blk.astype(np.float64)[..., :, None] - levels[..., None, :])
        idx = np.argmin(d, axis=-1)  # first minimum = lowest index
        idx = np.where((a == 0.0)[..., None], NF4_ZERO_INDEX, idx)
        codes[r0:r1] = idx.reshape(r1 - r0, K).astype(np.uint8)
        absmax[r0:r1] = a16
    return codes, absmax


def dequant_nf4(codes, absmax, B: int = 64) -> np.ndarray:
    """W' [N][K] in fp64: w' = c[idx] * a, exact in fp64."""
    codes = np.asarray(codes)
    N, K = codes.shape
    c = nf4_codebook().astype(np.float64)
    a = np.asarray(absmax, dtype=np.float16).astype(np.float64)
    return (c[codes.astype(np.int64)].reshape(N, K // B, B) * a[..., None]).reshape(N, K)


def dequant(fmt: int, codes, scale, zero, G: int) -> np.ndarray:
    if fmt == FMT_INT4_ASYM:
        return dequant_int4_asym(codes, scale, zero, G)
    if fmt == FMT_NF4:
        return dequant_nf4(codes, scale, G)
    raise ValueError(fmt)


# --------------------------------------------------------------------------
# nibble packing
# --------------------------------------------------------------------------
def pack_nibbles(codes) -> np.ndarray:
    """[N][K] codes (0..15) -> [N][K/2] bytes; byte j = q[2j] | q[2j+1] << 4.

    READING: the pages fix no layout.  The low nibble holds the even K index
    and rows stay K-contiguous (the PyTorch Linear weight layout, in keeping
    with the [NF4] page's drop-in compatibility aim).
    """
    codes = np.asarray(codes, dtype=np.uint8)
    assert codes.shape[1] % 2 == 0
    assert codes.max(initial=0) <= 15
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    N, H = packed.shape
    out = np.empty((N, 2 * H), dtype=np.uint8)
    out[:, 0::2] = packed & 0x0F
    out[:, 1::2] = packed >> 4
    return out


TILE_ROWS = 16   # weight rows (output columns) per tile
TILE_K = 128     # K positions per tile; one tile is 16 * 128 / 2 = 1024 bytes
# nibble p (bits 4p .. 4p+3) of a 4-byte word holds the code at K offset
# WORD_NIBBLE_K[p] of the word's 8 positions
WORD_NIBBLE_K = (0, 2, 4, 6, 1, 3, 5, 7)


def tile_offset(n: int, k: int, K: int):
    """Byte offset and nibble (0 low, 1 high) of code (n, k) in the stored form.

    READING: the pages fix no storage order.  The stored form is tiles of 16
    rows x 128 K positions, tile (n // 16, k // 128) at byte
    (n // 16 * K // 128 + k // 128) * 1024.  Inside a tile, "lane" l = 16 j + r
    owns 16 bytes at 16 l: four little-endian 4-byte words, word t holding the
    8 codes of row r at K positions 32 t + 8 j + 0..7, the code at offset o in
    nibble p where WORD_NIBBLE_K[p] = o (even offsets in nibbles 0-3, odd ones
    in nibbles 4-7).
    """
    nb, r = divmod(n, TILE_ROWS)
    kb, kk = divmod(k, TILE_K)
    t, rest = divmod(kk, 32)
    j, o = divmod(rest, 8)
    p = WORD_NIBBLE_K.index(o)
    lane = TILE_ROWS * j + r
    off = (nb * (K // TILE_K) + kb) * 1024 + lane * 16 + 4 * t + p // 2
    return off, p % 2


def pack_w4(codes) -> np.ndarray:
    """[N][K] codes (0..15) -> the stored form, [N][K/2] bytes (row tile nb
    occupies the bytes of rows 16 nb .. 16 nb + 15).  The arrangement of
    ``tile_offset``, written as reshapes and a transpose."""
    c = np.asarray(codes, dtype=np.uint32)
    assert c.max(initial=0) <= 15
    N, K = c.shape
    assert N % TILE_ROWS == 0 and K % TILE_K == 0
    c8 = c.reshape(N, K // 8, 8)  # 8-code words in K order
    word = np.zeros((N, K // 8), dtype=np.uint32)
    for p, o in enumerate(WORD_NIBBLE_K):
        word |= c8[:, :, o] << (4 * p)
    # row word w covers k = 8 w .. 8 w + 7, w = 16 kb + 4 t + j
    w = word.reshape(N // TILE_ROWS, TILE_ROWS, K // TILE_K, 4, 4)  # [nb][r][kb][t][j]
    tiles = np.ascontiguousarray(w.transpose(0, 2, 4, 1, 3))        # [nb][kb][j][r][t]
    return tiles.astype("<u4").view(np.uint8).reshape(N, K // 2)


def unpack_w4(stored) -> np.ndarray:
    """Inverse of ``pack_w4``."""
    b = np.ascontiguousarray(np.asarray(stored, dtype=np.uint8))
    N, H = b.shape
    K = 2 * H
    words = b.reshape(-1).view("<u4").reshape(N // TILE_ROWS, K // TILE_K, 4, TILE_ROWS, 4)  # [nb][kb][j][r][t]
    w = np.ascontiguousarray(words.transpose(0, 3, 1, 4, 2)).reshape(N, K // 8)           # [n][word]
    out = np.zeros((N, K // 8, 8), dtype=np.uint8)
    for p, o in enumerate(WORD_NIBBLE_K):
        out[:, :, o] = (w >> (4 * p)) & 15
    return out.reshape(N, K)


# --------------------------------------------------------------------------
# products
# --------------------------------------------------------------------------
def matmul_ref(x, w_deq) -> np.ndarray:
    """y = x . W'  with x [M][K] (fp16), W' given as W'^T [N][K]; fp64 result [M][N].

    The problem statement of mixed-precision GEMM ([MixPE] Abstract): low
    precision weights times higher precision activations.
    """
    xd = np.asarray(x).astype(np.float64)
    return xd @ np.asarray(w_deq, dtype=np.float64).T


def postscale_ref(fmt: int, x, codes, scale, zero, G: int) -> np.ndarray:
    """Per-group products scaled after accumulation ([MixPE] Abstract: scale and
    zero are shared inside a group, so the dequantization can come after the
    per-group product).

    y[m, n] = sum_g s[n, g] * sum_{k in g} x[m, k] * v[n, k], where v = q - z for
    INT4 and v = c[idx] for NF4.  Algebraically equal to ``matmul_ref`` of the
    dequantized weights; the fp64 results agree to rounding.
    """
    xd = np.asarray(x).astype(np.float64)
    M, K = xd.shape
    codes = np.asarray(codes)
    N = codes.shape[0]
    ng = K // G
    if fmt == FMT_INT4_ASYM:
        z = np.asarray(zero, dtype=np.float16).astype(np.float64)
        v = codes.astype(np.float64).reshape(N, ng, G) - z[..., None]
    else:
        c = nf4_codebook().astype(np.float64)
        v = c[codes.astype(np.int64)].reshape(N, ng, G)
    s = np.asarray(scale, dtype=np.float16).astype(np.float64)
    part = np.einsum("mgk,ngk->mgn", xd.reshape(M, ng, G), v)  # per-group sums
    return np.einsum("mgn,ng->mn", part, s)


# --------------------------------------------------------------------------
# Multi-Scale Dequant activation decomposition  ([MSD] Abstract)
# --------------------------------------------------------------------------
def decompose_activations(x, nslices: int = 2):
    """Split fp16 activations [M][K] into ``nslices`` int8 slices with per-token
    fp32 scales, so that x ~= sum_j s_j[m] * A_j[m, k].

    READING of [MSD] (the activations are split into several low-precision
    parts, two int8 passes for integer weights): a greedy residual
    quantization.  With r = x (in fp64), for each pass j:

    1. s_j = fp32(max_k |r[m, k]| / 127);
    2. A_j = clamp(rint(r / s_j), -127, 127)  (round-half-to-even);
    3. r <- r - s_j * A_j  (exact in fp64 for up to three passes: every
       residual is a short sum of fp16 and fp32 x int8 terms);
    4. a pass whose scale is 0 yields an all-zero slice.

    ``nslices`` = 1 is one int8 quantization of the activations; 3 adds a
    third pass on the second residual.

    Returns (A int8 [nslices][M][K], s float32 [nslices][M]).
    """
    r = np.asarray(x).astype(np.float64)
    M, K = r.shape
    A = np.zeros((nslices, M, K), dtype=np.int8)
    S = np.zeros((nslices, M), dtype=np.float32)
    for j in range(nslices):
        amax = np.abs(r).max(axis=1) if K else np.zeros(M)
        s = fp32_rne(amax / float(INT8_QMAX))
        nz = s != 0.0
        safe = np.where(nz, s, 1.0)
        a = np.clip(np.rint(r / safe[:, None]), -INT8_QMAX, INT8_QMAX)
        a = np.where(nz[:, None], a, 0.0)
        A[j] = a.astype(np.int8)
        S[j] = s.astype(np.float32)
        r = r - s[:, None] * a
    return A, S


FIXED_RATIO = 254  # s_2 = s_1 / 254 in the fixed-ratio decomposition


def decompose_fixed_ratio(x):
    """Two-slice decomposition with a fixed scale ratio, s_2 = s_1 / 254.

    READING of [MSD] Abstract (the pages do not say how the second scale is
    chosen): instead of the residual's own absmax, the second slice uses the
    first slice's step divided by 254.  Since |r_1| <= s_1 / 2, the second
    slice's codes then lie in [-127, 127] without clamping, and
    x ~= (s_1 / 254) * (254 * A_1 + A_2): the two integer products combine
    exactly as 254 * D_1 + D_2 before any conversion to floating point.

    Per token m, in fp64:

    1. s_1 = fp32(max_k |x[m, k]| / 127);
    2. A_1 = clamp(rint(x / s_1), -127, 127);
    3. r_1 = x - s_1 * A_1  (exact);
    4. A_2 = clamp(rint((254 * r_1) / s_1), -127, 127)  (254 * r_1 is exact,
       the division one correctly rounded fp64 operation);
    5. s_1 = 0 gives all-zero slices.

    Returns (A int8 [2][M][K], s float32 [2][M]); s[1] = fp32(s_1 / 254) is
    reported for reference only -- results use the exact ratio.
    """
    xd = np.asarray(x).astype(np.float64)
    M, K = xd.shape
    amax = np.abs(xd).max(axis=1) if K else np.zeros(M)
    s1 = fp32_rne(amax / float(INT8_QMAX))
    nz = s1 != 0.0
    safe = np.where(nz, s1, 1.0)
    a1 = np.where(nz[:, None], np.clip(np.rint(xd / safe[:, None]), -INT8_QMAX, INT8_QMAX), 0.0)
    r1 = xd - s1[:, None] * a1
    a2 = np.where(nz[:, None], np.clip(np.rint((FIXED_RATIO * r1) / safe[:, None]), -INT8_QMAX, INT8_QMAX), 0.0)
    A = np.stack([a1, a2]).astype(np.int8)
    S = np.stack([s1, fp32_rne(s1 / FIXED_RATIO)]).astype(np.float32)
    return A, S


def msd_accumulators(slices, codes, zero, G: int) -> np.ndarray:
    """Exact integer per-group products D_j[m, g, n] = sum_{k in g} A_j[m, k] *
    (q[n, k] - z[n, g]), as int64 [nslices][M][K/G][N].

    These are what the int8 matrix cores produce in [MSD]: slices multiplied
    directly with the integer weights, with no conversion of the weights to a
    floating type.
    """
    A = np.asarray(slices).astype(np.int64)
    J, M, K = A.shape
    codes = np.asarray(codes)
    N = codes.shape[0]
    ng = K // G
    z = np.asarray(zero, dtype=np.float16).astype(np.int64)
    qz = codes.astype(np.int64).reshape(N, ng, G) - z[..., None]
    return np.einsum("jmgk,ngk->jmgn", A.reshape(J, M, ng, G), qz)


def msd_result(tok_scale, acc, scale) -> np.ndarray:
    """y[m, n] = sum_j s_j[m] * sum_g s[n, g] * D_j[m, g, n]  in fp64
    (group scales applied after the integer accumulation, [MixPE] Abstract;
    slices recombined by their scales, [MSD] Abstract)."""
    S = np.asarray(tok_scale, dtype=np.float32).astype(np.float64)
    D = np.asarray(acc).astype(np.float64)
    s = np.asarray(scale, dtype=np.float16).astype(np.float64)  # [N][ng]
    per_slice = np.einsum("jmgn,ng->jmn", D, s)
    return np.einsum("jm,jmn->mn", S, per_slice)


def msd_fixed_result(s1, acc, scale) -> np.ndarray:
    """Fixed-ratio recombination: the integer combine E = 254 * D_1 + D_2 per
    group (exact), then y[m, n] = (s_1[m] / 254) * sum_g s[n, g] * E[m, g, n]
    in fp64."""
    D = np.asarray(acc).astype(np.int64)
    E = (FIXED_RATIO * D[0] + D[1]).astype(np.float64)
    s = np.asarray(scale, dtype=np.float16).astype(np.float64)
    t = np.asarray(s1, dtype=np.float32).astype(np.float64) / FIXED_RATIO
    return t[:, None] * np.einsum("mgn,ng->mn", E, s)


def msd_fixed_matmul(x, codes, scale, zero, G: int):
    """Full fixed-ratio MSD product: decompose, integer products, combine."""
    A, S = decompose_fixed_ratio(x)
    D = msd_accumulators(A, codes, zero, G)
    return msd_fixed_result(S[0], D, scale), A, S, D


def msd_matmul(x, codes, scale, zero, G: int, nslices: int = 2):
    """Full MSD product: decompose, integer per-group products, rescale."""
    A, S = decompose_activations(x, nslices)
    D = msd_accumulators(A, codes, zero, G)
    return msd_result(S, D, scale), A, S, D


# --------------------------------------------------------------------------
# MXFP4: 4-bit E2M1 elements with one E8M0 (power-of-two) scale per 32
# consecutive K positions  ([MSD] Abstract: MXFP4 weights, two-pass MXFP4
# decomposition of the activations).  Element and scale encodings follow the
# published OCP Microscaling (MX) format definition.
# --------------------------------------------------------------------------
MX_BLOCK = 32
E2M1_MAX = 6.0


def e2m1_value(code: int) -> float:
    """Value of a 4-bit E2M1 code: bit 3 sign, bits 2..1 exponent (bias 1),
    bit 0 mantissa; exponent 0 is subnormal (0 or 0.5)."""
    sign = -1.0 if code & 8 else 1.0
    e, m = (code >> 1) & 3, code & 1
    mag = 0.5 * m if e == 0 else 2.0 ** (e - 1) * (1.0 + 0.5 * m)
    return sign * mag


def mx_scale_exponent(amax):
    """READING of the scale rule (the pages do not give one): the smallest
    integer e with amax <= 6 * 2^e, so no element exceeds the largest E2M1
    magnitude (no saturation); e is clamped to the E8M0 range [-127, 127] and
    an all-zero block takes e = -127.  This rule reproduces the single-pass
    MXFP8 figure of the MSD abstract (see the pins)."""
    a = np.asarray(amax, dtype=np.float64)
    e = np.zeros(a.shape, dtype=np.int64)
    nz = a > 0
    # start from ceil(log2(a / 6)) and correct it against exact comparisons
    guess = np.ceil(np.log2(np.where(nz, a, 1.0) / E2M1_MAX)).astype(np.int64)
    guess = np.where(E2M1_MAX * np.ldexp(1.0, guess) < a, guess + 1, guess)
    guess = np.where(E2M1_MAX * np.ldexp(1.0, guess - 1) >= a, guess - 1, guess)
    e = np.where(nz, guess, -127)
    return np.clip(e, -127, 127)


def e2m1_round(t) -> np.ndarray:
    """E2M1 code nearest to t (|t| <= 6 expected; clamped), ties to the even
    code (mantissa bit 0); a result of magnitude zero carries no sign."""
    t = np.asarray(t, dtype=np.float64)
    mags = np.array([e2m1_value(c) for c in range(8)])
    a = np.minimum(np.abs(t), E2M1_MAX)
    d = np.abs(a[..., None] - mags)
    best = d.min(axis=-1, keepdims=True)
    tie = (d == best)
    even = tie & (np.arange(8) % 2 == 0)
    code = np.where(tie.sum(axis=-1) > 1, np.argmax(even, axis=-1), np.argmax(tie, axis=-1))
    neg = (t < 0) & (code != 0)
    return (code + 8 * neg).astype(np.uint8)


def e2m1_decode(codes) -> np.ndarray:
    table = np.array([e2m1_value(c) for c in range(16)])
    return table[np.asarray(codes, dtype=np.int64)]


def mx_quantize(v):
    """MXFP4 of v [..., K] (K a multiple of 32): codes uint8 [..., K] and
    scale exponents int [..., K/32]; value = e2m1(code) * 2^e of its block."""
    v = np.asarray(v, dtype=np.float64)
    shp = v.shape
    b = v.reshape(shp[:-1] + (shp[-1] // MX_BLOCK, MX_BLOCK))
    e = mx_scale_exponent(np.abs(b).max(axis=-1))
    codes = e2m1_round(b / np.ldexp(1.0, e)[..., None])  # exact: a power-of-two scaling
    return codes.reshape(shp), e


def mx_dequant(codes, e) -> np.ndarray:
    c = e2m1_decode(codes)
    shp = c.shape
    b = c.reshape(shp[:-1] + (shp[-1] // MX_BLOCK, MX_BLOCK))
    return (b * np.ldexp(1.0, np.asarray(e, dtype=np.int64))[..., None]).reshape(shp)


def quantize_mxfp4(wt):
    """MXFP4 weights from W^T fp32 [N][K]: codes [N][K], exponents [N][K/32]
    (stored as E8M0 bytes e + 127)."""
    return mx_quantize(np.asarray(wt, dtype=np.float32))


def decompose_mxfp4(x, nslices: int = 2):
    """[MSD] two-pass MXFP4 decomposition of fp16 activations [M][K]: slice 1
    is MXFP4(x), slice j + 1 is MXFP4 of the residual left by slices 1..j, all
    in fp64 (the residuals are exact: each is a short sum of fp16 and
    power-of-two-scaled E2M1 values).  Returns codes [nslices][M][K] and
    exponents [nslices][M][K/32].

    Bound: pass 1 leaves |r| <= 2^e1 (half the widest E2M1 gap, 2, at the
    top binade).  Pass 2 then has e2 <= e1 - 2.  With e2 = e1 - 2 the
    residual lies within 4 * 2^e2, below the top binade, so it is left within
    half the gap of [2, 4]: 2^(e2 - 1) = 2^(e1 - 3); with e2 <= e1 - 3 it is
    left within 2^e2 <= 2^(e1 - 3).  So |x - slice 1 - slice 2| <= 2^(e1 - 3)
    = 2^(e1 + 3) / 64 per block, where 2^(e1 + 3) is the power of two just
    above the first slice's largest value 6 * 2^e1: the 1/64 per block of the
    MSD abstract (the bound is attained).  Against the block's maximum,
    2^(e1 - 3) < amax / 24 (amax > 3 * 2^e1 by the scale rule)."""
    r = np.asarray(x).astype(np.float64)
    M, K = r.shape
    C = np.zeros((nslices, M, K), dtype=np.uint8)
    E = np.zeros((nslices, M, K // MX_BLOCK), dtype=np.int64)
    for j in range(nslices):
        C[j], E[j] = mx_quantize(r)
        r = r - mx_dequant(C[j], E[j])
    return C, E


def mx_matmul(x_codes, x_exp, w_codes, w_exp) -> np.ndarray:
    """y[m, n] = sum_j sum_k xhat_j[m, k] * what[n, k] in fp64 (every operand is
    an exact power-of-two multiple of an E2M1 value)."""
    W = mx_dequant(w_codes, w_exp)
    y = 0.0
    for j in range(np.asarray(x_codes).shape[0]):
        y = y + mx_dequant(x_codes[j], x_exp[j]) @ W.T
    return y


def pack_mx(codes) -> np.ndarray:
    """MXFP4 weight codes [N][K] (N % 16 == 0, K % 128 == 0) -> packed bytes in
    1 KB tiles of 16 rows x 128 K positions, tile (nb, kb) at byte offset
    (nb * K/128 + kb) * 1024 (the INT4 tile order).  Inside a tile, the 16
    bytes at 16 * (16 j + r) hold row r's K positions 128 kb + 32 j + e,
    e = 0..31, position e in byte e / 2, low nibble first: one 16-byte load
    per lane is the B operand of a 16x16x128 block-scaled fp4 product."""
    codes = np.asarray(codes, dtype=np.uint8)
    N, K = codes.shape
    t = codes.reshape(N // 16, 16, K // 128, 4, 16, 2)  # nb, r, kb, j, byte, nibble
    bytes_ = (t[..., 0] | (t[..., 1] << 4)).astype(np.uint8)  # nb, r, kb, j, byte
    return np.ascontiguousarray(bytes_.transpose(0, 2, 3, 1, 4)).reshape(-1)


def unpack_mx(packed, N: int, K: int) -> np.ndarray:
    b = np.asarray(packed, dtype=np.uint8).reshape(N // 16, K // 128, 4, 16, 16)  # nb, kb, j, r, byte
    codes = np.stack([b & 15, b >> 4], axis=-1)  # nb, kb, j, r, byte, nibble
    return np.ascontiguousarray(codes.transpose(0, 3, 1, 2, 4, 5)).reshape(N, K)


# --------------------------------------------------------------------------
# Multi-Scale Dequant for the KV cache in decode attention  ([MSD] Abstract:
# the KV cache is quantized and the activations on the other side of each
# product -- the queries for the scores, the attention weights for the values
# -- are decomposed instead of dequantizing the cache)
# --------------------------------------------------------------------------
ATTN_CHUNK = 256  # tokens per block of attention weights decomposed together


def attention_ref(q, k_deq, v_deq, n_kv: int) -> np.ndarray:
    """Plain decode attention in fp64 (one query token per head).

    q [Hq][d]; k_deq, v_deq [Hkv][L][d]; query head g attends with key/value
    head g // (Hq / Hkv) (grouped-query attention); scores scaled by 1/sqrt(d),
    softmax over the L positions."""
    q = np.asarray(q).astype(np.float64)
    Hq, d = q.shape
    G = Hq // n_kv
    out = np.zeros((Hq, d))
    for g in range(Hq):
        h = g // G
        s = np.asarray(k_deq[h], dtype=np.float64) @ q[g] / np.sqrt(d)
        p = np.exp(s - s.max())
        out[g] = (p / p.sum()) @ np.asarray(v_deq[h], dtype=np.float64)
    return out


def msd_attention(q, k_codes, k_scale, k_zero, v_codes, v_scale, v_zero, n_kv: int, chunk: int = ATTN_CHUNK):
    """Decode attention with an INT4 KV cache and Multi-Scale Dequant on both
    products, in fp64 with exact integer products.

    READING (the page names the idea and its traffic benefit, not the steps):
    * K and V are INT4 asymmetric with one scale and zero point per token and
      head (a group spans the head dimension d): k[t] = sK[t] (qK[t] - zK[t]).
    * Scores: the queries of each key/value head are split into two int8
      slices per query head (``decompose_activations``);
      D_j[g, t] = sum_d A_j[g, d] (qK[t, d] - zK[t]) exactly, and
      score[g, t] = sK[t] sum_j s_j[g] D_j[g, t] / sqrt(d).
    * Softmax: p = exp(score - max_t score), l = sum_t p.
    * Values: the per-token value scale is folded into the weights,
      w[g, t] = p[g, t] sV[t]; each block of ``chunk`` positions of w is split
      into two int8 slices per query head (same decomposition), and
      E_j[g, n] = sum_t B_j[g, t] (qV[t, n] - zV[t]) exactly;
      o[g, n] = sum_blocks sum_j r_j[g] E_j[g, n] / l[g].

    k_codes, v_codes [Hkv][L][d] uint8; scales, zeros [Hkv][L] fp16.
    Returns o [Hq][d] fp64."""
    q = np.asarray(q)
    Hq, d = q.shape
    G = Hq // n_kv
    L = np.asarray(k_codes).shape[1]
    out = np.zeros((Hq, d))
    for h in range(n_kv):
        rows = slice(h * G, (h + 1) * G)
        A, S = decompose_activations(q[rows], 2)                      # [2][G][d], [2][G]
        kz = np.asarray(k_zero[h], dtype=np.float16).astype(np.int64)
        qk = np.asarray(k_codes[h]).astype(np.int64) - kz[:, None]    # [L][d]
        D = np.einsum("jgd,td->jgt", A.astype(np.int64), qk)          # exact
        sK = np.asarray(k_scale[h], dtype=np.float16).astype(np.float64)
        score = sK[None, :] * np.einsum("jg,jgt->gt", S.astype(np.float64), D.astype(np.float64)) / np.sqrt(d)
        p = np.exp(score - score.max(axis=1, keepdims=True))
        l = p.sum(axis=1)
        sV = np.asarray(v_scale[h], dtype=np.float16).astype(np.float64)
        w = p * sV[None, :]
        vz = np.asarray(v_zero[h], dtype=np.float16).astype(np.int64)
        qv = np.asarray(v_codes[h]).astype(np.int64) - vz[:, None]    # [L][d]
        o = np.zeros((G, d))
        for c0 in range(0, L, chunk):
            Bc, R = decompose_activations(w[:, c0:c0 + chunk], 2)     # [2][G][chunk], [2][G]
            E = np.einsum("jgt,tn->jgn", Bc.astype(np.int64), qv[c0:c0 + chunk])
            o += np.einsum("jg,jgn->gn", R.astype(np.float64), E.astype(np.float64))
        out[rows] = o / l[:, None]
    return out


# --------------------------------------------------------------------------
# residual compensation of salient channels  ([DecDEC] Abstract)
# --------------------------------------------------------------------------
def residual_fp16(wt, w_deq) -> np.ndarray:
    """The residual matrix R = W - W' that [DecDEC] keeps in host memory, as
    fp16 [K][N] (row k: input channel k's residuals for every output n).

    READING: the pages do not fix the residual's precision or layout; here it
    is the exact fp64 difference rounded once to fp16, stored channel-major so
    that fetching one salient channel reads one contiguous row.
    """
    wt64 = np.asarray(wt, dtype=np.float32).astype(np.float64)  # [N][K]
    return (wt64 - np.asarray(w_deq, dtype=np.float64)).T.astype(np.float16)


def salient_channels(x, k: int) -> np.ndarray:
    """The k salient input channels of activations x [M][K], as int32 indices.

    READING of [DecDEC] (salient channels are the ones where the current
    step's activations have outliers, chosen anew at every decode step):
    channel c scores max_m |x[m, c]|; the k highest scores are taken, ordered
    by score (descending) and, among equal scores, by channel index
    (ascending).
    """
    a = np.abs(np.asarray(x).astype(np.float64))
    score = a.max(axis=0) if a.shape[0] else np.zeros(a.shape[1])
    order = np.lexsort((np.arange(score.size), -score))  # primary key: -score
    return order[:k].astype(np.int32)


def residual_correction(x, resid16, idx) -> np.ndarray:
    """corr[m, n] = sum over selected channels c of x[m, c] * R[c, n], fp64."""
    xd = np.asarray(x).astype(np.float64)
    idx = np.asarray(idx, dtype=np.int64)
    R = np.asarray(resid16, dtype=np.float16).astype(np.float64)
    return xd[:, idx] @ R[idx, :]


# --------------------------------------------------------------------------
# exact rational product for tiny shapes
# --------------------------------------------------------------------------
def matmul_exact(x, w_deq):
    """Exact rational x . W' for tiny shapes (pure Python Fractions)."""
    xf = [[Fraction(float(v)) for v in row] for row in np.asarray(x).astype(np.float64)]
    wf = [[Fraction(float(v)) for v in row] for row in np.asarray(w_deq, dtype=np.float64)]
    return [[sum((a * b for a, b in zip(xr, wr)), Fraction(0)) for wr in wf] for xr in xf]


# --------------------------------------------------------------------------
# parity metric
# --------------------------------------------------------------------------
def max_row_rel_l2(y, y_ref) -> float:
    """max over rows m of ||y[m] - y_ref[m]||_2 / ||y_ref[m]||_2."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    num = np.linalg.norm(y - y_ref, axis=1)
    den = np.linalg.norm(y_ref, axis=1)
    den = np.where(den == 0.0, 1.0, den)
    return float((num / den).max(initial=0.0))
