"""Study of the MXFP4 two-pass reading: effective bits and worst block error
of several scale rules, against the figures of the Multi-Scale Dequant page
("Multi-Scale Dequant: Eliminating Dequantization Bottleneck via Activation
Decomposition for Efficient LLM Inference", Abstract: single-pass MXFP8
5.24 effective bits; two-pass MXFP4 near 6.6 effective bits with an error
bound of 1/64 per block).  The page gives neither the scale rule, nor the
data, nor the definition of effective bits; this script tabulates the
candidates (test infrastructure: it uses the oracle's E2M1 arithmetic and
touches nothing of the library).

Rules for a pass with block maximum a (E2M1 largest magnitude 6):
  nosat      smallest e with a <= 6 * 2^e (no element saturates; the oracle's);
  ocp        e = floor(log2 a) - 2, elements beyond 6 * 2^e clamp to 6;
  e1-k       second pass only: e2 = e1 - k, a fixed offset from the first
             pass's exponent (elements beyond 6 * 2^e2 clamp).
Definitions of effective bits, over all elements:
  rms        -log2(rms(err) / rms(x))
  enob       (SNR_dB - 1.76) / 6.02
Worst block error: max over blocks of max|err| / amax, and of max|err| /
2^(e1 + 3) (2^(e1 + 3) is the power of two just above 6 * 2^e1, the largest
value the first slice can hold).

Run: python -m oracle.mx_readings  (prints the markdown table).
"""
from __future__ import annotations

import numpy as np

from .w4_oracle import E2M1_MAX, MX_BLOCK, e2m1_decode, e2m1_round, mx_scale_exponent

E4M3_MAX = 448.0


def e4m3_grid() -> np.ndarray:
    """Non-negative E4M3 values (3 mantissa bits, bias 7, subnormals, max 448)."""
    vals = {m / 8 * 2.0 ** -6 for m in range(8)}
    vals |= {(1 + m / 8) * 2.0 ** (e - 7) for e in range(1, 16) for m in range(8)
             if (1 + m / 8) * 2.0 ** (e - 7) <= E4M3_MAX}
    return np.array(sorted(vals))


def round_to_grid(t, grid) -> np.ndarray:
    """Nearest grid magnitude (clamped to the top), ties to the even index."""
    t = np.asarray(t, dtype=np.float64)
    a = np.minimum(np.abs(t), grid[-1])
    i = np.clip(np.searchsorted(grid, a), 1, len(grid) - 1)
    lo, hi = grid[i - 1], grid[i]
    q = np.where(a - lo < hi - a, lo, np.where(a - lo > hi - a, hi, np.where((i - 1) % 2 == 0, lo, hi)))
    return np.sign(t) * q


def exp_nosat(amax, top) -> np.ndarray:
    """Smallest e with amax <= top * 2^e (exact comparisons); -127 for 0."""
    a = np.asarray(amax, dtype=np.float64)
    g = np.ceil(np.log2(np.where(a > 0, a, 1.0) / top))
    g = np.where(top * np.ldexp(1.0, g.astype(np.int64)) < a, g + 1, g)
    g = np.where(top * np.ldexp(1.0, (g - 1).astype(np.int64)) >= a, g - 1, g)
    return np.where(a > 0, g, -127).astype(np.int64)


def exp_ocp(amax) -> np.ndarray:
    """floor(log2 amax) - 2 (the E2M1 element's largest exponent), -127 for 0."""
    a = np.asarray(amax, dtype=np.float64)
    return np.where(a > 0, np.floor(np.log2(np.where(a > 0, a, 1.0))) - 2, -127).astype(np.int64)


def e2m1_pass(v, e) -> np.ndarray:
    """v [B][32] quantized to E2M1 x 2^e per block (the oracle's rounding)."""
    s = np.ldexp(1.0, e)[:, None]
    return e2m1_decode(e2m1_round(v / s)) * s


def first_exponent(b, rule: str) -> np.ndarray:
    amax = np.abs(b).max(axis=1)
    return mx_scale_exponent(amax) if rule == "nosat" else exp_ocp(amax)


def two_pass_error(b, rule1: str, rule2: str):
    """Residual after two MXFP4 passes over blocks b [B][32]; returns (r2, e1)."""
    e1 = first_exponent(b, rule1)
    r1 = b - e2m1_pass(b, e1)
    a1 = np.abs(r1).max(axis=1)
    if rule2 == "nosat":
        e2 = exp_nosat(a1, E2M1_MAX)
    elif rule2 == "ocp":
        e2 = exp_ocp(a1)
    else:  # "e1-k"
        e2 = e1 - int(rule2.split("-")[1])
    return r1 - e2m1_pass(r1, e2), e1


def mxfp8_error(b) -> np.ndarray:
    """Single-pass MXFP8 (E4M3 elements, no-saturation scale rule)."""
    e = exp_nosat(np.abs(b).max(axis=1), E4M3_MAX)
    s = np.ldexp(1.0, e)[:, None]
    return b - round_to_grid(b / s, e4m3_grid()) * s


def rms_bits(x, err) -> float:
    return float(-np.log2(np.sqrt(np.mean(err ** 2)) / np.sqrt(np.mean(x ** 2))))


def enob(x, err) -> float:
    return float((10 * np.log10(np.sum(x ** 2) / np.sum(err ** 2)) - 1.76) / 6.02)


def blocks(dist: str, n_blocks: int, seed: int = 10) -> np.ndarray:
    """fp16-representable blocks of 32: standard normal, or uniform on [-1, 1]."""
    rng = np.random.default_rng(seed)
    v = rng.standard_normal(n_blocks * MX_BLOCK) if dist == "normal" else rng.uniform(-1, 1, n_blocks * MX_BLOCK)
    return v.astype(np.float16).astype(np.float64).reshape(n_blocks, MX_BLOCK)


def table(n_blocks: int = 40000):
    rows = []
    for dist in ("normal", "uniform"):
        b = blocks(dist, n_blocks)
        amax = np.abs(b).max(axis=1)
        err = mxfp8_error(b)
        rows.append((dist, "MXFP8, one pass", "nosat", rms_bits(b, err), enob(b, err),
                     float(np.max(np.abs(err).max(axis=1) / amax)), None))
        for rule1 in ("nosat", "ocp"):
            for rule2 in ("nosat", "ocp", "e1-1", "e1-2", "e1-3", "e1-4"):
                r2, e1 = two_pass_error(b, rule1, rule2)
                worst = np.abs(r2).max(axis=1)
                rows.append((dist, f"MXFP4, two passes ({rule1} / {rule2})", rule1, rms_bits(b, r2), enob(b, r2),
                             float(np.max(worst / amax)), float(np.max(worst / np.ldexp(1.0, e1 + 3)))))
    return rows


def main():
    print("| data | scheme (pass 1 / pass 2 rule) | rms bits | ENOB | worst max|err|/amax "
          "| worst max|err|/2^(e1+3) |")
    print("|---|---|---|---|---|---|")
    for dist, name, _, rb, en, wa, w8 in table():
        w8s = "-" if w8 is None else f"1/{1 / w8:.1f}"
        print(f"| {dist} | {name} | {rb:.2f} | {en:.2f} | 1/{1 / wa:.1f} | {w8s} |")


if __name__ == "__main__":
    main()
