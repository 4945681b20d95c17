"""Number formats and exact rounding -- TEST INFRASTRUCTURE ONLY (see oracle/__init__).

Formats (QUADS, arXiv 2607.15810, section 2.2):
  * E2M1 ("FP4" paragraph): one sign bit plus a 3-bit magnitude code whose
    values are 0, 0.5, 1, 1.5, 2, 3, 4, 6.  Nibble layout: bit 3 = sign,
    bits 2..0 = magnitude code (the OCP FP4 layout: 2 exponent bits with
    bias 1, 1 mantissa bit).
  * E4M3 ("FP8" paragraph): 4 exponent bits, 3 mantissa bits, largest
    magnitude 448.  Reading: the OCP "E4M3FN" variant (bias 7, subnormals
    m * 2^-9, no infinities, 0x7F = NaN), the only E4M3 whose maximum is 448.
  * bf16 inputs and fp32 scales are IEEE binary16-brain / binary32.

Rounding: every rounding in the method is round-to-nearest, ties to the even
code ("RNE"), applied to the exact real value.  ``rne_to_grid`` does that for
any finite grid; ``rn32_rational`` rounds an exact rational to fp32.
"""

from fractions import Fraction

import numpy as np

# E2M1 magnitudes, indexed by the 3-bit magnitude code (section 2.2, "FP4").
E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E2M1_MAX = 6.0
# Largest E4M3 magnitude (section 2.2, "FP8").
E4M3_MAX = 448.0
E4M3_MAX_CODE = 0x7E


def e2m1_decode(nibble):
    """Signed value of E2M1 nibbles (uint8 array, low 4 bits used)."""
    nibble = np.asarray(nibble, dtype=np.uint8) & 0xF
    mag = E2M1_MAG[nibble & 0x7]
    return np.where(nibble & 0x8, -mag, mag)


def e4m3_decode(code):
    """Value of E4M3FN bytes, closed form.  NaN bytes (0x7F, 0xFF) give NaN."""
    code = np.asarray(code, dtype=np.int64) & 0xFF
    sign = np.where(code & 0x80, -1.0, 1.0)
    e = (code >> 3) & 0xF
    f = (code & 0x7).astype(np.float64)
    sub = f * 2.0 ** -9
    norm = (1.0 + f / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    val = sign * np.where(e == 0, sub, norm)
    return np.where((code & 0x7F) == 0x7F, np.nan, val)


# Non-negative finite E4M3 values, indexed by their byte code 0x00..0x7E.
# Byte order is value order for non-negative codes.
E4M3_GRID = e4m3_decode(np.arange(E4M3_MAX_CODE + 1))


def rne_to_grid(q, grid):
    """Index of the grid point nearest to each q >= 0, ties to the even index.

    ``grid`` is ascending, starts at 0 and holds exactly-representable fp64
    values whose pairwise midpoints are exact in fp64 (true for E2M1 and E4M3).
    Values above the last point saturate to it.  For E2M1 and E4M3 the index
    is the code, and an even index is an even mantissa, so "ties to even
    index" is round-half-to-even.

    ``q`` must lie on the same side of every midpoint as the exact real value
    it stands for (see nvfp4.py for why the fp64 quotients used here do).
    """
    q = np.asarray(q, dtype=np.float64)
    n = len(grid)
    idx = np.clip(np.searchsorted(grid, q, side="left"), 1, n - 1)
    lo = grid[idx - 1]
    hi = grid[idx]
    mid = (lo + hi) * 0.5
    up = (q > mid) | ((q == mid) & (idx % 2 == 0))
    return np.where(up, idx, idx - 1).astype(np.int64)


def _floor_log2(fr: Fraction) -> int:
    """floor(log2(fr)) for a positive Fraction, in exact integer arithmetic."""
    num, den = fr.numerator, fr.denominator
    e = num.bit_length() - den.bit_length()
    # now 2^(e-1) < fr < 2^(e+1)
    if e >= 0:
        if num < (den << e):
            e -= 1
    else:
        if (num << -e) < den:
            e -= 1
    return e


def rn32_rational(fr) -> np.float32:
    """Round an exact rational to the nearest fp32, ties to even (IEEE RN).

    Subnormals are kept; magnitudes beyond the fp32 range give +-inf.
    """
    fr = Fraction(fr)
    if fr == 0:
        return np.float32(0.0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = max(_floor_log2(a), -126)
    quantum = Fraction(2) ** (e - 23)          # spacing of fp32 values at exponent e
    scaled = a / quantum
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    value = Fraction(n) * quantum
    if value >= Fraction(2) ** 128:
        return np.float32(sign * np.inf)
    # value is exactly representable in fp32, so these conversions are exact
    return np.float32(sign * float(value))


def bf16_to_f64(bits):
    """Exact value of bf16 bit patterns (uint16 array)."""
    bits = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return bits.view(np.float32).astype(np.float64)


def f32_to_f64(x):
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def f64_to_bf16_rne(x):
    """bf16 bit patterns nearest to fp64 values, ties to even, subnormals kept.

    Exact: the rounding is done on the fp64 bit pattern (normal range) or on
    x * 2^133, an exact scaling (bf16 subnormal range), never via fp32.
    Values beyond the bf16 range are not expected here and raise.
    """
    x = np.asarray(x, dtype=np.float64)
    sign = np.signbit(x)
    a = np.abs(x)
    if np.any(~np.isfinite(a)) or np.any(a >= 2.0 ** 128):
        raise ValueError("value outside the bf16 range")
    bits = a.view(np.uint64)
    # normal bf16 range: keep 7 of the 52 mantissa bits, round half to even
    lsb = (bits >> np.uint64(45)) & np.uint64(1)
    rounded = (bits + np.uint64((1 << 44) - 1) + lsb) >> np.uint64(45)
    # rounded = (biased fp64 exponent << 7) | mantissa7, carry included
    exp64 = (rounded >> np.uint64(7)).astype(np.int64)
    man7 = (rounded & np.uint64(0x7F)).astype(np.int64)
    normal_bits = ((exp64 - 1023 + 127) << 7) | man7
    # subnormal bf16 range (below 2^-126): multiples of 2^-133
    small = a < 2.0 ** -126
    sub_bits = np.rint(np.where(small, a, 0.0) * 2.0 ** 133).astype(np.int64)  # half to even
    out = np.where(small, sub_bits, normal_bits)
    if np.any(out >= 0x7F80):
        raise ValueError("value rounds beyond the bf16 range")
    out = out | np.where(sign, 0x8000, 0)
    return out.astype(np.uint16)


def f32_bits(x):
    return np.asarray(x, dtype=np.float32).view(np.uint32)
