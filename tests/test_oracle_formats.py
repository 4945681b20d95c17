"""Pins for oracle/formats.py against the pages, closed forms and independent
library routines (CPU only)."""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F


def _golden(golden_dir):
    with open(os.path.join(golden_dir, "nvfp4_format.json")) as f:
        return json.load(f)


def test_e2m1_grid_matches_pages(golden_dir):
    g = _golden(golden_dir)
    vals = F.e2m1_decode(np.arange(16))
    assert list(vals[:8]) == g["e2m1_magnitudes"]["values"]
    assert list(-vals[8:]) == g["e2m1_magnitudes"]["values"]
    # sign bit on zero gives -0.0
    assert np.signbit(vals[8]) and not np.signbit(vals[0])


def test_e4m3_decode_against_torch_and_pages(golden_dir):
    g = _golden(golden_dir)
    codes = np.arange(256, dtype=np.uint8)
    ours = F.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()
    assert np.nanmax(ours) == g["e4m3_max"]["value"] == F.E4M3_GRID[-1]
    assert F.E4M3_GRID[0x7E] == 448.0 and len(F.E4M3_GRID) == 127
    assert np.all(np.diff(F.E4M3_GRID) > 0)
    # at most 1 + 3 significant bits (section 2.2, three mantissa bits)
    for v in F.E4M3_GRID[1:]:
        m, _ = np.frexp(v)
        assert (m * 16) == int(m * 16)


def _nearest_even_bruteforce(q: Fraction, grid):
    """Nearest grid index by exact distance, ties to the even index (Fraction)."""
    best = None
    for i, g in enumerate(grid):
        d = abs(q - Fraction(g))
        if best is None or d < best[0] or (d == best[0] and i % 2 == 0):
            best = (d, i)
    return best[1]


def test_rne_to_grid_bruteforce_e2m1():
    rng = np.random.default_rng(0)
    qs = [Fraction(n, 8) for n in range(0, 70)]                # every multiple of 1/8 to 8.6
    qs += [Fraction(int(a), int(b)) for a, b in rng.integers(1, 997, size=(300, 2))]
    for q in qs:
        got = F.rne_to_grid(np.float64(q), F.E2M1_MAG)
        exp = _nearest_even_bruteforce(q, F.E2M1_MAG)
        if q >= 6:
            exp = 7
        assert int(got) == exp, q


def test_rne_to_grid_e4m3_against_torch():
    rng = np.random.default_rng(1)
    # fp32 values in [0, 448]: torch's fp32 -> float8_e4m3fn conversion is RNE
    x = np.concatenate([
        rng.uniform(0, 448, 20000), np.exp2(rng.uniform(-14, 8.8, 20000)),
        (F.E4M3_GRID[:-1] + F.E4M3_GRID[1:]) / 2,                      # exact midpoints
        F.E4M3_GRID]).astype(np.float32)
    x = x[x <= 448]
    ours = F.rne_to_grid(x.astype(np.float64), F.E4M3_GRID)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref.astype(np.int64))
    # saturation above 448 (torch gives NaN there; the method saturates)
    assert np.all(F.rne_to_grid(np.array([448.0, 464.0, 465.0, 1e9]), F.E4M3_GRID) == 0x7E)


def test_rn32_rational_against_numpy():
    rng = np.random.default_rng(2)
    # doubles: np.float32(double) is exactly RN32 of that double
    d = np.concatenate([rng.standard_normal(3000) * np.exp2(rng.integers(-140, 120, 3000)),
                        np.exp2(rng.uniform(-149, -120, 500))])
    for v in d:
        assert F.rn32_rational(Fraction(float(v))) == np.float32(v)
    # exact fp32 midpoints and their neighbours (double rounding would fail here)
    for v in rng.standard_normal(300).astype(np.float32):
        nxt = np.nextafter(v, np.float32(np.inf))
        mid = (Fraction(float(v)) + Fraction(float(nxt))) / 2
        even = v if (v.view(np.uint32) & 1) == 0 else nxt
        assert F.rn32_rational(mid) == even
        assert F.rn32_rational(mid + Fraction(1, 2 ** 200)) == nxt
        assert F.rn32_rational(mid - Fraction(1, 2 ** 200)) == v
    assert F.rn32_rational(0) == 0
    assert F.rn32_rational(Fraction(2) ** 130) == np.inf


def test_bf16_roundtrip_against_torch():
    bits = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    bits = bits[((bits & 0x7F80) != 0x7F80)]                     # finite only
    ours = F.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(ours, ref)
    back = F.f64_to_bf16_rne(ours)
    assert np.array_equal(back, bits)


def test_f64_to_bf16_rne_against_torch_on_fp32_values():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(50000) * np.exp2(rng.integers(-135, 120, 50000)),
                        rng.standard_normal(1000)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = F.f64_to_bf16_rne(x.astype(np.float64))
    assert np.array_equal(ours, ref)


def test_f64_to_bf16_rne_no_double_rounding():
    # a double just above a bf16 midpoint that fp32 would round onto the midpoint
    lo = np.float64(1.0)
    mid = lo + 2.0 ** -8                   # midpoint between 1.0 and 1.0078125
    x = mid + 2.0 ** -40                   # above the midpoint, below fp32 resolution
    assert F.f64_to_bf16_rne(np.array([x]))[0] == 0x3F81     # rounds up
    assert F.f64_to_bf16_rne(np.array([mid]))[0] == 0x3F80   # tie to even
    assert np.float32(x) == np.float32(mid)                  # fp32 would lose it


@pytest.mark.parametrize("x,code", [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4),
                                    (2.5, 4), (3.5, 6), (5.0, 6), (5.0001, 7),
                                    (0.2499, 0), (0.2501, 1), (7.0, 7)])
def test_e2m1_ties_to_even_closed_form(x, code):
    assert int(F.rne_to_grid(np.float64(x), F.E2M1_MAG)) == code
