"""Pins for oracle/mx.py (CPU only): the MX block rule worked by hand, ties
and saturation, a Fraction brute force of element rounding, and the GEMM as
an exact rational sum on a tiny case."""

import itertools
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats as F
from oracle import mx as M


def _block(vals):
    x = np.zeros((1, 32))
    x[0, :len(vals)] = vals
    return x


def test_hand_example_fp8():
    # amax 56 = 1.75 * 2^5 -> E = 5 - 8 = -3; the elements are x * 8
    x = _block([56.0, 1.0, -0.5, 0.125, 3.0 / 64])
    codes, sc = M.quantize(x, "fp8")
    assert sc[0, 0] == 127 - 3
    # 448 = 0x7E; 8 = 0 1010 000 = 0x50; -4 = 0xC8; 1 = 0x38; 3/8 = 1.5*2^-2 = 0 0101 100 = 0x2C
    assert list(codes[0, :5]) == [0x7E, 0x50, 0xC8, 0x38, 0x2C]
    assert np.array_equal(M.dequantize(codes, sc, "fp8"), x)


def test_hand_example_fp4():
    # amax 6 = 1.5 * 2^2 -> E = 2 - 2 = 0: the values are on the E2M1 grid
    x = _block([6.0, -0.5, 3.0, 1.5])
    codes, sc = M.quantize(x, "fp4")
    assert sc[0, 0] == 127
    assert codes[0, 0] == (0x7 | (0x9 << 4))        # 6 low nibble, -0.5 high nibble
    assert codes[0, 1] == (0x5 | (0x3 << 4))        # 3, 1.5
    assert np.array_equal(M.dequantize(codes, sc, "fp4"), x)


def test_saturation_and_ties():
    # fp8: amax 500 (E = 0): 500 -> 448; ties at 1.0625 -> 1 (even), 1.1875 -> 1.25 (even)
    x = _block([500.0, 1.0625, 1.1875, 465.0, 460.0])
    codes, sc = M.quantize(x, "fp8")
    dq = M.dequantize(codes, sc, "fp8")[0, :5]
    assert sc[0, 0] == 127 and list(dq) == [448.0, 1.0, 1.25, 448.0, 448.0]
    # fp4: amax 7 (E = 0): 7 -> 6, 5 -> 4 (tie to even), 2.5 -> 2, 0.25 -> 0, -0.75 -> -1
    x = _block([7.0, 5.0, 2.5, 0.25, -0.75])
    codes, sc = M.quantize(x, "fp4")
    dq = M.dequantize(codes, sc, "fp4")[0, :5]
    assert sc[0, 0] == 127 and list(dq) == [6.0, 4.0, 2.0, 0.0, -1.0]


def test_zero_block_and_range_ends():
    x = np.zeros((2, 64))
    x[1, 32] = 2.0 ** 127 * 1.5           # the shared exponent clamps at 127 - 8
    x[1, 0] = 2.0 ** -133                 # the smallest bf16 subnormal: E clamps at -127
    codes, sc = M.quantize(x, "fp8")
    assert list(sc[0]) == [0, 0] and not codes[0].any()
    assert sc[1, 0] == 0 and sc[1, 1] == 127 + 119
    # 2^-133 / 2^-127 = 2^-6, E4M3's smallest normal (0x08): still exact
    assert codes[1, 0] == 0x08
    dq = M.dequantize(codes, sc, "fp8")
    assert dq[1, 0] == 2.0 ** -133 and dq[1, 32] == 2.0 ** 127 * 1.5


def _rne_fraction(q, grid):
    """Nearest grid point to the exact rational q, ties to the even index, saturating."""
    g = [Fraction(v) for v in grid]
    if q >= g[-1]:
        return len(g) - 1
    best = min(range(len(g)), key=lambda i: (abs(g[i] - q), i % 2))
    return best


@pytest.mark.parametrize("fmt", ["fp8", "fp4"])
def test_element_rounding_brute_force(fmt):
    rng = np.random.default_rng(11)
    x = (rng.standard_t(3, size=(6, 64)) * np.exp2(rng.integers(-8, 8, size=(6, 1))))
    x = x.astype(np.float32).astype(np.float64)
    codes, sc = M.quantize(x, fmt)
    grid = F.E4M3_GRID if fmt == "fp8" else F.E2M1_MAG
    dq = M.dequantize(codes, sc, fmt)
    for r, c in itertools.product(range(6), range(64)):
        blk = x[r, (c // 32) * 32:(c // 32 + 1) * 32]
        amax = Fraction(float(np.abs(blk).max()))
        e = amax.numerator.bit_length() - amax.denominator.bit_length()
        if Fraction(2) ** e > amax:
            e -= 1                                      # floor(log2 amax), exact
        e -= M.EMAX[fmt]
        assert sc[r, c // 32] == e + 127
        q = abs(Fraction(float(x[r, c]))) / Fraction(2) ** e
        idx = _rne_fraction(q, grid)
        assert abs(dq[r, c]) == float(Fraction(grid[idx]) * Fraction(2) ** e)
        assert np.signbit(dq[r, c]) == np.signbit(x[r, c]) or dq[r, c] == 0


def test_fp8_relative_error_bound():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((64, 256)).astype(np.float32).astype(np.float64)
    codes, sc = M.quantize(x, "fp8")
    dq = M.dequantize(codes, sc, "fp8")
    scale = np.repeat(np.exp2(sc.astype(np.float64) - 127), 32, axis=1)
    q = np.abs(x) / scale                              # the element before rounding
    sat = q > 448.0                                    # max|x| / 2^E can reach 512
    normal = (q >= 2.0 ** -6) & ~sat                   # E4M3's normal range
    assert sat.any() and np.all(np.abs(dq) == np.where(sat, 448.0 * scale, np.abs(dq)))
    assert np.all(np.abs(dq - x)[normal] <= 2.0 ** -4 * np.abs(x)[normal])   # half an ulp
    sub = ~normal & ~sat
    assert np.all(np.abs(dq - x)[sub] <= 2.0 ** -10 * scale[sub])


def test_grouped_gemm_exact_small():
    rng = np.random.default_rng(13)
    for fmt in ("fp8", "fp4"):
        a = rng.standard_normal((5, 64))
        w = rng.standard_normal((2, 3, 64))
        aq = M.quantize(a, fmt)
        wq = [M.quantize(w[e], fmt) for e in range(2)]
        wc = (np.stack([q[0] for q in wq]), np.stack([q[1] for q in wq]))
        off = np.array([0, 2, 5])
        rt = np.array([4, 0, 1, 3, 2])
        y, bound = M.grouped_gemm(aq, wc, off, rt, fmt)
        ad = M.dequantize(*aq, fmt)
        for p in range(5):
            e = 0 if p < 2 else 1
            wd = M.dequantize(wc[0][e], wc[1][e], fmt)
            for n in range(3):
                exact = sum(Fraction(float(ad[rt[p], k])) * Fraction(float(wd[n, k]))
                            for k in range(64))
                assert abs(Fraction(float(y[p, n])) - exact) <= Fraction(2) ** -40 * (
                    Fraction(float(bound[p, n])) + 1)


# ---- RAC on the MX FP4 mode (section 3.3 with the MX FP4 quantizer) -------

def _mx_rac_input(seed, rows=96, kdim=256):
    rng = np.random.default_rng(seed)
    x = rng.standard_t(3, size=(rows, kdim))
    x[:, 5] *= 20.0                                   # outlier channels
    x[:, (77 % kdim)] *= 12.0
    return x.astype(np.float32).astype(np.float64)   # fp32 inputs: exact residuals


def test_mx_rac_never_increases_error():
    """|x - X~| <= |x - DQ(Q(x))| element by element (0 is on the element
    grid, so re-quantizing the residual never moves it further from 0), with
    equality off S and a strict drop somewhere on S."""
    x = _mx_rac_input(1)
    out = M.rac_quantize(x, 64, "fp4")
    dq = M.dequantize(out["codes"], out["scales"], "fp4")
    xt = M.compensated(out, "fp4")
    before, after = np.abs(x - dq), np.abs(x - xt)
    assert np.all(after <= before)
    off = np.setdiff1d(np.arange(x.shape[1]), out["sel"])
    assert np.array_equal(after[:, off], before[:, off])
    assert (after[:, out["sel"]] < before[:, out["sel"]]).any()
    # the residual is x - DQ(Q(x)) itself, and S holds the k largest column sums of r^2
    assert np.array_equal(out["r"].astype(np.float64), x - dq)
    s = (out["r"].astype(np.float64) ** 2).sum(axis=0)
    assert s[out["sel"]].min() >= np.delete(s, out["sel"]).max()


def test_mx_rac_closed_form_block():
    """A hand-built case: each 32-block holds one 6.0 and 0.25 elsewhere.  The
    shared exponent is 0 (6 = 1.5 * 2^2), 0.25 lies midway between the codes 0
    and 0.5 and rounds to the even code 0, so r = 0.25 there; the gathered
    residual blocks are all 0.25 (exponent -4, code 4), exact.  So X~ = x on
    the selected channels, and the scores pick the 0.25 channels of the
    lowest indices (ties)."""
    x = np.full((4, 64), 0.25)
    x[:, 0] = 6.0
    x[:, 32] = -6.0
    out = M.rac_quantize(x, 32, "fp4")
    assert np.all(out["scales"] == 127)
    dq = M.dequantize(out["codes"], out["scales"], "fp4")
    assert np.all(dq[:, [0, 32]] == x[:, [0, 32]]) and np.all(np.delete(dq, [0, 32], axis=1) == 0)
    assert np.array_equal(out["sel"], np.r_[1:32, 33])            # 1..31, then 33
    assert np.all(out["r_scales"] == 127 - 4)
    xt = M.compensated(out, "fp4")
    assert np.array_equal(xt[:, out["sel"]], x[:, out["sel"]])


def test_mx_rac_gemm_exact_small():
    """The compensated GEMM as an exact rational sum on a tiny grouped case,
    against the compensated activations contracted by hand."""
    rng = np.random.default_rng(21)
    a = _mx_rac_input(3, rows=5, kdim=64)
    out = M.rac_quantize(a, 32, "fp4")
    w = rng.standard_normal((2, 3, 64))
    wq = [M.quantize(w[e], "fp4") for e in range(2)]
    wc = (np.stack([q[0] for q in wq]), np.stack([q[1] for q in wq]))
    off = np.array([0, 2, 5])
    rt = np.array([4, 0, 1, 3, 2])
    y, bound = M.grouped_gemm_rac((out["codes"], out["scales"]),
                                  (out["r_codes"], out["r_scales"]), out["sel"], wc, off, rt,
                                  "fp4")
    xt = M.compensated(out, "fp4")
    ad = M.dequantize(out["codes"], out["scales"], "fp4")
    rd = M.dequantize(out["r_codes"], out["r_scales"], "fp4")
    for p in range(5):
        e = 0 if p < 2 else 1
        wd = M.dequantize(wc[0][e], wc[1][e], "fp4")
        for n in range(3):
            exact = sum(Fraction(float(xt[rt[p], j])) * Fraction(float(wd[n, j]))
                        for j in range(64))
            assert abs(Fraction(float(y[p, n])) - exact) <= Fraction(2) ** -40 * (
                Fraction(float(bound[p, n])) + 1)
            b = sum(abs(Fraction(float(ad[rt[p], j])) * Fraction(float(wd[n, j])))
                    for j in range(64)) + sum(
                abs(Fraction(float(rd[rt[p], i])) * Fraction(float(wd[n, out["sel"][i]])))
                for i in range(32))
            assert abs(Fraction(float(bound[p, n])) - b) <= Fraction(2) ** -40 * (b + 1)
