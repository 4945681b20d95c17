"""Pins for oracle/nvfp4.py: closed forms, invariants and Fraction brute force
(CPU only)."""

import itertools
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import formats as F
from oracle import nvfp4 as Q


def _brute_block_code(amax_b: Fraction, s_t: Fraction):
    """E4M3 scale byte by exhaustive nearest-even search over all 127 values."""
    if s_t == 0:
        return 0
    q = amax_b / (6 * s_t)
    best = None
    for code, v in enumerate(F.E4M3_GRID):
        d = abs(q - Fraction(v))
        if best is None or d < best[0] or (d == best[0] and code % 2 == 0):
            best = (d, code)
    return best[1]


def _brute_elem_code(x: Fraction, d: Fraction):
    if d == 0:
        mag = 0
    else:
        y = abs(x) / d
        best = None
        for code, v in enumerate(F.E2M1_MAG):
            dist = abs(y - Fraction(v))
            if best is None or dist < best[0] or (dist == best[0] and code % 2 == 0):
                best = (dist, code)
        mag = best[1]
    return mag


def _bruteforce_quantize(xvals):
    """Whole NVFP4 quantization in exact rational arithmetic, by exhaustive
    nearest-value search (independent of rne_to_grid and fp64 division)."""
    rows, k = len(xvals), len(xvals[0])
    amax = max(abs(Fraction(v)) for row in xvals for v in row)
    s_t = Fraction(float(F.rn32_rational(amax / 2688)))
    nib = np.zeros((rows, k), np.uint8)
    sb = np.zeros((rows, k // 16), np.uint8)
    for r in range(rows):
        for b in range(k // 16):
            blk = [Fraction(v) for v in xvals[r][16 * b:16 * b + 16]]
            code = _brute_block_code(max(abs(v) for v in blk), s_t)
            sb[r, b] = code
            d = Fraction(float(F.E4M3_GRID[code])) * s_t
            for i, v in enumerate(blk):
                mag = _brute_elem_code(v, d)
                neg = np.signbit(float(xvals[r][16 * b + i]))
                nib[r, 16 * b + i] = mag | (8 if neg else 0)
    return Q.pack_nibbles(nib), sb, np.float32(float(s_t))


def test_tensor_scale_all_bf16_against_fp64_route():
    """RN32(A/2688) computed exactly equals fp32(fp64(A)/2688) for every
    positive finite bf16 A -- the double rounding never bites for this
    divisor.  (The GPU computes the latter.)"""
    bits = np.arange(1, 0x7F80, dtype=np.uint16)
    a = F.bf16_to_f64(bits)
    fast = (a / 2688.0).astype(np.float32)
    exact = np.array([Q.tensor_scale(v) for v in a[::7]], dtype=np.float32)
    assert np.array_equal(fast[::7], exact)
    assert Q.tensor_scale(0.0) == 0.0
    assert Q.tensor_scale(2688.0) == 1.0


def test_bruteforce_tiny_blocks_small_alphabet():
    """Every combination of a small alphabet in a 16-wide row, compared against
    exact rational nearest-even search for scales and codes."""
    alphabet = [0.0, -0.0, 0.1, -0.3, 0.75, 1.0, -1.25, 2.5, 3.5, -5.0, 6.0, 7.0]
    rng = np.random.default_rng(5)
    rows = []
    for combo in itertools.product(alphabet[:6], repeat=2):
        row = list(combo) + list(rng.choice(alphabet, 14))
        rows.append(row)
    rows = [[float(np.float32(v)) for v in r] for r in rows]
    x = np.array(rows, dtype=np.float64)
    got = Q.quantize(x)
    exp = _bruteforce_quantize(rows)
    assert np.array_equal(got[0], exp[0])
    assert np.array_equal(got[1], exp[1])
    assert got[2] == exp[2]


def test_bruteforce_random_bf16_blocks():
    rng = np.random.default_rng(6)
    xb = synth.f32_to_bf16_bits(rng.standard_normal((6, 64)).astype(np.float32)
                                * np.float32(3.0))
    xb[2, 5] = 0x8000          # -0.0
    x = F.bf16_to_f64(xb)
    got = Q.quantize(x)
    exp = _bruteforce_quantize(x.tolist())
    for g, e in zip(got, exp):
        assert np.array_equal(np.asarray(g), np.asarray(e))


def test_block_amax_maps_to_six():
    """Whenever the block scale is a normal E4M3 value, the block maximum gets
    the largest magnitude code (mag 7 = 6.0); the tensor-max block gets 448."""
    d = synth.make(2, m=64, k_dim=512)
    x = F.bf16_to_f64(d["x"])
    nib, sb, ts = Q.quantize(x)
    codes = Q.unpack_nibbles(nib).reshape(64, 32, 16) & 7
    blocks = np.abs(x.reshape(64, 32, 16))
    arg = blocks.argmax(axis=-1)
    top = np.take_along_axis(codes, arg[..., None], -1)[..., 0]
    normal = sb >= 0x08
    assert normal.any()
    assert np.all(top[normal] == 7)
    r, b = np.unravel_index(np.argmax(blocks.max(-1)), sb.shape)
    assert sb[r, b] == 0x7E


def test_identity_on_grid():
    """Inputs already on the NVFP4 grid, each block holding a +-6*s_b element and
    the tensor maximum 2688 * 2^p, come back exactly."""
    rng = np.random.default_rng(7)
    for p in (-20, -3, 0, 5):
        sb = rng.integers(0x30, 0x7F, size=(8, 4))
        sb[0, 0] = 0x7E
        mag = rng.integers(0, 8, size=(8, 64))
        mag[:, ::16] = 7                 # each block's maximum is 6 * s_b
        sign = rng.integers(0, 2, size=(8, 64))
        v = F.E2M1_MAG[mag] * np.where(sign, -1, 1) * np.repeat(F.E4M3_GRID[sb], 16, -1)
        x = v * 2.0 ** p
        nib, sbq, ts = Q.quantize(x)
        assert ts == np.float32(2.0 ** p)
        assert np.array_equal(Q.dequantize(nib, sbq, ts), x)


def test_odd_symmetry_and_scale_invariance():
    d = synth.make(1)
    x = F.bf16_to_f64(d["x"])
    n1, s1, t1 = Q.quantize(x)
    n2, s2, t2 = Q.quantize(-x)
    assert np.array_equal(n1 ^ 0x88, n2) and np.array_equal(s1, s2) and t1 == t2
    for p in (-30, 7):
        n3, s3, t3 = Q.quantize(x * 2.0 ** p)
        assert np.array_equal(n1, n3) and np.array_equal(s1, s3)
        assert t3 == np.float32(t1 * 2.0 ** p)


def test_zero_tensor_and_zero_blocks():
    x = np.zeros((3, 32))
    x[1, 3] = -0.0
    nib, sb, ts = Q.quantize(x)
    assert ts == 0 and not sb.any()
    assert Q.unpack_nibbles(nib)[1, 3] == 8 and (Q.unpack_nibbles(nib) & 7).max() == 0
    x = np.zeros((2, 32))
    x[0, 20] = 1.0
    nib, sb, ts = Q.quantize(x)
    assert sb[0, 0] == 0 and sb[1].max() == 0 and sb[0, 1] == 0x7E


def test_static_tensor_scale_saturates():
    x = np.array([[1000.0] + [0.0] * 15])
    nib, sb, ts = Q.quantize(x, ts=np.float32(0.01))
    assert sb[0, 0] == 0x7E and (Q.unpack_nibbles(nib)[0, 0] & 7) == 7


def test_subnormal_scales():
    """A block far below the tensor maximum gets a subnormal or zero E4M3 scale."""
    x = np.zeros((1, 48))
    x[0, 0] = 2688.0                       # s_t = 1
    x[0, 16] = 6 * 2.0 ** -9 * 3           # amax_b/(6 s_t) = 3 * 2^-9: subnormal code 3
    x[0, 32] = 6 * 2.0 ** -11              # 2^-11 < 2^-10: rounds to scale 0
    nib, sb, ts = Q.quantize(x)
    assert list(sb[0]) == [0x7E, 0x03, 0x00]
    assert (Q.unpack_nibbles(nib)[0, 16] & 7) == 7
    assert (Q.unpack_nibbles(nib)[0, 32] & 7) == 0


def test_weight_qdq_batched_equals_per_expert():
    rng = np.random.default_rng(8)
    w = synth.weights(rng, 3, 8, 32)
    p, s, t, dq = Q.weight_qdq(w)
    for e in range(3):
        p1, s1, t1 = Q.quantize_bf16(w[e])
        assert np.array_equal(p[e], p1) and np.array_equal(s[e], s1) and t[e] == t1
    # idempotence on the exact-value path for normal scales
    x = Q.dequantize(p[0], s[0], t[0])
    p2, s2, t2 = Q.quantize(x)
    assert np.array_equal(Q.dequantize(p2, s2, t2), x)
    # bf16 output lies within half a bf16 ulp of the exact value
    exact = Q.dequantize(p[0], s[0], t[0])
    got = F.bf16_to_f64(dq[0])
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(exact), 2.0 ** -126))) - 7)
    assert np.all(np.abs(got - exact) <= ulp / 2)


@pytest.mark.parametrize("cfg", [1])
def test_quantize_error_bound(cfg):
    """|x - dq| <= half the local grid step: at most 1 * s_b * s_t (the 4..6 gap)
    for non-saturated elements."""
    d = synth.make(cfg)
    x = F.bf16_to_f64(d["x"])
    nib, sb, ts = Q.quantize(x)
    dq = Q.dequantize(nib, sb, ts)
    step = np.repeat(F.E4M3_GRID[sb], 16, -1) * np.float64(ts)
    assert np.all(np.abs(x - dq) <= step * 1.0 + 1e-300)


# ---------------------------------------------------------------------------
# per-token (per-row) FP32 scales: a variant where every row is its own tensor

def test_quantize_rows_bruteforce():
    """Each row against the exhaustive rational quantizer run on that row alone."""
    rng = np.random.default_rng(71)
    x = rng.standard_normal((5, 32)) * np.exp2(rng.integers(-6, 7, (5, 1)))
    x = F.bf16_to_f64(F.f64_to_bf16_rne(x))
    packed, scales, ts = Q.quantize_rows(x)
    for i in range(5):
        bp, bs, bt = _bruteforce_quantize([list(map(float, x[i]))])
        assert np.array_equal(packed[i], bp[0]) and np.array_equal(scales[i], bs[0])
        assert ts[i] == bt


def test_quantize_rows_power_of_two_and_independence():
    """Scaling one row by 2^j scales its s_t by 2^j exactly and leaves its codes,
    its block scales and every other row unchanged."""
    rng = np.random.default_rng(72)
    x = F.bf16_to_f64(F.f64_to_bf16_rne(rng.standard_normal((6, 64))))
    p0, s0, t0 = Q.quantize_rows(x)
    for j in (-20, -3, 5, 40):
        y = x.copy()
        y[2] *= 2.0 ** j
        p1, s1, t1 = Q.quantize_rows(y)
        assert np.array_equal(p1, p0) and np.array_equal(s1, s0)
        assert t1[2] == np.float32(t0[2] * 2.0 ** j)
        assert np.array_equal(np.delete(t1, 2), np.delete(t0, 2))


def test_quantize_rows_equal_maxima_match_tensor_scale():
    """When every row has the same max |x|, per-row and per-tensor agree."""
    rng = np.random.default_rng(73)
    x = rng.standard_normal((7, 48))
    x[:, 5] = 3.5
    x = np.clip(x, -3.5, 3.5)
    x = F.bf16_to_f64(F.f64_to_bf16_rne(x))
    pr, sr, tr = Q.quantize_rows(x)
    pt, st, tt = Q.quantize(x)
    assert np.array_equal(pr, pt) and np.array_equal(sr, st) and np.all(tr == tt)


def test_quantize_rows_row_holding_2688():
    """A row whose max is 2688 * 2^j gets s_t = 2^j, scale byte 0x7E (448) and
    code 7 (6) for that element."""
    x = np.zeros((2, 16))
    x[0, 3] = 2688.0 * 2.0 ** -7
    x[1, 9] = -2688.0 * 2.0 ** 4
    packed, scales, ts = Q.quantize_rows(x)
    assert list(ts) == [np.float32(2.0 ** -7), np.float32(2.0 ** 4)]
    assert scales[0, 0] == 0x7E and scales[1, 0] == 0x7E
    nib = Q.unpack_nibbles(packed)
    assert nib[0, 3] == 7 and nib[1, 9] == 0xF
