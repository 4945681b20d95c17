"""NVFP4 quantize / dequantize -- TEST INFRASTRUCTURE ONLY (see oracle/__init__).

What is computed (QUADS, arXiv 2607.15810, section 2.2 "FP4" paragraph, and
the QDQ operators Q_A of Eq. (9) and Q_W of Eq. (7) in section 3.1):

  x is a tensor of rows (tokens, or weight output features) by K channels,
  K a multiple of 16.  Every row is cut into 16-element blocks along K.

  1. tensor scale   A = max |x| over the tensor;  s_t = RN32(A / 2688).
  2. block scale    s_b = min(448, RNE_E4M3(amax_b / (6 * s_t)))  (s_t > 0),
                    s_b = 0 when s_t = 0.
  3. element code   mag = RNE_E2M1(|x| / (s_b * s_t)), saturating at 6;
                    mag = 0 when s_b * s_t = 0.  The nibble is
                    (signbit(x) << 3) | mag.
  4. dequant        v(mag) * s_b * s_t with the nibble's sign (exact).

Readings taken where the pages leave the step open:
  * The pages only say an optional per-tensor FP32 scale exists.  Reading:
    s_t = RN32(A / (6 * 448)), so the block holding the tensor maximum gets
    the largest E4M3 scale and its largest element the largest E2M1 code.
    A caller may instead pass a fixed tensor scale.
  * Block and element rounding: round-to-nearest, ties to the even code, on
    the exact real quotient; block scales saturate at 448, codes at 6.
  * The sign bit is the sign bit of x, also for codes whose magnitude is 0,
    so that quantizing -x gives exactly the sign-flipped nibbles.
  * Packing: two codes per byte, the even channel in the low nibble.  Scale
    bytes are row-major [rows, K/16].

Why fp64 division gives the exact rounding decisions: a quotient p/d here has
p with at most 24 significant bits (bf16 or fp32 input) and d = 6*s_t or
s_b*s_t with at most 28 significant bits, both exact in fp64.  Every rounding
boundary m (an E4M3 or E2M1 midpoint) has at most 5 significant bits, so m*d
is exact with at most 33 bits.  If p != m*d the two differ by at least one
unit in the 31st-33rd bit of m*d, a relative gap near 2^-33 or more, far
above the 2^-53 error of a correctly rounded fp64 division; if p == m*d the
quotient is exactly m.  Hence RN64(p/d) lies on the same side of every
boundary as p/d, and equals a boundary only when p/d does.
"""

from fractions import Fraction

import numpy as np

from .formats import (E2M1_MAG, E4M3_GRID, bf16_to_f64, e2m1_decode,
                      f64_to_bf16_rne, rn32_rational, rne_to_grid)

BLOCK = 16
TENSOR_DIVISOR = 6 * 448     # E2M1 maximum times E4M3 maximum


def tensor_scale(amax) -> np.float32:
    """s_t = RN32(A / 2688) for the tensor maximum A (>= 0); 0 when A = 0."""
    return rn32_rational(Fraction(float(amax)) / TENSOR_DIVISOR)


def block_scale_codes(amax_b, s_t):
    """E4M3 scale byte of each block from its maximum |x| (fp64 array)."""
    amax_b = np.asarray(amax_b, dtype=np.float64)
    s_t = np.float64(np.float32(s_t))
    if s_t == 0.0:
        return np.zeros(amax_b.shape, dtype=np.uint8)
    q = amax_b / (6.0 * s_t)           # 6*s_t is exact in fp64
    return rne_to_grid(q, E4M3_GRID).astype(np.uint8)


def element_codes(x, scale_codes, s_t):
    """E2M1 nibbles (sign | magnitude code) of x [..., K] given block scales."""
    x = np.asarray(x, dtype=np.float64)
    s_b = E4M3_GRID[np.asarray(scale_codes, dtype=np.int64)]
    d = np.repeat(s_b * np.float64(np.float32(s_t)), BLOCK, axis=-1)   # exact
    a = np.abs(x)
    live = d > 0
    with np.errstate(divide="ignore", invalid="ignore"):
        y = np.where(live, a / np.where(live, d, 1.0), 0.0)
    mag = np.where(live, rne_to_grid(y, E2M1_MAG), 0)
    sign = np.signbit(x).astype(np.int64)
    return (mag | (sign << 3)).astype(np.uint8)


def pack_nibbles(nib):
    nib = np.asarray(nib, dtype=np.uint8)
    return (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed):
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


def quantize(x, ts=None):
    """NVFP4-quantize exact values x [rows, K] (fp64 holding bf16/fp32 values).

    Returns (packed nibbles uint8 [rows, K/2], scale bytes uint8 [rows, K/16],
    tensor scale np.float32).  ``ts`` overrides the dynamic tensor scale.
    """
    x = np.asarray(x, dtype=np.float64)
    rows, k = x.shape
    if k % BLOCK:
        raise ValueError("K must be a multiple of 16")
    amax = float(np.max(np.abs(x))) if x.size else 0.0
    s_t = tensor_scale(amax) if ts is None else np.float32(ts)
    amax_b = np.max(np.abs(x.reshape(rows, k // BLOCK, BLOCK)), axis=-1) if x.size \
        else np.zeros((rows, k // BLOCK))
    sb = block_scale_codes(amax_b, s_t)
    nib = element_codes(x, sb, s_t)
    return pack_nibbles(nib), sb, s_t


def quantize_rows(x):
    """NVFP4 with one FP32 scale per row (per token) instead of per tensor:
    steps 1-3 above with A taken over each row alone, i.e. quantize() applied
    to every row as a tensor of its own.

    Reading (a variant, not the pages' default): the pages' tensor scale is
    one number per tensor; the per-token form trades one FP32 value per row
    for rows whose magnitudes differ widely.  Returns (packed [rows, K/2],
    scale bytes [rows, K/16], s_t float32 [rows]).
    """
    x = np.asarray(x, dtype=np.float64)
    rows, k = x.shape
    if k % BLOCK:
        raise ValueError("K must be a multiple of 16")
    packed = np.empty((rows, k // 2), np.uint8)
    scales = np.empty((rows, k // BLOCK), np.uint8)
    ts = np.empty(rows, np.float32)
    for i in range(rows):
        packed[i], scales[i], ts[i] = quantize(x[i:i + 1])
    return packed, scales, ts


def quantize_bf16(bits, ts=None):
    """quantize() of bf16 bit patterns."""
    return quantize(bf16_to_f64(bits), ts)


def dequantize(packed, scale_codes, s_t):
    """Exact values v * s_b * s_t (fp64) of an NVFP4 tensor; signs kept (-0.0)."""
    v = e2m1_decode(unpack_nibbles(packed))
    s_b = np.repeat(E4M3_GRID[np.asarray(scale_codes, dtype=np.int64)], BLOCK, axis=-1)
    return v * s_b * np.float64(np.float32(s_t))       # <= 30 significant bits: exact


def dequantize_unscaled(packed, scale_codes):
    """v * s_b (exact), the per-block-scaled values before the tensor scale."""
    v = e2m1_decode(unpack_nibbles(packed))
    s_b = np.repeat(E4M3_GRID[np.asarray(scale_codes, dtype=np.int64)], BLOCK, axis=-1)
    return v * s_b


def weight_qdq(w_bits):
    """Shared NVFP4 weight QDQ (Eq. (7), (12)): every expert matrix W_e [N, K]
    gets its own dynamic tensor scale; rows are output features, blocks run
    along K.  Returns (packed [E,N,K/2], scales [E,N,K/16], s_t float32 [E],
    dequantized bf16 bits [E,N,K] = RNE_bf16 of the exact value v*s_b*s_t).
    """
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    e, n, k = w_bits.shape
    packed = np.empty((e, n, k // 2), np.uint8)
    scales = np.empty((e, n, k // BLOCK), np.uint8)
    ts = np.empty(e, np.float32)
    dq = np.empty((e, n, k), np.uint16)
    for i in range(e):
        packed[i], scales[i], ts[i] = quantize_bf16(w_bits[i])
        dq[i] = f64_to_bf16_rne(dequantize(packed[i], scales[i], ts[i]))
    return packed, scales, ts, dq
