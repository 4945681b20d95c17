"""MX block-scaled formats and the MX grouped GEMM -- TEST INFRASTRUCTURE ONLY.

What it is for (QUADS, arXiv 2607.15810, section 2.2 "FP8" paragraph and
section 4.4, Fig. 9(a)): the paper's speed claim is relative to FP8 W8A8
rollout with fine-grained block scaling, where each tile of values carries
its own scale.  On MI355X the block-scaled MFMA takes one power-of-two scale
per 32 consecutive elements of each operand row, so the comparator GEMM uses
that form: the OCP Microscaling (MX) layout.

Definitions (reading: the OCP MX rule with round-to-nearest-even elements):
  * a block is 32 consecutive elements of a row (K % 32 == 0);
  * its shared exponent is E = floor(log2(max|x|)) - emax, with emax = 8
    for FP8 E4M3 (largest 448 = 1.75 * 2^8) and emax = 2 for FP4 E2M1
    (largest 6 = 1.5 * 2^2), clamped to [-127, 127]; an all-zero block gets
    E = -127; the scale byte (E8M0) is E + 127;
  * each element is x / 2^E (exact) rounded to the nearest value of the
    element grid, ties to the even code, saturating at the largest finite
    value; the sign bit is the sign bit of x;
  * decode: v * 2^E.
The GEMM is the plain sum over k of the decoded products, in fp64.

RAC on the MX FP4 mode (section 3.3, Eq. (20)-(24), with the MX FP4 format
the "FP4" paragraph of section 2.2 sets beside NVFP4): the same steps as
oracle/rac.py with the MX quantizer in place of NVFP4 -- the residual
r = RN32(x - DQ(Q(x))), the per-channel scores (Eq. (23) squared, the same
fixed-order sum), S (Eq. (24), ties to the lower index, ascending), and the
second pass: r[:, S] gathered and MX-quantized with 32-element blocks along
the compacted index.  Readings: k is a multiple of 32 (whole MX blocks of
the gathered residual); MX quantization is odd-symmetric (the shared
exponent ignores signs, rounding is symmetric, the sign bit is copied), so
Eq. (21) reads X~ = DQ(Q(x)) + scatter_S(DQ(Q(r_S))) as in oracle/rac.py.
"""

import numpy as np

from . import formats as F
from . import rac as R

MX_BLOCK = 32
EMAX = {"fp8": 8, "fp4": 2}


def _grid(fmt):
    return F.E4M3_GRID if fmt == "fp8" else F.E2M1_MAG


def shared_exponent(amax, fmt):
    """E = floor(log2 amax) - emax, clamped to [-127, 127]; -127 for amax = 0."""
    amax = np.asarray(amax, dtype=np.float64)
    mant, ex = np.frexp(amax)              # amax = mant * 2^ex, mant in [0.5, 1)
    e = ex.astype(np.int64) - 1 - EMAX[fmt]
    e = np.where(amax > 0, e, -127)
    return np.clip(e, -127, 127)


def quantize(x, fmt):
    """MX quantization of exact values x [rows, K] -> (codes, scale bytes [rows, K/32]).

    codes: fp8 -> uint8 [rows, K] E4M3 bytes; fp4 -> uint8 [rows, K/2] with
    the even element in the low nibble.
    """
    x = np.asarray(x, dtype=np.float64)
    rows, k = x.shape
    if k % MX_BLOCK:
        raise ValueError("K must be a multiple of 32")
    blocks = x.reshape(rows, k // MX_BLOCK, MX_BLOCK)
    e = shared_exponent(np.abs(blocks).max(axis=-1), fmt)
    q = np.abs(blocks) / np.exp2(e)[..., None].astype(np.float64)      # exact
    mag = F.rne_to_grid(q, _grid(fmt))
    sign = np.signbit(blocks)
    if fmt == "fp8":
        codes = (mag | np.where(sign, 0x80, 0)).astype(np.uint8).reshape(rows, k)
    else:
        nib = (mag | np.where(sign, 0x8, 0)).astype(np.uint8).reshape(rows, k)
        codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    return codes, (e + 127).astype(np.uint8)


def dequantize(codes, scales, fmt):
    """Exact fp64 values of MX codes."""
    codes = np.asarray(codes, dtype=np.uint8)
    if fmt == "fp8":
        v = F.e4m3_decode(codes)
    else:
        nib = np.empty((codes.shape[0], codes.shape[1] * 2), np.uint8)
        nib[:, 0::2] = codes & 0xF
        nib[:, 1::2] = codes >> 4
        v = F.e2m1_decode(nib)
    s = np.exp2(np.asarray(scales, dtype=np.float64) - 127.0)
    return v * np.repeat(s, MX_BLOCK, axis=-1)


def grouped_gemm(a, w, offsets, row_token=None, fmt="fp8"):
    """Y[p, n] = sum_k dq_a[row(p), k] * dq_w[e(p), n, k] in fp64, and the
    bound sum_k |dq_a * dq_w| per output.

    a = (codes, scales) [rows_a, ...]; w = (codes [E, N, ...], scales [E, N, K/32]);
    offsets [E+1] packed-row ranges; row_token[p] = A row of packed row p
    (identity when None)."""
    a_dq = dequantize(a[0], a[1], fmt)
    offsets = np.asarray(offsets)
    rows = int(offsets[-1])
    rt = np.arange(rows) if row_token is None else np.asarray(row_token)
    n = w[0].shape[1]
    y = np.zeros((rows, n))
    bound = np.zeros((rows, n))
    for e in range(len(offsets) - 1):
        sl = slice(offsets[e], offsets[e + 1])
        if offsets[e] == offsets[e + 1]:
            continue
        wd = dequantize(w[0][e], w[1][e], fmt)
        xa = a_dq[rt[sl]]
        y[sl] = xa @ wd.T
        bound[sl] = np.abs(xa) @ np.abs(wd).T
    return y, bound


def residual(x, codes, scales, fmt="fp4"):
    """r = RN32(x - DQ(Q(x))) [rows, K] float32 for the MX quantization of x.

    The fp64 difference is exact (x and DQ have few significant bits and
    the elements that round to zero return x itself); that is asserted."""
    x = np.asarray(x, dtype=np.float64)
    dq = dequantize(codes, scales, fmt)
    diff = x - dq
    bb = diff - x
    err = (x - (diff - bb)) + (-dq - bb)         # TwoSum error term
    if np.any(err != 0):
        raise AssertionError("x - dq is not exact in fp64")
    return diff.astype(np.float32)


def rac_quantize(x, k, fmt="fp4"):
    """RAC on exact values x [rows, K] with the MX quantizer: main codes and
    scales, the fp32 residual, scores, S and the second pass ([rows, k]
    layout, 32-element blocks along the compacted index)."""
    x = np.asarray(x, dtype=np.float64)
    rows, kdim = x.shape
    if k % MX_BLOCK or not 0 <= k <= kdim:
        raise ValueError("k must be a multiple of 32 in [0, K]")
    codes, scales = quantize(x, fmt)
    r = residual(x, codes, scales, fmt)
    score = R.channel_scores(r)
    sel = R.select_channels(score, k)
    if k:
        r_codes, r_scales = quantize(r[:, sel].astype(np.float64), fmt)
    else:
        r_codes = np.zeros((rows, 0), np.uint8)
        r_scales = np.zeros((rows, 0), np.uint8)
    return dict(codes=codes, scales=scales, r=r, score=score, sel=sel, r_codes=r_codes,
                r_scales=r_scales)


def compensated(out, fmt="fp4"):
    """X~ of Eq. (21) (fp64): the dequantized main codes plus, on S, the
    dequantized second pass."""
    xt = dequantize(out["codes"], out["scales"], fmt)
    if len(out["sel"]):
        xt[:, out["sel"]] += dequantize(out["r_codes"], out["r_scales"], fmt)
    return xt


def grouped_gemm_rac(a, r, sel, w, offsets, row_token=None, fmt="fp4"):
    """Y[p, n] = sum_j dq_a[row(p), j] dq_w[e(p), n, j]
              + sum_i dq_r[row(p), i] dq_w[e(p), n, sel[i]]   (Eq. (21) into Eq. (6)),
    in fp64, with the bound (the same sums of |products|).  r = (codes, scales)
    of the second pass, or None for plain MX W4A4."""
    y, bound = grouped_gemm(a, w, offsets, row_token, fmt)
    if r is None or len(sel) == 0:
        return y, bound
    r_dq = dequantize(r[0], r[1], fmt)
    offsets = np.asarray(offsets)
    rows = int(offsets[-1])
    rt = np.arange(rows) if row_token is None else np.asarray(row_token)
    for e in range(len(offsets) - 1):
        sl = slice(offsets[e], offsets[e + 1])
        if offsets[e] == offsets[e + 1]:
            continue
        ws = dequantize(w[0][e], w[1][e], fmt)[:, sel]
        xr = r_dq[rt[sl]]
        y[sl] += xr @ ws.T
        bound[sl] += np.abs(xr) @ np.abs(ws).T
    return y, bound
