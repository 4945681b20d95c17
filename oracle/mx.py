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
"""

import numpy as np

from . import formats as F

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
