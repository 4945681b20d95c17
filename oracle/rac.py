"""Residual Activation Compensation (RAC) -- TEST INFRASTRUCTURE ONLY.

What is computed (QUADS, arXiv 2607.15810, section 3.3):
  * Eq. (20): the activation quantization error, dX = Q_A(X) - X.  This
    build stores its negation r = x - DQ(Q(x)), rounded once to fp32.
  * Eq. (23): a score per channel j, the L2 norm of the error column over
    the current token batch.  Ranking by the sum of squares gives the same
    order as ranking by the norm, and avoids square-root ties.
  * Eq. (24): S = the k channels with the largest score.
  * Eq. (21): X~ = Q_A(X) - M_S (.) Q_A(dX): the selected channels get a
    second NVFP4 term.  Since NVFP4 quantization is odd-symmetric bit for bit
    (scales ignore signs, rounding is symmetric, sign bits are copied),
    Q(-r) = -Q(r), so X~ = DQ(Q(x)) + scatter_S(DQ(Q(r_S))).

Readings taken where the pages leave the step open:
  * Score arithmetic: r^2 is exact in fp64 (r is fp32).  The sum over tokens
    is fp64 in a fixed order -- a 64-ary tree of sequential sums: tokens in
    groups of 64 are added in order starting from +0.0, then the group sums
    in groups of 64 the same way, and so on until one value is left.  A fixed
    order makes the selected set a function of the input alone.
  * k is an absolute channel count (a multiple of 16, 0 <= k <= K); the
    pages' k% is 100*k/K.  Ties in the score go to the lower channel index;
    S is stored in ascending channel order.  One S per call, shared by every
    row of the tensor.
  * Second pass ("extract, then re-quantize", section 4.4.1): the residual
    columns r[:, S] are gathered into a [rows, k] tensor and NVFP4-quantized
    on their own, with 16-element blocks along the compacted index and their
    own dynamic tensor scale.
"""

import numpy as np

from .nvfp4 import dequantize, quantize

SCORE_FANIN = 64


def residual(x, packed, scales, s_t):
    """r = RN32(x - DQ(Q(x))) as float32 [rows, K].

    The fp64 difference is exact whenever the tensor scale is the dynamic one
    (|x| and |dq| are then within a small factor of each other or dq = 0);
    that is asserted, so the single fp32 rounding is the only rounding.
    """
    x = np.asarray(x, dtype=np.float64)
    dq = dequantize(packed, scales, s_t)
    diff = x - dq
    # TwoSum error term: zero iff the fp64 subtraction was exact
    bb = diff - x
    err = (x - (diff - bb)) + (-dq - bb)
    if np.any(err != 0):
        raise AssertionError("x - dq is not exact in fp64")
    return diff.astype(np.float32)


def tree_sum_rows(v, fanin=SCORE_FANIN):
    """Fixed-order sum over axis 0 of v [n, K]: the 64-ary tree of sequential sums."""
    v = np.asarray(v, dtype=np.float64)
    if v.shape[0] == 0:
        return np.zeros(v.shape[1:], dtype=np.float64)
    while True:
        n = v.shape[0]
        groups = -(-n // fanin)
        acc = np.zeros((groups,) + v.shape[1:], dtype=np.float64)     # +0.0
        for i in range(fanin):
            rows = np.arange(groups) * fanin + i
            ok = rows < n
            acc[ok] = acc[ok] + v[rows[ok]]
        v = acc
        if groups == 1:
            return v[0]


def channel_scores(r):
    """Sum over tokens of r^2 per channel (fp64, fixed order) -- Eq. (23) squared."""
    r64 = np.asarray(r, dtype=np.float32).astype(np.float64)
    return tree_sum_rows(r64 * r64)          # fp32 squares are exact in fp64


def select_channels(score, k):
    """Eq. (24): the k largest scores, ties to the lower index, ascending int32."""
    score = np.asarray(score, dtype=np.float64)
    order = np.lexsort((np.arange(score.shape[0]), -score))
    return np.sort(order[:k]).astype(np.int32)


def rac_quantize(x, k):
    """Full RAC on exact values x [rows, K]: main NVFP4, scores, S, second pass.

    Returns a dict with nib/scale/ts (main), score, sel, r (fp32 residual),
    r_nib/r_scale/r_ts (second pass, [rows, k] layout).
    """
    x = np.asarray(x, dtype=np.float64)
    rows, kdim = x.shape
    if k % 16 or not 0 <= k <= kdim:
        raise ValueError("k must be a multiple of 16 in [0, K]")
    nib, scale, ts = quantize(x)
    r = residual(x, nib, scale, ts)
    score = channel_scores(r)
    sel = select_channels(score, k)
    rsel = r[:, sel].astype(np.float64)
    r_nib, r_scale, r_ts = quantize(rsel)
    return dict(nib=nib, scale=scale, ts=ts, r=r, score=score, sel=sel,
                r_nib=r_nib, r_scale=r_scale, r_ts=r_ts)


def compensated(out, kdim):
    """X~ of Eq. (21) (fp64): DQ(Q(x)) plus the dequantized second pass on S."""
    xt = dequantize(out["nib"], out["scale"], out["ts"])
    if len(out["sel"]):
        xt[:, out["sel"]] += dequantize(out["r_nib"], out["r_scale"], out["r_ts"])
    return xt


def rac_quantize_experts(x, k, offsets):
    """RAC with one channel selection per expert (a variant; the pages select
    "more adaptive" residual channels as future work): for packed activation
    rows x [rows, K] whose expert e owns rows offsets[e] .. offsets[e+1]-1.

    Reading: the main NVFP4 of the whole tensor and the residual r are those
    of rac_quantize (one tensor scale); then every expert's rows are treated
    as a tensor of their own for Eq. (23)-(24) and the second pass: scores
    by the same fixed-order tree over that expert's rows alone, S_e the k
    best (ties to the lower index), and r[rows_e][:, S_e] quantized with its
    own dynamic tensor scale.  An expert without rows gets scores 0, so
    S_e = 0 .. k-1, and s_tR[e] = 0.

    Returns nib/scale/ts, r, score [E, K], sel [E, k], r_nib [rows, k/2],
    r_scale [rows, k/16] (row p in its expert's S_e order), r_ts [E].
    """
    x = np.asarray(x, dtype=np.float64)
    rows, kdim = x.shape
    offsets = np.asarray(offsets, dtype=np.int64)
    if k % 16 or not 0 <= k <= kdim:
        raise ValueError("k must be a multiple of 16 in [0, K]")
    if offsets[0] != 0 or offsets[-1] != rows or np.any(np.diff(offsets) < 0):
        raise ValueError("offsets must run from 0 to rows, non-decreasing")
    e_count = len(offsets) - 1
    nib, scale, ts = quantize(x)
    r = residual(x, nib, scale, ts)
    score = np.zeros((e_count, kdim))
    sel = np.zeros((e_count, k), dtype=np.int32)
    r_nib = np.zeros((rows, k // 2), dtype=np.uint8)
    r_scale = np.zeros((rows, k // 16), dtype=np.uint8)
    r_ts = np.zeros(e_count, dtype=np.float32)
    for e in range(e_count):
        p0, p1 = int(offsets[e]), int(offsets[e + 1])
        score[e] = channel_scores(r[p0:p1])
        sel[e] = select_channels(score[e], k)
        if p1 > p0 and k:
            r_nib[p0:p1], r_scale[p0:p1], r_ts[e] = quantize(
                r[p0:p1][:, sel[e]].astype(np.float64))
    return dict(nib=nib, scale=scale, ts=ts, r=r, score=score, sel=sel,
                r_nib=r_nib, r_scale=r_scale, r_ts=r_ts)


def compensated_experts(out, offsets):
    """X~ of Eq. (21) per expert (fp64): DQ(Q(x)), plus on each expert's rows
    the dequantized second pass scattered onto its S_e."""
    xt = dequantize(out["nib"], out["scale"], out["ts"])
    offsets = np.asarray(offsets, dtype=np.int64)
    for e in range(len(offsets) - 1):
        p0, p1 = int(offsets[e]), int(offsets[e + 1])
        if p1 > p0 and out["sel"].shape[1]:
            xt[p0:p1][:, out["sel"][e]] += dequantize(out["r_nib"][p0:p1], out["r_scale"][p0:p1],
                                                      out["r_ts"][e])
    return xt

