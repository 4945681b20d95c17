"""MoE expert path: packing, grouped W4A4 GEMM with compensation, SwiGLU,
combine -- TEST INFRASTRUCTURE ONLY (see oracle/__init__).

What is computed:
  * The layer product Y = W X of QUADS (arXiv 2607.15810) section 3.1,
    Eq. (6), with both operands NVFP4-quantized (W4A4) and the activation
    replaced by the compensated X~ of section 3.3, Eq. (21).  For a packed
    row p routed to expert e and output feature n:

      Y[p, n] = s_tA s_tW[e] sum_{j<K} a[row(p), j] w_e[n, j]
              + s_tR s_tW[e] sum_{i<k} r[row(p), i] w_e[n, S_i]

    where a = v * s_b (exact) for the activation, w likewise for the weight
    and r likewise for the second-pass residual.  The oracle forms the exact
    dequantized matrices and multiplies them in fp64 (one matmul per expert).
  * The pages name MoE layers and the fused gate/up ("W13") projection but
    give no routing or layer shapes.  Readings: a stable counting sort of
    (token, slot) pairs by expert id gives the packed row order (experts
    ascending, then flattened token*top_k + slot ascending); the gate is the
    first N/2 output features of W13 and the up projection the second N/2;
    h = bf16_RNE(silu(g) * u); the combine is the routing-weighted sum of a
    token's expert outputs in slot order.
"""

import numpy as np

from .formats import f64_to_bf16_rne
from .nvfp4 import dequantize_unscaled


def pack_routes(topk_ids, num_experts):
    """Stable counting sort of (token, slot) pairs by expert.

    Returns offsets int32 [E+1], row_token int32 [rows] (token of each packed
    row) and pos int32 [T*top_k] (packed row of each (token, slot)).
    """
    ids = np.asarray(topk_ids, dtype=np.int64)
    t, topk = ids.shape
    flat = ids.reshape(-1)
    if np.any((flat < 0) | (flat >= num_experts)):
        raise ValueError("expert id out of range")
    order = np.argsort(flat, kind="stable")
    counts = np.bincount(flat, minlength=num_experts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    row_token = (order // topk).astype(np.int32)
    pos = np.empty(t * topk, dtype=np.int32)
    pos[order] = np.arange(t * topk, dtype=np.int32)
    return offsets, row_token, pos


def grouped_gemm(a, r, sel, w, offsets, row_token=None, want_bound=True):
    """Grouped W4A4 GEMM with the residual compensation term, in fp64.

    a   = (packed [Ta, K/2], scales [Ta, K/16], s_tA)   activation NVFP4; s_tA
          is a scalar, or an array [Ta] of per-row (per-token) scales, in
          which case packed row p takes s_tA[row(p)] (compensation: k = 0)
    r   = (packed [Ta, k/2], scales [Ta, k/16], s_tR) or None   second pass
    sel = int array [k] of selected channels (ascending), shared by every
          expert; or [E, k] with s_tR an array [E]: one selection and one
          residual tensor scale per expert (rac_quantize_experts; the rows
          are then the packed rows, row_token None)
    w   = (packed [E, N, K/2], scales [E, N, K/16], s_tW [E])   weights
    offsets [E+1]: packed rows of expert e are offsets[e] .. offsets[e+1]-1
    row_token [rows] or None: activation row feeding each packed row

    Returns Y (fp64 [rows, N]) and, if asked, the bound sum |a_i w_i| per
    element (fp64 [rows, N]) over both terms, scales included.
    """
    a_nib, a_sc, a_ts = a
    w_nib, w_sc, w_ts = w
    offsets = np.asarray(offsets, dtype=np.int64)
    e_count = len(offsets) - 1
    rows = int(offsets[-1])
    n = w_nib.shape[1]
    sel_arr = None if r is None else np.asarray(sel, dtype=np.int64)
    per_expert = sel_arr is not None and sel_arr.ndim == 2
    if per_expert and row_token is not None:
        raise ValueError("per-expert selection needs activations in packed order")
    if row_token is None:
        row_token = np.arange(rows)
    row_token = np.asarray(row_token, dtype=np.int64)
    k = 0 if r is None else sel_arr.shape[-1]
    y = np.zeros((rows, n), dtype=np.float64)
    bound = np.zeros((rows, n), dtype=np.float64) if want_bound else None
    sa_arr = np.asarray(a_ts, dtype=np.float32).astype(np.float64)
    per_row = sa_arr.ndim > 0
    if per_row and k:
        raise ValueError("per-row activation scales take no compensation term")
    sr_arr = np.asarray(r[2], dtype=np.float32).astype(np.float64) if k else None
    for e in range(e_count):
        p0, p1 = int(offsets[e]), int(offsets[e + 1])
        if p1 == p0:
            continue
        src = row_token[p0:p1]
        ah = dequantize_unscaled(a_nib[src], a_sc[src])               # [m, K] exact
        wh = dequantize_unscaled(w_nib[e], w_sc[e])                   # [N, K] exact
        sw = np.float64(np.float32(w_ts[e]))
        sa = sa_arr[src][:, None] if per_row else sa_arr
        y[p0:p1] = (sa * sw) * (ah @ wh.T)
        if want_bound:
            bound[p0:p1] = (sa * sw) * (np.abs(ah) @ np.abs(wh).T)
        if k:
            rh = dequantize_unscaled(r[0][src], r[1][src])            # [m, k]
            ws = wh[:, sel_arr[e] if per_expert else sel_arr]         # [N, k]
            sr = sr_arr[e] if per_expert else sr_arr
            y[p0:p1] += (sr * sw) * (rh @ ws.T)
            if want_bound:
                bound[p0:p1] += (sr * sw) * (np.abs(rh) @ np.abs(ws).T)
    return y, bound


def swiglu(y1):
    """h = bf16_RNE(silu(g) * u), g = first half of the columns, u = second half."""
    y1 = np.asarray(y1, dtype=np.float64)
    half = y1.shape[1] // 2
    g, u = y1[:, :half], y1[:, half:]
    with np.errstate(over="ignore"):
        h = g / (1.0 + np.exp(-g)) * u
    return f64_to_bf16_rne(h)


def combine(y2, pos, topk_w, num_tokens, topk):
    """out[t] = sum over slots (in order) of w[t, slot] * y2[pos[t, slot]] (fp64)."""
    y2 = np.asarray(y2, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.int64).reshape(num_tokens, topk)
    w = np.asarray(topk_w, dtype=np.float32).astype(np.float64).reshape(num_tokens, topk)
    out = np.zeros((num_tokens, y2.shape[1]), dtype=np.float64)
    for s in range(topk):
        out += w[:, s:s + 1] * y2[pos[:, s]]
    return out
