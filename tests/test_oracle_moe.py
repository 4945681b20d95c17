"""Pins for oracle/moe.py (CPU only): packing against a brute-force bucket
sort, the GEMM against an exact rational triple loop and against the dense
product of the compensated activation (Eq. (6) applied to X~ of Eq. (21)),
SwiGLU against scipy's logistic function, combine against the brute-force
bucket rows (one-hot routing weights) and an exact rational sum."""

from fractions import Fraction

import numpy as np
import pytest
from scipy.special import expit

import synth
from oracle import formats as F
from oracle import moe as M
from oracle import nvfp4 as Q
from oracle import rac as R


def test_pack_bruteforce():
    rng = np.random.default_rng(0)
    for t, e, topk in [(5, 3, 2), (37, 16, 4), (64, 128, 8), (1, 1, 1)]:
        ids = np.stack([rng.choice(e, topk, replace=False) for _ in range(t)]).astype(np.int32)
        off, row_token, pos = M.pack_routes(ids, e)
        buckets = [[] for _ in range(e)]
        for tt in range(t):
            for s in range(topk):
                buckets[ids[tt, s]].append((tt, s))
        flat = [p for b in buckets for p in b]
        assert list(off) == list(np.cumsum([0] + [len(b) for b in buckets]))
        assert list(row_token) == [tt for tt, _ in flat]
        for p, (tt, s) in enumerate(flat):
            assert pos[tt * topk + s] == p
    # empty experts and all-to-one routing
    off, row_token, pos = M.pack_routes(np.zeros((4, 1), np.int32), 3)
    assert list(off) == [0, 4, 4, 4] and list(row_token) == [0, 1, 2, 3]


def _tiny_problem(seed, rows_a, k_dim, n, e, k, routing_rows):
    rng = np.random.default_rng(seed)
    x = synth.f32_to_bf16_bits(rng.standard_normal((rows_a, k_dim)).astype(np.float32))
    out = R.rac_quantize(F.bf16_to_f64(x), k)
    w = synth.weights(rng, e, n, k_dim, std=0.5)
    wp, ws, wt, _ = Q.weight_qdq(w)
    return x, out, (wp, ws, wt)


def test_gemm_dense_exact_rational_triple_loop():
    x, out, w = _tiny_problem(1, 3, 32, 4, 1, 16, None)
    a = (out["nib"], out["scale"], out["ts"])
    r = (out["r_nib"], out["r_scale"], out["r_ts"])
    y, bound = M.grouped_gemm(a, r, out["sel"], w, [0, 3])
    ad = Q.dequantize(*a)
    rd = Q.dequantize(*r)
    wd = Q.dequantize(w[0][0], w[1][0], w[2][0])
    for p in range(3):
        for nn in range(4):
            acc = sum(Fraction(float(ad[p, j])) * Fraction(float(wd[nn, j])) for j in range(32))
            acc += sum(Fraction(float(rd[p, i])) * Fraction(float(wd[nn, out["sel"][i]]))
                       for i in range(16))
            assert abs(Fraction(float(y[p, nn])) - acc) <= abs(acc) * Fraction(1, 2 ** 50)


def test_gemm_equals_product_of_compensated_activation():
    """Eq. (21) then Eq. (6): W X~ computed densely equals the split formula."""
    x, out, w = _tiny_problem(2, 24, 64, 12, 1, 16, None)
    a = (out["nib"], out["scale"], out["ts"])
    r = (out["r_nib"], out["r_scale"], out["r_ts"])
    y, bound = M.grouped_gemm(a, r, out["sel"], w, [0, 24])
    xt = R.compensated(out, 64)
    wd = Q.dequantize(w[0][0], w[1][0], w[2][0])
    ref = xt @ wd.T
    assert np.all(np.abs(y - ref) <= 1e-13 * bound)
    assert np.all(bound >= np.abs(y) * (1 - 1e-12))


def test_grouped_equals_per_expert_dense():
    rng = np.random.default_rng(3)
    t, e, topk, h, n = 40, 5, 2, 32, 8
    ids = np.stack([rng.choice(e, topk, replace=False) for _ in range(t)]).astype(np.int32)
    off, row_token, pos = M.pack_routes(ids, e)
    x = synth.f32_to_bf16_bits(rng.standard_normal((t, h)).astype(np.float32))
    out = R.rac_quantize(F.bf16_to_f64(x), 16)
    wp, ws, wt, _ = Q.weight_qdq(synth.weights(rng, e, n, h, std=0.3))
    a = (out["nib"], out["scale"], out["ts"])
    r = (out["r_nib"], out["r_scale"], out["r_ts"])
    y, bound = M.grouped_gemm(a, r, out["sel"], (wp, ws, wt), off, row_token)
    xt = R.compensated(out, h)
    for p in range(len(row_token)):
        ex = int(np.searchsorted(off, p, side="right") - 1)
        wd = Q.dequantize(wp[ex], ws[ex], wt[ex])
        assert np.all(np.abs(y[p] - wd @ xt[row_token[p]]) <= 1e-13 * bound[p])


def test_swiglu_against_scipy_and_torch_rounding():
    rng = np.random.default_rng(4)
    y1 = rng.standard_normal((7, 16)) * 4
    h = M.swiglu(y1)
    g, u = y1[:, :8], y1[:, 8:]
    ref = g * expit(g) * u
    got = F.bf16_to_f64(h)
    ulp = np.exp2(np.floor(np.log2(np.abs(ref))) - 7)
    assert np.all(np.abs(got - ref) <= ulp / 2 * (1 + 1e-9))


def _bucket_row_of(ids, e):
    """Brute force: the packed row of every (token, slot) pair, filling experts
    in ascending order and, within an expert, pairs in (token, slot) order."""
    t, topk = ids.shape
    row, p = {}, 0
    for ex in range(e):
        for tt in range(t):
            for s in range(topk):
                if ids[tt, s] == ex:
                    row[(tt, s)] = p
                    p += 1
    return row


def test_combine_one_hot_picks_the_bucket_row():
    """With routing weight 1 on one slot and 0 on the others, token t's output
    is exactly the expert output row that the brute-force bucket sort gives
    (t, slot): pins the pos convention (index t * top_k + slot) of combine."""
    rng = np.random.default_rng(15)
    for t, e, topk, n in [(9, 5, 3, 6), (17, 16, 8, 4), (1, 1, 1, 3)]:
        ids = np.stack([rng.choice(e, topk, replace=False) for _ in range(t)]).astype(np.int32)
        bucket = _bucket_row_of(ids, e)
        pos = np.array([bucket[(tt, s)] for tt in range(t) for s in range(topk)], np.int32)
        y2 = rng.standard_normal((t * topk, n))
        for s in range(topk):
            w = np.zeros((t, topk), np.float32)
            w[:, s] = 1.0
            out = M.combine(y2, pos, w, t, topk)
            for tt in range(t):
                assert np.array_equal(out[tt], y2[bucket[(tt, s)]])


def test_combine_exact_rational():
    """Dyadic expert outputs (multiples of 1/8 below 64) and routing weights
    (multiples of 1/16 below 1): every partial sum is exact in fp64, so the
    output equals the exact rational weighted sum over the token's slots."""
    rng = np.random.default_rng(16)
    t, e, topk, n = 7, 6, 4, 5
    ids = np.stack([rng.choice(e, topk, replace=False) for _ in range(t)]).astype(np.int32)
    bucket = _bucket_row_of(ids, e)
    pos = np.array([bucket[(tt, s)] for tt in range(t) for s in range(topk)], np.int32)
    y_int = rng.integers(-511, 512, size=(t * topk, n))
    w_int = rng.integers(0, 16, size=(t, topk))
    out = M.combine(y_int / 8.0, pos, (w_int / 16.0).astype(np.float32), t, topk)
    for tt in range(t):
        for c in range(n):
            ref = sum(Fraction(int(w_int[tt, s]), 16) * Fraction(int(y_int[bucket[(tt, s)], c]), 8)
                      for s in range(topk))
            assert Fraction(float(out[tt, c])) == ref


def test_combine_loop():
    rng = np.random.default_rng(5)
    t, topk, n = 6, 3, 4
    y2 = rng.standard_normal((t * topk, n))
    pos = rng.permutation(t * topk).astype(np.int32)
    w = rng.random((t, topk)).astype(np.float32)
    out = M.combine(y2, pos, w, t, topk)
    for tt in range(t):
        acc = np.zeros(n)
        for s in range(topk):
            acc = acc + np.float64(w[tt, s]) * y2[pos[tt * topk + s]]
        assert np.array_equal(out[tt], acc)


def test_gemm_per_row_scales_exact_rational():
    """Per-row activation scales: y[p, n] = s_t[row(p)] s_tW sum_j a w, against
    a Fraction triple loop; with all scales equal it is the per-tensor GEMM."""
    rng = np.random.default_rng(74)
    x = rng.standard_normal((4, 32)) * np.exp2(rng.integers(-5, 6, (4, 1)))
    x = F.bf16_to_f64(F.f64_to_bf16_rne(x))
    ap, asc, ats = Q.quantize_rows(x)
    w = synth.weights(rng, 1, 3, 32, std=0.5)
    wp, ws, wt, _ = Q.weight_qdq(w)
    row_token = np.array([2, 0, 3, 1, 2])
    y, bound = M.grouped_gemm((ap, asc, ats), None, None, (wp, ws, wt), [0, 5], row_token)
    wd = Q.dequantize(wp[0], ws[0], wt[0])
    for p in range(5):
        t = row_token[p]
        ad = Q.dequantize(ap[t:t + 1], asc[t:t + 1], ats[t])[0]
        for nn in range(3):
            acc = sum(Fraction(float(ad[j])) * Fraction(float(wd[nn, j])) for j in range(32))
            assert abs(Fraction(float(y[p, nn])) - acc) <= abs(acc) * Fraction(1, 2 ** 50)
    same = np.full(4, ats[0], np.float32)
    y1, _ = M.grouped_gemm((ap, asc, same), None, None, (wp, ws, wt), [0, 5], row_token)
    y2, _ = M.grouped_gemm((ap, asc, ats[0]), None, None, (wp, ws, wt), [0, 5], row_token)
    assert np.array_equal(y1, y2)
