"""Pins for oracle/rac.py (CPU only): exact residual, the fixed-order score
against exactly rounded sums, top-k by brute force, and the pages' RAC
invariant (compensation never moves X~ further from X, Eq. (22))."""

import itertools
import math
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import formats as F
from oracle import nvfp4 as Q
from oracle import rac as R


def test_residual_is_single_rounding_of_exact_difference():
    d = synth.make(1)
    x = F.bf16_to_f64(d["x"])
    nib, sb, ts = Q.quantize(x)
    r = R.residual(x, nib, sb, ts)
    dq = Q.dequantize(nib, sb, ts)
    idx = np.random.default_rng(0).choice(x.size, 400, replace=False)
    for i in idx:
        exact = Fraction(float(x.flat[i])) - Fraction(float(dq.flat[i]))
        assert F.rn32_rational(exact) == r.flat[i]


def test_tree_sum_order_definition():
    # n = 65: group 0 = rows 0..63 in order, group 1 = row 64; then (0 + g0) + g1
    rng = np.random.default_rng(1)
    v = rng.standard_normal((65, 3)) * np.exp2(rng.integers(-30, 30, (65, 3)))
    g0 = np.zeros(3)
    for i in range(64):
        g0 = g0 + v[i]
    exp = (np.zeros(3) + g0) + v[64]
    assert np.array_equal(R.tree_sum_rows(v), exp)
    # a single row is returned as is; no rows gives zeros
    assert np.array_equal(R.tree_sum_rows(v[:1]), v[0])
    assert np.array_equal(R.tree_sum_rows(np.zeros((0, 3))), np.zeros(3))


@pytest.mark.parametrize("m", [1, 63, 64, 65, 4096 + 17])
def test_scores_close_to_exact_sum(m):
    rng = np.random.default_rng(m)
    r = (rng.standard_normal((m, 5)) * np.exp2(rng.integers(-20, 5, (m, 5)))).astype(np.float32)
    s = R.channel_scores(r)
    for j in range(5):
        col = r[:, j].astype(np.float64) ** 2
        exact = math.fsum(col)                      # correctly rounded sum
        levels = max(1, math.ceil(math.log(max(m, 2), 64)))
        bound = (64 * levels) * 2.0 ** -53 * exact
        assert abs(s[j] - exact) <= bound


def _brute_topk(score, k):
    best = None
    n = len(score)
    for sub in itertools.combinations(range(n), k):
        rest = [j for j in range(n) if j not in sub]
        ok = all((score[a] > score[b]) or (score[a] == score[b] and a < b)
                 for a in sub for b in rest)
        if ok:
            assert best is None
            best = sub
    return list(best)


def test_topk_bruteforce_with_ties():
    rng = np.random.default_rng(2)
    for trial in range(40):
        n = int(rng.integers(1, 10))
        k = int(rng.integers(0, n + 1))
        score = rng.integers(0, 4, n).astype(np.float64)     # many ties
        assert list(R.select_channels(score, k)) == _brute_topk(score, k)


def test_topk_degenerate():
    s = np.zeros(48)
    assert list(R.select_channels(s, 16)) == list(range(16))
    s = np.arange(48.0)
    assert list(R.select_channels(s, 48)) == list(range(48))
    assert len(R.select_channels(s, 0)) == 0


def test_rac_never_increases_error_and_eq22():
    d = synth.make(1)
    x = F.bf16_to_f64(d["x"])
    out = R.rac_quantize(x, 16)
    base = Q.dequantize(out["nib"], out["scale"], out["ts"])
    comp = R.compensated(out, x.shape[1])
    e0 = np.abs(base - x)
    e1 = np.abs(comp - x)
    # per element: |r - dq_R| <= |r| (0 is on the grid, rounding is to the nearest)
    assert np.all(e1 <= e0)
    # per channel L2 non-increase, strict on channels with a nonzero second code
    c0 = np.sqrt((e0 ** 2).sum(0))
    c1 = np.sqrt((e1 ** 2).sum(0))
    assert np.all(c1 <= c0)
    rnz = (Q.unpack_nibbles(out["r_nib"]) & 7).any(axis=0)
    assert rnz.any()
    assert np.all(c1[out["sel"][rnz]] < c0[out["sel"][rnz]])
    # Eq. (22): ||X~ - X|| < ||Q(X) - X||
    assert np.linalg.norm(comp - x) < np.linalg.norm(base - x)
    # Fig. 4(a)'s vertical bands: the blocks holding an outlier channel get a
    # coarse scale, so the residual concentrates in those blocks' channels
    assert set(out["sel"] // 16).issubset(set(d["outlier_cols"] // 16))


def test_rac_on_grid_input_selects_low_indices_and_zero_compensation():
    rng = np.random.default_rng(3)
    sb = rng.integers(0x30, 0x7F, size=(4, 4))
    sb[0, 0] = 0x7E
    mag = rng.integers(0, 8, size=(4, 64))
    mag[:, ::16] = 7
    x = F.E2M1_MAG[mag] * np.repeat(F.E4M3_GRID[sb], 16, -1)
    out = R.rac_quantize(x, 16)
    assert not out["r"].any()
    assert list(out["sel"]) == list(range(16))
    assert out["r_ts"] == 0 and not out["r_scale"].any()
    assert np.array_equal(R.compensated(out, 64), x)


def test_rac_k_equals_K_and_zero():
    d = synth.make(1)
    x = F.bf16_to_f64(d["x"])
    full = R.rac_quantize(x, x.shape[1])
    assert list(full["sel"]) == list(range(x.shape[1]))
    # with every channel selected, R is the whole residual
    assert np.array_equal(Q.quantize(full["r"].astype(np.float64))[0], full["r_nib"])
    none = R.rac_quantize(x, 0)
    assert none["r_nib"].shape == (x.shape[0], 0)


def test_rac_error_falls_with_k():
    """Table 3's trend on a synthetic layer input: more channels, less error."""
    d = synth.make(2, m=256, k_dim=512)
    x = F.bf16_to_f64(d["x"])
    errs = []
    for k in (0, 64, 128, 256, 384, 512):
        errs.append(np.linalg.norm(R.compensated(R.rac_quantize(x, k), 512) - x))
    assert all(a > b for a, b in zip(errs, errs[1:]))
