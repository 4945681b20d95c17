"""Pins for the per-expert channel selection of oracle/rac.py and the
per-expert compensation term of oracle/moe.py (CPU only).

Reading pinned: the main NVFP4 and the residual are the whole tensor's; each
expert's rows are a tensor of their own for the scores (Eq. (23)), the
selection (Eq. (24)) and the second pass.  Pins: one expert reduces to the
shared-selection RAC; relabelling the experts permutes every per-expert
output and nothing else; the selection against exact rational scores; the
compensation never moves an element away from x (Eq. (22)) and touches only
the expert's own S_e; the grouped GEMM equals the product with the
explicitly compensated activation, expert by expert."""

from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import formats as F
from oracle import moe as M
from oracle import nvfp4 as Q
from oracle import rac as R


def _x(seed, rows, k_dim, outliers=3):
    rng = np.random.default_rng(seed)
    x = rng.standard_t(3.0, (rows, k_dim)).astype(np.float32)
    x[:, rng.choice(k_dim, outliers, replace=False)] *= 20
    return F.bf16_to_f64(synth.f32_to_bf16_bits(x))


def test_one_expert_is_the_shared_selection():
    x = _x(1, 70, 96)
    a = R.rac_quantize(x, 32)
    b = R.rac_quantize_experts(x, 32, [0, 70])
    for key in ("nib", "scale", "r_nib", "r_scale"):
        assert np.array_equal(a[key], b[key]), key
    assert a["ts"] == b["ts"] and a["r_ts"] == b["r_ts"][0]
    assert np.array_equal(a["sel"], b["sel"][0])
    assert np.array_equal(a["score"].view(np.uint64), b["score"][0].view(np.uint64))


def test_relabelling_experts_permutes_the_outputs():
    """Blocks of rows moved to other experts (same rows, so the same tensor
    scale): every per-expert output moves with its block."""
    x = _x(2, 150, 64)
    cuts = [0, 40, 40, 105, 150]                   # expert 1 empty
    blocks = [x[cuts[e]:cuts[e + 1]] for e in range(4)]
    perm = [2, 0, 3, 1]                            # new expert i holds old block perm[i]
    x2 = np.concatenate([blocks[p] for p in perm])
    off2 = np.concatenate([[0], np.cumsum([len(blocks[p]) for p in perm])])
    a = R.rac_quantize_experts(x, 16, cuts)
    b = R.rac_quantize_experts(x2, 16, off2)
    assert a["ts"] == b["ts"]
    for i, p in enumerate(perm):
        assert np.array_equal(b["sel"][i], a["sel"][p])
        assert b["r_ts"][i] == a["r_ts"][p]
        assert np.array_equal(b["score"][i], a["score"][p])
        s0, s1 = off2[i], off2[i + 1]
        assert np.array_equal(b["r_nib"][s0:s1], a["r_nib"][cuts[p]:cuts[p + 1]])
        assert np.array_equal(b["r_scale"][s0:s1], a["r_scale"][cuts[p]:cuts[p + 1]])
        assert np.array_equal(b["nib"][s0:s1], a["nib"][cuts[p]:cuts[p + 1]])
    assert list(a["sel"][1]) == list(range(16)) and a["r_ts"][1] == 0


@pytest.mark.parametrize("seed", [3, 4, 5])
def test_selection_against_exact_scores(seed):
    """Exact rational sum of the fp32 residual squares per expert; the k best
    by that exact score (ties to the lower index) is S_e whenever the k-th and
    (k+1)-th exact scores differ by more than the fp64 tree's error."""
    x = _x(seed, 90, 48, outliers=2)
    off = [0, 30, 31, 90]
    out = R.rac_quantize_experts(x, 16, off)
    for e in range(3):
        rows = out["r"][off[e]:off[e + 1]]
        exact = [sum((Fraction(float(v)) ** 2 for v in rows[:, j]), Fraction(0))
                 for j in range(48)]
        order = sorted(range(48), key=lambda j: (-exact[j], j))
        kth, nxt = exact[order[15]], exact[order[16]]
        if kth - nxt <= kth * Fraction(1, 10 ** 12):
            continue                                # too close to call: skip
        assert list(out["sel"][e]) == sorted(order[:16])


def test_compensation_per_expert_never_moves_away():
    x = _x(6, 120, 80)
    off = [0, 10, 64, 64, 120]
    out = R.rac_quantize_experts(x, 32, off)
    base = Q.dequantize(out["nib"], out["scale"], out["ts"])
    xt = R.compensated_experts(out, off)
    assert np.all(np.abs(x - xt) <= np.abs(x - base))            # Eq. (22) per element
    for e in range(4):
        p0, p1 = off[e], off[e + 1]
        mask = np.ones(80, bool)
        mask[out["sel"][e]] = False
        assert np.array_equal(xt[p0:p1][:, mask], base[p0:p1][:, mask])   # only S_e moves


def test_grouped_gemm_with_per_expert_selection():
    """Y equals, per expert, X~ (per-expert compensation) times the
    dequantized weights, in fp64, within rounding of the fp64 sums."""
    rng = np.random.default_rng(7)
    e_count, n, k_dim = 5, 24, 96
    off = np.array([0, 12, 12, 40, 41, 70])
    x = _x(8, 70, k_dim)
    out = R.rac_quantize_experts(x, 32, off)
    w = Q.weight_qdq(synth.weights(rng, e_count, n, k_dim))
    wq = w[:3]
    y, bound = M.grouped_gemm((out["nib"], out["scale"], out["ts"]),
                              (out["r_nib"], out["r_scale"], out["r_ts"]), out["sel"], wq, off)
    xt = R.compensated_experts(out, off)
    for e in range(e_count):
        p0, p1 = off[e], off[e + 1]
        wd = Q.dequantize(wq[0][e], wq[1][e], wq[2][e])
        ref = xt[p0:p1] @ wd.T
        assert np.all(np.abs(y[p0:p1] - ref) <= 1e-12 * bound[p0:p1] + 1e-300)
    with pytest.raises(ValueError):
        M.grouped_gemm((out["nib"], out["scale"], out["ts"]),
                       (out["r_nib"], out["r_scale"], out["r_ts"]), out["sel"], wq, off,
                       row_token=np.arange(70))


def test_k_zero_and_bad_offsets():
    x = _x(9, 20, 32)
    out = R.rac_quantize_experts(x, 0, [0, 5, 20])
    assert out["sel"].shape == (2, 0) and np.all(out["r_ts"] == 0)
    with pytest.raises(ValueError):
        R.rac_quantize_experts(x, 16, [0, 5, 19])
