"""GPU parity of the per-expert channel selection: the RAC call against the
oracle's per-expert RAC (main NVFP4, per-expert scores bitwise, selections,
second-pass nibbles, scale bytes and residual scales, all bit-exact), and the
grouped GEMM with per-expert compensation against the oracle's GEMM
(|y_gpu - y_oracle| <= 1e-5 * sum_i |a_i w_i| per element) on the decode
kernel, both tilings and both compensation orders of the 256 x 256 kernel
(captured columns at k = 64, gathered columns first at k = 128)."""

import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from oracle import moe as OM
from oracle import nvfp4 as ON
from oracle import rac as OR

pytestmark = pytest.mark.gpu
TOL = 1e-5


@pytest.fixture(scope="module")
def Q():
    import nvfp4_w4a4_quantized_act_amd as lib
    lib.lib()
    return lib


def _t(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda:0")


def _x(seed, rows, kd, outliers=8):
    rng = np.random.default_rng(seed)
    x = rng.standard_t(3.0, (rows, kd)).astype(np.float32)
    if outliers:
        x[:, rng.choice(kd, outliers, replace=False)] *= 20
    return synth.f32_to_bf16_bits(x)


def _routed_offsets(seed, t, e, topk, zipf=None):
    rng = np.random.default_rng(seed)
    if zipf:
        p = 1.0 / np.arange(1, e + 1) ** zipf
        ids = np.stack([rng.choice(e, topk, replace=False, p=p / p.sum()) for _ in range(t)])
    else:
        ids = np.stack([rng.choice(e, topk, replace=False) for _ in range(t)])
    return OM.pack_routes(ids.astype(np.int32), e)[0]


def _check_rac(Q, bits, k, off):
    print(f"rac experts shape={bits.shape} k={k} E={len(off) - 1}", flush=True)
    g = Q.quads_rac_quantize_experts(_t(bits), k, _t(np.asarray(off, np.int32)),
                                     want_score=True)
    torch.cuda.synchronize()
    e = OR.rac_quantize_experts(F.bf16_to_f64(bits), k, off)
    assert g["ts"].item() == e["ts"]
    assert np.array_equal(g["scale"].cpu().numpy(), e["scale"])
    assert np.array_equal(g["nib"].cpu().numpy(), e["nib"])
    gs = g["score"].cpu().numpy()
    bad = np.argwhere(gs.view(np.uint64) != e["score"].view(np.uint64))
    assert len(bad) == 0, bad[:5]
    assert np.array_equal(g["sel"].cpu().numpy(), e["sel"])
    assert np.array_equal(g["r_ts"].cpu().numpy().view(np.uint32), e["r_ts"].view(np.uint32))
    if k:
        assert np.array_equal(g["r_scale"].cpu().numpy(), e["r_scale"])
        assert np.array_equal(g["r_nib"].cpu().numpy(), e["r_nib"])
    return e


def test_rac_experts_decode_step_shape(Q):
    """512 packed rows over 128 experts with Zipf(1.2) routing: most experts
    have 0-4 rows, a few dozens; K = 768 (the down projection's input)."""
    off = _routed_offsets(1, 64, 128, 8, zipf=1.2)
    assert (np.diff(off) == 0).any()
    _check_rac(Q, _x(2, int(off[-1]), 768), 64, off)


def test_rac_experts_tree_levels(Q):
    """Experts of 0, 1, 63, 64, 65, 4096 and 4161 rows: one group, exactly
    one full group, one level of groups, exactly 64 groups, and the second
    level."""
    sizes = [0, 1, 63, 64, 65, 4096, 4161, 0]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    _check_rac(Q, _x(3, int(off[-1]), 64, outliers=2), 16, off)


@pytest.mark.parametrize("kd,k", [(2048, 64), (256, 0), (80, 80)])
def test_rac_experts_shapes(Q, kd, k):
    off = _routed_offsets(4 + kd, 200, 16, 4)
    _check_rac(Q, _x(5, int(off[-1]), kd), k, off)


def test_rac_experts_ties_and_empty(Q):
    rng = np.random.default_rng(6)
    base = rng.standard_normal((60, 16)).astype(np.float32)
    x = synth.f32_to_bf16_bits(np.tile(base, (1, 6)))          # identical channel groups
    _check_rac(Q, x, 32, [0, 0, 25, 60, 60])
    g = Q.quads_rac_quantize_experts(torch.zeros((0, 64), dtype=torch.int16, device="cuda:0"), 16,
                                     _t(np.zeros(4, np.int32)), want_score=True)
    torch.cuda.synchronize()
    assert g["sel"].cpu().tolist() == [list(range(16))] * 3
    assert g["r_ts"].cpu().tolist() == [0.0] * 3


@pytest.mark.parametrize("t,e,topk,kd,n,k,path", [
    (64, 32, 4, 256, 192, 64, "decode"),               # <= 32 rows per expert, K % 128 == 0
    (300, 8, 2, 512, 256, 64, "tiled 256x256, captured columns"),
    (300, 8, 2, 512, 320, 128, "tiled 256x256, gathered columns first"),
    (200, 6, 2, 208, 96, 48, "tiled 128x128"),
])
def test_gemm_sel_experts(Q, t, e, topk, kd, n, k, path):
    off = _routed_offsets(7 + t, t, e, topk)
    rows = int(off[-1])
    x = _x(8 + kd, rows, kd)
    out = OR.rac_quantize_experts(F.bf16_to_f64(x), k, off)
    rng = np.random.default_rng(9)
    wq = ON.weight_qdq(synth.weights(rng, e, n, kd))[:3]
    exp, bound = OM.grouped_gemm((out["nib"], out["scale"], out["ts"]),
                                 (out["r_nib"], out["r_scale"], out["r_ts"]), out["sel"], wq, off)
    a = (_t(out["nib"]), _t(out["scale"]), _t(np.array([out["ts"]], np.float32)))
    r = (_t(out["r_nib"]), _t(out["r_scale"]), _t(out["r_ts"]))
    args = dict(r=r, sel=_t(out["sel"]), offsets=_t(off))
    y = Q.quads_moe_w4a4_gemm_sel_experts(a, tuple(_t(v) for v in wq), n, **args)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    bad = np.abs(y - exp) > TOL * bound
    assert not bad.any(), (np.argwhere(bad)[:5], y[bad][:5], exp[bad][:5])
    hb = Q.quads_moe_w4a4_gemm_sel_experts(a, tuple(_t(v) for v in wq), n, epilogue=Q.EPI_SWIGLU,
                                           out_dtype=Q.OUT_BF16, **args)
    torch.cuda.synchronize()
    ref = F.bf16_to_f64(OM.swiglu(y.astype(np.float64)))
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126))) - 7)
    assert np.all(np.abs(F.bf16_to_f64(hb.cpu().numpy().view(np.uint16)) - ref) <= ulp * 1.0001)
