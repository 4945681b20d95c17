"""GPU parity of the per-row (per-token) tensor-scale variant: the quantizer
that gives every activation row its own FP32 scale, and the grouped W4A4 GEMM
that applies those scales per packed row.

Quantizer: bit-exact codes, block-scale bytes and row scales against the
oracle's per-row NVFP4 (rows of magnitudes spread over 2^-40 .. 2^40, an
all-zero row, K below one wave's width, K with a ragged last wave pass).
GEMM: |y_gpu - y_oracle| <= 1e-5 * sum_i |a_i w_i| per element, on the
256 x 256 tiling (K % 64 == 0, many rows per expert), the 128 x 128 tiling
(K % 64 != 0) and the decode kernel (few rows per expert), with f32, bf16
and SwiGLU outputs."""

import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from oracle import moe as OM
from oracle import nvfp4 as ON

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


def _spread_rows(rng, m, k, span=40, zero_row=True):
    """bf16 rows of standard normals, each scaled by 2^u with u uniform in
    [-span, span], a few outliers, and (optionally) one all-zero row."""
    x = rng.standard_normal((m, k)) * np.exp2(rng.integers(-span, span + 1, (m, 1)))
    x[rng.integers(0, m, 3), rng.integers(0, k, 3)] *= 50.0
    if zero_row and m > 2:
        x[m // 2] = 0.0
    return synth.f32_to_bf16_bits(x.astype(np.float32))


@pytest.mark.parametrize("m,k", [(37, 48), (64, 1024), (9, 7168), (130, 1040), (1, 16)])
def test_quantize_rows_bit_exact(Q, m, k):
    rng = np.random.default_rng(m * 131 + k)
    x = _spread_rows(rng, m, k)
    nib, sc, ts = Q.quads_nvfp4_quantize_rows(_t(x))
    torch.cuda.synchronize()
    enib, esc, ets = ON.quantize_rows(F.bf16_to_f64(x))
    assert np.array_equal(ts.cpu().numpy().view(np.uint32), ets.view(np.uint32))
    assert np.array_equal(sc.cpu().numpy(), esc)
    assert np.array_equal(nib.cpu().numpy(), enib)


def test_quantize_rows_empty(Q):
    nib, sc, ts = Q.quads_nvfp4_quantize_rows(torch.zeros((0, 64), dtype=torch.int16,
                                                          device="cuda:0"))
    torch.cuda.synchronize()
    assert nib.shape == (0, 32) and sc.shape == (0, 4) and ts.shape == (0,)


def _case(seed, t, e, topk, h, n):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.choice(e, topk, replace=False) for _ in range(t)]).astype(np.int32)
    # rows 2^-10 .. 2^10 apart: SwiGLU's product of two outputs stays inside
    # fp32's normal range
    x = _spread_rows(rng, t, h, span=10)
    w = synth.weights(rng, e, n, h)
    a = ON.quantize_rows(F.bf16_to_f64(x))
    wq = ON.weight_qdq(w)[:3]
    off, rt, _pos = OM.pack_routes(ids, e)
    return a, wq, off, rt


def _gpu(Q, a, wq, n, off, rt, **kw):
    y = Q.quads_moe_w4a4_gemm_rowscale(tuple(_t(v) for v in a), tuple(_t(v) for v in wq), n,
                                       offsets=_t(off), row_token=_t(rt), **kw)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _check(got, exp, bound, bf16=False):
    lim = TOL * bound
    if bf16:
        lim = lim + np.abs(exp) * 2.0 ** -8
    bad = np.abs(got - exp) > lim
    assert not bad.any(), (np.argwhere(bad)[:5], got[bad][:5], exp[bad][:5])


@pytest.mark.parametrize("t,e,topk,h,n,path", [
    (300, 4, 2, 512, 320, "tiled 256x256"),      # K % 64 == 0, > 32 rows per expert
    (200, 4, 2, 208, 136, "tiled 128x128"),      # K % 64 != 0
    (40, 16, 4, 384, 200, "decode"),             # <= 32 rows per expert, K % 128 == 0
    (60, 8, 2, 192, 96, "tiled 256x256, K % 128 != 0"),
])
def test_gemm_rowscale(Q, t, e, topk, h, n, path):
    a, wq, off, rt = _case(t + h, t, e, topk, h, n)
    y = _gpu(Q, a, wq, n, off, rt)
    exp, bound = OM.grouped_gemm(a, None, None, wq, off, rt)
    _check(y, exp, bound)
    yb = _gpu(Q, a, wq, n, off, rt, out_dtype=Q.OUT_BF16).view(np.uint16)
    _check(F.bf16_to_f64(yb), exp, bound, bf16=True)
    hb = _gpu(Q, a, wq, n, off, rt, epilogue=Q.EPI_SWIGLU, out_dtype=Q.OUT_BF16).view(np.uint16)
    ref = F.bf16_to_f64(OM.swiglu(y.astype(np.float64)))
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126))) - 7)
    assert np.all(np.abs(F.bf16_to_f64(hb) - ref) <= ulp * 1.0001)


def test_gemm_rowscale_equal_scales_match_tensor_scale(Q):
    """Rows whose scales all equal the tensor scale: the per-row GEMM gives
    the per-tensor GEMM's output exactly (same products, same order)."""
    rng = np.random.default_rng(3)
    t, e, h, n = 96, 4, 256, 128
    ids = np.stack([rng.choice(e, 2, replace=False) for _ in range(t)]).astype(np.int32)
    x = synth.f32_to_bf16_bits(rng.standard_normal((t, h)).astype(np.float32))
    nib, sc, s_t = ON.quantize(F.bf16_to_f64(x))
    wq = ON.weight_qdq(synth.weights(rng, e, n, h))[:3]
    off, rt, _pos = OM.pack_routes(ids, e)
    rows_ts = np.full(t, s_t, np.float32)
    y_rows = _gpu(Q, (nib, sc, rows_ts), wq, n, off, rt)
    y_tensor = Q.quads_moe_w4a4_gemm((_t(nib), _t(sc), _t(np.array([s_t], np.float32))),
                                     tuple(_t(v) for v in wq), n, offsets=_t(off),
                                     row_token=_t(rt))
    torch.cuda.synchronize()
    assert np.array_equal(y_rows, y_tensor.cpu().numpy())
