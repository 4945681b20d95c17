"""GPU parity of the grouped W4A4 GEMM in the few-rows-per-expert regime
(decode): at most 32 packed rows per expert on average, K a multiple of 128
and k <= 64 select the weight-streaming kernel (one work-group of two waves
per expert and 128-row weight slab, K streamed in 128-deep chunks through a
three-deep register ring, the compensation columns taken from the stream)
for every expert with at most 128 rows, the tiled kernel the others; with at
most 512 packed rows in all the decode kernel takes every expert.
Same bar as the tiled kernels: |y_gpu - y_oracle| <= 1e-5 * sum_i |a_i w_i|
per element.

Cases cover experts with no rows, with more than 32 and more than 64 rows
(several passes over the slab), chunk counts that are not a multiple of the
ring depth, feature counts that end inside a slab or are not a multiple of 4
(scalar stores), bf16 and SwiGLU outputs, the dense (E = 1) form, and packed
activations without a row index."""

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


def _case(seed, t, e, topk, h, n, k, heavy=(0, 1)):
    """Routing with a few heavy experts (every token picks `heavy` first when
    it can), some light ones and expert e - 1 empty."""
    rng = np.random.default_rng(seed)
    ids = np.empty((t, topk), np.int32)
    light = np.arange(len(heavy), e - 1)
    for i in range(t):
        pick = [x for x in heavy if rng.random() < 0.9][:topk]
        rest = rng.choice(light, topk - len(pick), replace=False)
        ids[i] = np.concatenate([pick, rest]).astype(np.int32)
    x = synth.f32_to_bf16_bits(rng.standard_normal((t, h)).astype(np.float32))
    x[:, rng.choice(h, 3, replace=False)] = synth.f32_to_bf16_bits(
        (rng.standard_normal((t, 3)) * 20).astype(np.float32))
    w = synth.weights(rng, e, n, h)
    out = OR.rac_quantize(F.bf16_to_f64(x), k)
    wq = ON.weight_qdq(w)[:3]
    off, rt, pos = OM.pack_routes(ids, e)
    assert int(off[-1]) <= 32 * e                    # the decode regime
    return out, wq, off, rt


def _gpu(Q, out, w, n, k, offsets=None, row_token=None, rows=None, **kw):
    a = (_t(out["nib"]), _t(out["scale"]), _t(np.array([out["ts"]], np.float32)))
    r = (_t(out["r_nib"]), _t(out["r_scale"]), _t(np.array([out["r_ts"]], np.float32))) \
        if k else None
    y = Q.quads_moe_w4a4_gemm(a, tuple(_t(v) for v in w), n, rows=rows, r=r,
                              sel=_t(out["sel"]) if k else None,
                              offsets=None if offsets is None else _t(offsets),
                              row_token=None if row_token is None else _t(row_token), **kw)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _oracle(out, w, k, offsets, row_token=None):
    r = (out["r_nib"], out["r_scale"], out["r_ts"]) if k else None
    return OM.grouped_gemm((out["nib"], out["scale"], out["ts"]), r, out["sel"], w, offsets,
                           row_token)


def _assert_close(got, exp, bound, bf16=False):
    err = np.abs(got - exp)
    lim = TOL * bound
    if bf16:
        lim = lim + np.abs(exp) * 2.0 ** -8
    bad = err > lim
    assert not bad.any(), (np.argwhere(bad)[:5], err[bad][:5], lim[bad][:5])


@pytest.mark.parametrize("t,e,h,n,k", [
    (40, 16, 384, 200, 48),      # 3 chunks (one ring turn); N ends inside a slab
    (90, 12, 256, 138, 64),      # N % 4 != 0; an expert with > 64 rows (3 passes)
    (48, 32, 512, 64, 0),        # no compensation; half a slab
    (64, 128, 896, 192, 64),     # 128 experts, top-8, most with 0-4 rows; 7 chunks
])
def test_decode_grouped(Q, t, e, h, n, k):
    out, wq, off, rt = _case(100 + t, t, e, 4 if e < 64 else 8, h, n, k)
    cnt = np.diff(off)
    assert cnt.max() > 32 and (cnt == 0).any()
    y = _gpu(Q, out, wq, n, k, offsets=off, row_token=rt)
    exp, bound = _oracle(out, wq, k, off, rt)
    _assert_close(y, exp, bound)


@pytest.mark.parametrize("t,e,topk,k", [(200, 24, 3, 64), (200, 24, 3, 48), (150, 16, 3, 64),
                                         (500, 16, 1, 64)])
def test_decode_with_a_large_expert(Q, t, e, topk, k):
    """Decode regime with one expert above 128 rows.  Above 512 packed rows
    (t = 200, top-3) the tiled kernel takes that expert (k = 48: the 128 x 128
    tiling) and the decode kernel the rest; at 450 and 500 packed rows the
    decode kernel takes it too, split into work-groups of at most 128 rows
    (two, and four with a last one of fewer rows)."""
    out, wq, off, rt = _case(77 + k + t, t, e, topk, 256, 160, k, heavy=(0,))
    cnt = np.diff(off)
    assert cnt.max() > 128 and ((cnt > 0) & (cnt <= 128)).sum() > 8
    assert topk == 3 or cnt.max() > 384
    assert (int(off[-1]) > 512) == (t == 200)
    y = _gpu(Q, out, wq, 160, k, offsets=off, row_token=rt)
    exp, bound = _oracle(out, wq, k, off, rt)
    _assert_close(y, exp, bound)
    h = _gpu(Q, out, wq, 160, k, offsets=off, row_token=rt, epilogue=Q.EPI_SWIGLU,
             out_dtype=Q.OUT_BF16).view(np.uint16)
    ref = F.bf16_to_f64(OM.swiglu(y.astype(np.float64)))
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126))) - 7)
    assert np.all(np.abs(F.bf16_to_f64(h) - ref) <= ulp * 1.0001)


def test_decode_bf16_output(Q):
    out, wq, off, rt = _case(7, 50, 16, 4, 768, 2048 // 8, 64)
    y = _gpu(Q, out, wq, 256, 64, offsets=off, row_token=rt, out_dtype=Q.OUT_BF16)
    exp, bound = _oracle(out, wq, 64, off, rt)
    _assert_close(F.bf16_to_f64(y.view(np.uint16)), exp, bound, bf16=True)


@pytest.mark.parametrize("feat,k", [(80, 32), (42, 0), (768, 64)])
def test_decode_swiglu(Q, feat, k):
    out, wq, off, rt = _case(11 + feat, 48, 16, 4, 256, 2 * feat, k)
    g = _gpu(Q, out, wq, 2 * feat, k, offsets=off, row_token=rt)
    exp, bound = _oracle(out, wq, k, off, rt)
    _assert_close(g, exp, bound)
    hb = _gpu(Q, out, wq, 2 * feat, k, offsets=off, row_token=rt, epilogue=Q.EPI_SWIGLU,
              out_dtype=Q.OUT_BF16).view(np.uint16)
    ref = F.bf16_to_f64(OM.swiglu(g.astype(np.float64)))
    got = F.bf16_to_f64(hb)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126))) - 7)
    assert np.all(np.abs(got - ref) <= ulp * 1.0001)


@pytest.mark.parametrize("m,kd,n,k", [(20, 256, 72, 16), (32, 640, 130, 0), (1, 128, 64, 16)])
def test_decode_dense(Q, m, kd, n, k):
    """One expert, no routing arrays, at most 32 rows."""
    rng = np.random.default_rng(m + kd)
    x = synth.f32_to_bf16_bits(rng.standard_normal((m, kd)).astype(np.float32))
    w = synth.weights(rng, 1, n, kd)
    out = OR.rac_quantize(F.bf16_to_f64(x), k)
    wq = ON.weight_qdq(w)[:3]
    y = _gpu(Q, out, wq, n, k)
    exp, bound = _oracle(out, wq, k, [0, m])
    _assert_close(y, exp, bound)


def test_decode_packed_rows_without_row_token(Q):
    """Activations already in packed order (the down GEMM's input)."""
    out, wq, off, rt = _case(5, 30, 8, 4, 256, 96, 16)
    rows = int(off[-1])
    x = synth.f32_to_bf16_bits(np.random.default_rng(6).standard_normal((rows, 256))
                               .astype(np.float32))
    out = OR.rac_quantize(F.bf16_to_f64(x), 16)
    y = _gpu(Q, out, wq, 96, 16, offsets=off)
    exp, bound = _oracle(out, wq, 16, off)
    _assert_close(y, exp, bound)
