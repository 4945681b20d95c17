"""GPU parity of the MX block-scaled comparator (quads_mx_quantize,
quads_moe_mx_gemm) against oracle/mx.py: codes and scale bytes bit-exact,
GEMM outputs within K * 2^-24 * sum|a*w| for FP4 (fp32 accumulation of K
exact products in any order) and 2^-12 * sum|a*w| for FP8 (the hardware's
fp8 dot products are less precise than fp32),
for FP8 E4M3 and FP4 E2M1, dense and grouped (ragged experts, row_token),
fp32 / bf16 / SwiGLU outputs."""

import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from oracle import moe as OM
from oracle import mx as M

pytestmark = pytest.mark.gpu
FMTS = [("fp8", 0), ("fp4", 4)]


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


def _special_rows(k):
    """bf16 rows with the edge cases: zero blocks, ties, saturation, subnormals,
    negative zeros, the largest bf16."""
    rows = []
    z = np.zeros(k, np.float32)
    rows.append(z.copy())                                         # all-zero blocks
    r = z.copy(); r[0] = 500.0; r[1] = 1.0625; r[2] = 1.1875; r[3] = -465.0; r[4] = -0.0
    rows.append(r)                                                # fp8 ties / saturation
    r = z.copy(); r[32] = 7.0; r[33] = 5.0; r[34] = 2.5; r[35] = 0.25; r[36] = -0.75
    rows.append(r)                                                # fp4 ties / saturation
    r = z.copy(); r[64 % k] = 2.0 ** -133; r[(64 % k) + 1] = -(2.0 ** -130)
    rows.append(r)                                                # bf16 subnormals
    r = z.copy(); r[0] = 3.3895313892515355e38; r[1] = -1.0; r[2] = 1e-30
    rows.append(r)                                                # largest bf16
    r = np.full(k, -0.0, np.float32); r[5] = -3.0
    rows.append(r)                                                # signed zeros
    return synth.f32_to_bf16_bits(np.stack(rows))


@pytest.mark.parametrize("name,fmt", FMTS)
@pytest.mark.parametrize("m,k", [(37, 64), (256, 512), (5, 4096)])
def test_mx_quantize_bit_exact(Q, name, fmt, m, k):
    rng = np.random.default_rng(100 + m + k)
    x = rng.standard_t(3, size=(m, k)) * np.exp2(rng.integers(-20, 20, size=(m, 1)))
    bits = np.concatenate([synth.f32_to_bf16_bits(x.astype(np.float32)), _special_rows(k)])
    codes, scales = Q.quads_mx_quantize(_t(bits), fmt)
    torch.cuda.synchronize()
    ec, es = M.quantize(F.bf16_to_f64(bits), name)
    assert np.array_equal(scales.cpu().numpy(), es)
    assert np.array_equal(codes.cpu().numpy(), ec)


def _weights(rng, e, n, k, name):
    w = synth.weights(rng, e, n, k)
    q = [M.quantize(F.bf16_to_f64(w[i]), name) for i in range(e)]
    return w, (np.stack([c for c, _ in q]), np.stack([s for _, s in q]))


def _check(got, exp, bound, kdim, name, bf16=False):
    # FP4: fp32 accumulation of kdim exact products in any order, |err| <= kdim u
    # sum|a w| (u = 2^-24; measured: exact).  FP8: the block-scaled MFMA's fp8
    # dot products carry less than fp32 precision (measured up to about 740 u
    # sum|a w| at K = 256); the bound is 2^-12 sum|a w|.
    rel = kdim * 2.0 ** -24 if name == "fp4" else 2.0 ** -12
    lim = rel * bound + (np.abs(exp) * 2.0 ** -8 if bf16 else 0)
    bad = np.abs(got - exp) > lim
    assert not bad.any(), (np.argwhere(bad)[:5], got[bad][:5], exp[bad][:5])


@pytest.mark.parametrize("name,fmt", FMTS)
@pytest.mark.parametrize("m,k,n", [(300, 256, 320), (64, 1024, 256), (513, 384, 96)])
def test_mx_gemm_dense(Q, name, fmt, m, k, n):
    rng = np.random.default_rng(m * 7 + k + n)
    xb = synth.f32_to_bf16_bits(rng.standard_t(4, size=(m, k)).astype(np.float32))
    w, wq = _weights(rng, 1, n, k, name)
    ac, asc = Q.quads_mx_quantize(_t(xb), fmt)
    out = Q.quads_moe_mx_gemm((ac, asc), (_t(wq[0]), _t(wq[1])), n, fmt=fmt)
    torch.cuda.synchronize()
    aq = M.quantize(F.bf16_to_f64(xb), name)
    exp, bound = M.grouped_gemm(aq, wq, np.array([0, m]), None, name)
    _check(out.cpu().numpy(), exp, bound, k, name)


@pytest.mark.parametrize("name,fmt", FMTS)
def test_mx_gemm_grouped(Q, name, fmt):
    rng = np.random.default_rng(5)
    t, e, topk, k, n = 200, 6, 2, 256, 192
    xb = synth.f32_to_bf16_bits(rng.standard_normal((t, k)).astype(np.float32))
    ids = np.stack([rng.choice(e, size=topk, replace=False) for _ in range(t)]).astype(np.int32)
    ids[ids == 3] = 2                       # expert 3 gets no rows
    ids[:, 1] = np.where(ids[:, 0] == ids[:, 1], (ids[:, 0] + 1) % e, ids[:, 1])
    ids[ids == 3] = 4
    off, rt, _ = OM.pack_routes(ids, e)
    w, wq = _weights(rng, e, n, k, name)
    ac, asc = Q.quads_mx_quantize(_t(xb), fmt)
    wt = (_t(wq[0]), _t(wq[1]))
    aq = M.quantize(F.bf16_to_f64(xb), name)
    exp, bound = M.grouped_gemm(aq, wq, off, rt, name)
    y = Q.quads_moe_mx_gemm((ac, asc), wt, n, rows=int(off[-1]), offsets=_t(off),
                            row_token=_t(rt), fmt=fmt)
    yb = Q.quads_moe_mx_gemm((ac, asc), wt, n, rows=int(off[-1]), offsets=_t(off),
                             row_token=_t(rt), fmt=fmt, out_dtype=Q.OUT_BF16)
    h = Q.quads_moe_mx_gemm((ac, asc), wt, n, rows=int(off[-1]), offsets=_t(off),
                            row_token=_t(rt), fmt=fmt, epilogue=Q.EPI_SWIGLU,
                            out_dtype=Q.OUT_BF16)
    torch.cuda.synchronize()
    _check(y.cpu().numpy(), exp, bound, k, name)
    _check(F.bf16_to_f64(yb.cpu().numpy().view(np.uint16)), exp, bound, k, name, bf16=True)
    # SwiGLU of the GPU's own fp32 outputs, one bf16 ulp
    ref = F.bf16_to_f64(OM.swiglu(y.cpu().numpy().astype(np.float64)))
    got = F.bf16_to_f64(h.cpu().numpy().view(np.uint16))
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126))) - 7)
    assert np.all(np.abs(got - ref) <= ulp * 1.0001)


# ---- RAC on the MX FP4 mode ------------------------------------------------

@pytest.mark.parametrize("m,kd,k", [(64, 256, 32), (300, 512, 128), (37, 64, 64),
                                    (4096, 2048, 64), (3000, 768, 64)])
def test_mx_rac_quantize_bit_exact(Q, m, kd, k):
    """Codes, scales, scores, S and the second pass bit-exact against the
    oracle (outlier channels, ragged row counts, k = K, the edge rows)."""
    rng = np.random.default_rng(m + kd + k)
    x = rng.standard_t(3, size=(m, kd))
    x[:, rng.choice(kd, max(1, kd // 64), replace=False)] *= 20.0
    bits = np.concatenate([synth.f32_to_bf16_bits(x.astype(np.float32)), _special_rows(kd)])
    print(f"mx rac m={bits.shape[0]} K={kd} k={k}", flush=True)
    g = Q.quads_mx_rac_quantize(_t(bits), k, want_score=True)
    torch.cuda.synchronize()
    e = M.rac_quantize(F.bf16_to_f64(bits), k, "fp4")
    assert np.array_equal(g["scales"].cpu().numpy(), e["scales"])
    assert np.array_equal(g["codes"].cpu().numpy(), e["codes"])
    gs = g["score"].cpu().numpy()
    assert np.array_equal(gs.view(np.uint64), e["score"].view(np.uint64))
    assert np.array_equal(g["sel"].cpu().numpy(), e["sel"])
    assert np.array_equal(g["r_scales"].cpu().numpy(), e["r_scales"])
    assert np.array_equal(g["r_codes"].cpu().numpy(), e["r_codes"])


def _mx_rac_operands(Q, bits, k):
    g = Q.quads_mx_rac_quantize(_t(bits), k)
    torch.cuda.synchronize()
    e = M.rac_quantize(F.bf16_to_f64(bits), k, "fp4")
    assert np.array_equal(g["sel"].cpu().numpy(), e["sel"])
    return g, e


@pytest.mark.parametrize("m,kd,n,k", [(300, 512, 256, 128), (64, 1024, 96, 64),
                                      (129, 256, 320, 256)])
def test_mx_rac_gemm_dense(Q, m, kd, n, k):
    rng = np.random.default_rng(7 * m + kd + n + k)
    x = rng.standard_t(4, size=(m, kd))
    x[:, :: max(1, kd // 7)] *= 16.0
    bits = synth.f32_to_bf16_bits(x.astype(np.float32))
    w, wq = _weights(rng, 1, n, kd, "fp4")
    g, e = _mx_rac_operands(Q, bits, k)
    y = Q.quads_moe_mx_rac_gemm((g["codes"], g["scales"]), (g["r_codes"], g["r_scales"]), g["sel"],
                                (_t(wq[0]), _t(wq[1])), n)
    torch.cuda.synchronize()
    exp, bound = M.grouped_gemm_rac((e["codes"], e["scales"]), (e["r_codes"], e["r_scales"]),
                                    e["sel"], wq, np.array([0, m]), None, "fp4")
    _check(y.cpu().numpy(), exp, bound, kd + k, "fp4")
    # and the compensation changes the result (it is not silently skipped)
    y0, _ = M.grouped_gemm((e["codes"], e["scales"]), wq, np.array([0, m]), None, "fp4")
    assert np.abs(exp - y0).max() > 0


def test_mx_rac_gemm_grouped_swiglu(Q):
    rng = np.random.default_rng(17)
    t, e_, topk, kd, n, k = 300, 6, 2, 512, 192, 64
    x = rng.standard_normal((t, kd))
    x[:, 3] *= 20.0
    bits = synth.f32_to_bf16_bits(x.astype(np.float32))
    ids = np.stack([rng.choice(e_, size=topk, replace=False) for _ in range(t)]).astype(np.int32)
    ids[ids == 3] = 2                           # expert 3 gets no rows
    ids[:, 1] = np.where(ids[:, 0] == ids[:, 1], (ids[:, 0] + 1) % e_, ids[:, 1])
    ids[ids == 3] = 4
    off, rt, _ = OM.pack_routes(ids, e_)
    w, wq = _weights(rng, e_, n, kd, "fp4")
    g, e = _mx_rac_operands(Q, bits, k)
    wt = (_t(wq[0]), _t(wq[1]))
    a, r = (g["codes"], g["scales"]), (g["r_codes"], g["r_scales"])
    y = Q.quads_moe_mx_rac_gemm(a, r, g["sel"], wt, n, rows=int(off[-1]), offsets=_t(off),
                                row_token=_t(rt))
    h = Q.quads_moe_mx_rac_gemm(a, r, g["sel"], wt, n, rows=int(off[-1]), offsets=_t(off),
                                row_token=_t(rt), epilogue=Q.EPI_SWIGLU, out_dtype=Q.OUT_BF16)
    torch.cuda.synchronize()
    exp, bound = M.grouped_gemm_rac((e["codes"], e["scales"]), (e["r_codes"], e["r_scales"]),
                                    e["sel"], wq, off, rt, "fp4")
    _check(y.cpu().numpy(), exp, bound, kd + k, "fp4")
    ref = F.bf16_to_f64(OM.swiglu(y.cpu().numpy().astype(np.float64)))
    got = F.bf16_to_f64(h.cpu().numpy().view(np.uint16))
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126))) - 7)
    assert np.all(np.abs(got - ref) <= ulp * 1.0001)
