"""GPU parity: grouped W4A4 GEMM with the RAC compensation term against the
oracle.  Tolerance |y_gpu - y_oracle| <= 1e-5 * sum_i |a_i w_i| per element
(bf16 outputs add half a bf16 ulp of the oracle value); SwiGLU within one bf16
ulp of the oracle's SwiGLU of the GPU's own fp32 gate and up values."""

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


def _operands(x_bits, w_bits, k):
    """Oracle-side quantization of the GEMM inputs (independent of the GPU)."""
    out = OR.rac_quantize(F.bf16_to_f64(x_bits), k)
    wp, ws, wt, _ = ON.weight_qdq(w_bits)
    return out, (wp, ws, wt)


def _gpu_gemm(Q, out, w, n, k, offsets=None, row_token=None, rows=None, **kw):
    a = (_t(out["nib"]), _t(out["scale"]), _t(np.array([out["ts"]], np.float32)))
    r = (_t(out["r_nib"]), _t(out["r_scale"]), _t(np.array([out["r_ts"]], np.float32))) \
        if k else None
    sel = _t(out["sel"]) if k else None
    wt = (_t(w[0]), _t(w[1]), _t(w[2]))
    y = Q.quads_moe_w4a4_gemm(a, wt, n, rows=rows, r=r, sel=sel,
                              offsets=None if offsets is None else _t(offsets),
                              row_token=None if row_token is None else _t(row_token), **kw)
    torch.cuda.synchronize()
    return y


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
    return float((err / np.maximum(bound, 1e-300)).max())


@pytest.mark.parametrize("m,kd,n,k", [(32, 256, 128, 16), (200, 272, 136, 32), (64, 512, 256, 0),
                                      (1, 16, 1, 16), (129, 1024, 130, 64),
                                      # k > 256 at a long contraction: the tiled kernel
                                      # with W[:, S] gathered into the workspace
                                      (300, 1024, 256, 512), (64, 2048, 130, 1024),
                                      (256, 4096, 128, 2048)])
def test_dense(Q, m, kd, n, k):
    print(f"dense gemm m={m} K={kd} N={n} k={k}", flush=True)
    rng = np.random.default_rng(m * 7 + kd + n + k)
    x = synth.f32_to_bf16_bits(rng.standard_normal((m, kd)).astype(np.float32))
    x[:, :: max(1, kd // 5)] = synth.f32_to_bf16_bits(
        rng.standard_normal((m, len(range(0, kd, max(1, kd // 5))))).astype(np.float32) * 16)
    w = synth.weights(rng, 1, n, kd)
    out, wq = _operands(x, w, k)
    y = _gpu_gemm(Q, out, wq, n, k).cpu().numpy()
    exp, bound = _oracle(out, wq, k, [0, m])
    _assert_close(y, exp, bound)


def test_config1(Q):
    d = synth.make(1)
    out, wq = _operands(d["x"], d["w"], d["rac_k"])
    y = _gpu_gemm(Q, out, wq, 128, d["rac_k"]).cpu().numpy()
    exp, bound = _oracle(out, wq, d["rac_k"], [0, 32])
    _assert_close(y, exp, bound)


def test_all_positive_operands(Q):
    """sum |a w| = |sum a w|: the tolerance is exercised at its edge (K = 4096)."""
    rng = np.random.default_rng(5)
    x = synth.f32_to_bf16_bits(np.abs(rng.standard_normal((96, 4096))).astype(np.float32))
    w = np.abs(synth.weights(rng, 1, 64, 4096).view(np.int16)).view(np.uint16)
    out, wq = _operands(x, w, 128)
    y = _gpu_gemm(Q, out, wq, 64, 128).cpu().numpy()
    exp, bound = _oracle(out, wq, 128, [0, 96])
    rel = _assert_close(y, exp, bound)
    print("max relative error", rel)


def _adversarial_chain(m, kd, n, k):
    """NVFP4 operands (codes built directly, tensor scales 1) whose products in
    every output are one large product 4*256 x 4*256 = 2^20 in channel 0 and,
    in every 8-channel group from channel 16 on, one small product
    1.5*0.3125 x 1*0.125 = 0.0586, just under half an fp32 ulp of 2^20.  The
    MFMA rounds once per group of 8 products, so an accumulator chain that
    rounds each such addition back to 2^20 loses them all: for K = 2048 that is
    254 * 0.0586 = 14.9, or 1.4e-5 * sum|a w| -- over the 1e-5 bar -- while
    restarting the chain every 1024 channels (then adding the chain sums) keeps
    the loss to one chain's 126 terms.  Returns (oracle-layout operands)."""
    nb = kd // 16
    a_nib = np.zeros((m, kd // 2), np.uint8)
    a_sc = np.zeros((m, nb), np.uint8)
    a_nib[:, 0] = 6                       # 4.0
    a_sc[:, 0] = 0x78                     # 256
    a_nib[:, 8::4] = 3                    # 1.5 at channels 16, 24, ... (low nibble of byte c / 2)
    a_sc[:, 1:] = 0x2A                    # 0.3125
    w_nib = np.zeros((1, n, kd // 2), np.uint8)
    w_sc = np.zeros((1, n, nb), np.uint8)
    w_nib[:, :, 0] = 6
    w_sc[:, :, 0] = 0x78
    w_nib[:, :, 8::4] = 2                 # 1.0
    w_sc[:, :, 1:] = 0x20                 # 0.125
    out = {"nib": a_nib, "scale": a_sc, "ts": np.float32(1.0), "sel": np.zeros(0, np.int32)}
    if k:
        out.update(r_nib=np.zeros((m, k // 2), np.uint8), r_scale=np.zeros((m, k // 16), np.uint8),
                   r_ts=np.float32(0.0), sel=np.arange(k, dtype=np.int32))
    return out, (w_nib, w_sc, np.ones(1, np.float32))


@pytest.mark.parametrize("m,kd,k", [(256, 4096, 0), (256, 4096, 256), (32, 4096, 0),
                                    (256, 4032, 0), (96, 2048, 64), (32, 2048, 64)])
def test_accumulation_bound_adversarial(Q, m, kd, k):
    """The 1e-5 sum|a w| bar holds by construction against the worst case of
    gfx950's per-8-product rounding (the tiled kernel at 256 rows, the few-rows
    kernel at 32, the fallback kernel for K % 128 != 0, each at K >= 2048)."""
    print(f"adversarial chain m={m} K={kd} k={k}", flush=True)
    out, wq = _adversarial_chain(m, kd, 128, k)
    y = _gpu_gemm(Q, out, wq, 128, k).cpu().numpy()
    exp, bound = _oracle(out, wq, k, [0, m])
    # the case is meaningful: losing every small term would break the bar
    lost = exp[:, 0] - 2.0 ** 20
    assert np.all(lost > TOL * bound[:, 0])
    rel = _assert_close(y, exp, bound)
    print("max relative error", rel)


def test_exact_power_of_two_scales(Q):
    """On-grid inputs with power-of-two tensor scales and few terms: every
    partial sum is exact in fp32, so the GPU must equal the oracle exactly."""
    rng = np.random.default_rng(6)
    m, kd, n = 64, 64, 64
    sb = np.full((m, kd // 16), 0x38)                 # s_b = 1
    mag = rng.integers(0, 8, (m, kd))
    mag[:, ::16] = 7
    sb[0, 0] = 0x7E
    x = F.E2M1_MAG[mag] * np.where(rng.random((m, kd)) < .5, -1, 1) * \
        np.repeat(F.E4M3_GRID[sb], 16, -1)
    wm = rng.integers(0, 8, (n, kd))
    wm[:, ::16] = 7
    wv = F.E2M1_MAG[wm] * np.where(rng.random((n, kd)) < .5, -1, 1)
    wv[0, 16] = 6 * 448        # the two tensor maxima never meet in one product
    out, wq = _operands(F.f64_to_bf16_rne(x), F.f64_to_bf16_rne(wv)[None], 0)
    y = _gpu_gemm(Q, out, wq, n, 0).cpu().numpy()
    exp, _ = _oracle(out, wq, 0, [0, m])
    assert np.array_equal(y.astype(np.float64), exp)


@pytest.mark.parametrize("kd", [320, 256])
def test_extreme_dynamic_range(Q, kd):
    """Blocks far below the tensor maximum get subnormal or zero E4M3 scales;
    one row is all zero."""
    rng = np.random.default_rng(kd)
    x = rng.standard_normal((90, kd)).astype(np.float32)
    x *= np.exp2(rng.integers(-14, 1, (90, kd // 16))).repeat(16, axis=1).astype(np.float32)
    x[3] = 0
    x[0, 0] = 64.0
    w = synth.weights(rng, 1, 72, kd)
    w[0, :, 16:32] = synth.f32_to_bf16_bits(
        rng.standard_normal((72, 16)).astype(np.float32) * np.float32(1e-7))
    out, wq = _operands(synth.f32_to_bf16_bits(x), w, 64)
    assert (out["scale"] < 8).any() and (wq[1] < 8).any()        # subnormal scales present
    y = _gpu_gemm(Q, out, wq, 72, 64).cpu().numpy()
    exp, bound = _oracle(out, wq, 64, [0, 90])
    _assert_close(y, exp, bound)


def test_bf16_output(Q):
    rng = np.random.default_rng(7)
    x = synth.f32_to_bf16_bits(rng.standard_normal((70, 320)).astype(np.float32))
    w = synth.weights(rng, 1, 96, 320)
    out, wq = _operands(x, w, 32)
    y = _gpu_gemm(Q, out, wq, 96, 32, out_dtype=Q.OUT_BF16).cpu().numpy().view(np.uint16)
    exp, bound = _oracle(out, wq, 32, [0, 70])
    _assert_close(F.bf16_to_f64(y), exp, bound, bf16=True)


def _moe_case(seed, t, e, topk, h, n, k):
    rng = np.random.default_rng(seed)
    choices = [j for j in range(e) if j != 3]          # expert 3 gets no rows
    ids = np.stack([rng.choice(choices, topk, replace=False) for _ in range(t)]).astype(np.int32)
    x = synth.f32_to_bf16_bits(rng.standard_normal((t, h)).astype(np.float32))
    w = synth.weights(rng, e, n, h)
    return ids, x, w


@pytest.mark.parametrize("t,h,n,k", [(150, 256, 192, 32), (400, 256, 320, 64), (700, 512, 96, 128)])
def test_grouped_gather_rows(Q, t, h, n, k):
    """Packed rows gathered through row_token, uneven experts (several 256-row
    tiles and ragged tails), an empty expert; both tilings (k % 64 != 0 and
    == 0)."""
    ids, x, w = _moe_case(8 + t, t, 8, 3, h, n, k)
    off, rt, pos = OM.pack_routes(ids, 8)
    out, wq = _operands(x, w, k)
    y = _gpu_gemm(Q, out, wq, n, k, offsets=off, row_token=rt).cpu().numpy()
    exp, bound = _oracle(out, wq, k, off, rt)
    _assert_close(y, exp, bound)


@pytest.mark.parametrize("h,k", [(2048, 64), (512, 64), (512, 0)])
def test_expert_tails(Q, h, k):
    """Experts of 256, 257, 300, 320 and 321 rows (and smaller ones, and an
    empty one) near 256 rows per expert on average.  At K = 2048 the rows
    past 256 of an expert of 257 .. 320 rows go to the decode kernel and the
    rest to full 256-row tiles of the long-chain kernel; at K = 512 the
    single-chain kernel splits such experts over two tiles.  Every row is
    checked, plain and SwiGLU."""
    counts = np.array([256, 257, 300, 0, 320, 321, 100, 250], np.int64)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rows = int(off[-1])
    rng = np.random.default_rng(h + k)
    x = synth.f32_to_bf16_bits(rng.standard_normal((rows, h)).astype(np.float32))
    feat = 96
    w = synth.weights(rng, len(counts), 2 * feat, h)
    out, wq = _operands(x, w, k)
    print(f"expert tails K={h} k={k}", flush=True)
    y = _gpu_gemm(Q, out, wq, 2 * feat, k, offsets=off).cpu().numpy()
    exp, bound = _oracle(out, wq, k, off)
    _assert_close(y, exp, bound)
    hh = _gpu_gemm(Q, out, wq, 2 * feat, k, offsets=off, epilogue=Q.EPI_SWIGLU,
                   out_dtype=Q.OUT_BF16).cpu().numpy().view(np.uint16)
    ref = F.bf16_to_f64(OM.swiglu(y.astype(np.float64)))
    got = F.bf16_to_f64(hh)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126))) - 7)
    assert np.all(np.abs(got - ref) <= ulp * 1.0001)


@pytest.mark.parametrize("k,h,feat", [(16, 192, 80), (64, 256, 200), (0, 128, 64),
                                      (512, 1024, 200), (1024, 2048, 96)])
def test_grouped_swiglu(Q, k, h, feat):
    ids, x, w = _moe_case(9 + k, 600, 6, 2, h, 2 * feat, k)
    off, rt, pos = OM.pack_routes(ids, 6)
    out, wq = _operands(x, w, k)
    g = _gpu_gemm(Q, out, wq, 2 * feat, k, offsets=off, row_token=rt).cpu().numpy()
    exp, bound = _oracle(out, wq, k, off, rt)
    _assert_close(g, exp, bound)
    h = _gpu_gemm(Q, out, wq, 2 * feat, k, offsets=off, row_token=rt, epilogue=Q.EPI_SWIGLU,
                  out_dtype=Q.OUT_BF16).cpu().numpy().view(np.uint16)
    ref = F.bf16_to_f64(OM.swiglu(g.astype(np.float64)))
    got = F.bf16_to_f64(h)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126))) - 7)
    assert np.all(np.abs(got - ref) <= ulp * 1.0001)


def test_moe_config3_gate_up_sampled(Q):
    """Full gate/up GEMM of the 128-expert layer (32768 packed rows, K = 2048,
    N = 1536, k = 64); the oracle checks 12 experts' rows."""
    d = synth.make(3, with_weights=False)
    rng = np.random.default_rng(31)
    ids = d["topk_ids"]
    off, rt, pos = OM.pack_routes(ids, 128)
    out = OR.rac_quantize(F.bf16_to_f64(d["x"]), 64)
    experts = [0, 1, 17, 40, 63, 64, 90, 100, 111, 120, 126, 127]
    # unsampled experts hold all-zero weights (codes, scales and tensor scale 0)
    wp = np.zeros((128, 1536, 1024), np.uint8)
    ws = np.zeros((128, 1536, 128), np.uint8)
    wt = np.zeros(128, np.float32)
    wsub = synth.weights(rng, len(experts), 1536, 2048)
    for i, e in enumerate(experts):
        wp[e], ws[e], wt[e] = ON.quantize_bf16(wsub[i])
    print("config3 gate_up gemm", flush=True)
    y = _gpu_gemm(Q, out, (wp, ws, wt), 1536, 64, offsets=off, row_token=rt).cpu().numpy()
    for e in experts:
        sub_off = np.array([0, off[e + 1] - off[e]])
        sub_rt = rt[off[e]:off[e + 1]]
        exp, bound = OM.grouped_gemm(
            (out["nib"], out["scale"], out["ts"]), (out["r_nib"], out["r_scale"], out["r_ts"]),
            out["sel"], (wp[e:e + 1], ws[e:e + 1], wt[e:e + 1]), sub_off, sub_rt)
        _assert_close(y[off[e]:off[e + 1]], exp, bound)


def test_dense_config2_sampled(Q):
    """Config 2 shape (4096 x 4096 x 4096, k = 128); the oracle checks 256 rows."""
    d = synth.make(2)
    out, wq = _operands(d["x"], d["w"], 128)
    print("config2 gemm", flush=True)
    y = _gpu_gemm(Q, out, wq, 4096, 128).cpu().numpy()
    rows = np.random.default_rng(2).choice(4096, 256, replace=False)
    sub = dict(out)
    for key in ("nib", "scale", "r_nib", "r_scale"):
        sub[key] = out[key][rows]
    exp, bound = _oracle(sub, wq, 128, [0, 256])
    rel = _assert_close(y[rows], exp, bound)
    print("max relative error", rel)


@pytest.mark.parametrize("p2,lo,hi", [(50, -80, -60), (62, -200, -80)])
def test_tiny_residual_scale(Q, p2, lo, hi):
    """s_tR / s_tA far below 1.  Between 2^-80 and 2^-60 the main accumulator
    is scaled up by s_tA / s_tR before the compensation stage; below 2^-80 the
    compensation runs first with gathered weight columns.  Both must match."""
    rng = np.random.default_rng(41)
    x = (rng.standard_normal((80, 256)) * 2.0 ** -10).astype(np.float32)
    x[:, :16] = 0.0
    x[0, 0] = 2688.0 * 2.0 ** p2        # s_t = 2^p2 exactly, so this element has r = 0
    out, wq = _operands(synth.f32_to_bf16_bits(x), synth.weights(rng, 1, 64, 256), 64)
    assert 2.0 ** lo < out["r_ts"] / out["ts"] < 2.0 ** hi
    y = _gpu_gemm(Q, out, wq, 64, 64).cpu().numpy()
    exp, bound = _oracle(out, wq, 64, [0, 80])
    _assert_close(y, exp, bound)


@pytest.mark.parametrize("k", [64, 192])
def test_compensation_chunks_across_stages(Q, k):
    """Selected channels spread over many K stages, several 64-column chunks."""
    rng = np.random.default_rng(42 + k)
    x = rng.standard_normal((300, 1024)).astype(np.float32)
    x[:, rng.choice(1024, 40, replace=False)] *= 30
    out, wq = _operands(synth.f32_to_bf16_bits(x), synth.weights(rng, 1, 320, 1024), k)
    y = _gpu_gemm(Q, out, wq, 320, k).cpu().numpy()
    exp, bound = _oracle(out, wq, k, [0, 300])
    _assert_close(y, exp, bound)
