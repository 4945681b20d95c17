"""GPU parity on the three MoE workloads at full size.

Config 3 (the prefill layer: 4096 tokens, softmax top-8 over 128 experts,
hidden 2048, intermediate 768, k = 64) runs as a whole layer, stage by stage,
through the same calls and launch configuration the benchmark times: RAC(x)
bit-exact, pack bit-exact, the gate/up GEMM with the SwiGLU bf16 epilogue,
RAC(h) bit-exact on the GPU's h, the down GEMM with bf16 output, combine.
The gate/up GEMM is the form that also writes the partial maxima of |h|, and
RAC(h) takes max|h| from them, as the benchmark runs it.  All 128 experts
carry NVFP4 weights; 16 sampled experts (the 8 tallest, all
above 256 rows so each spans two row tiles, the 4 shortest and 4 from the
middle) are checked row by row against the oracle, and every other expert on
its first and last packed row.

Config 4 (decode: 64 tokens, Zipf(1.2) routing over 128 experts, hidden 2048,
intermediate 768, k = 64) runs as a whole layer the same way.  In both, each
stage's oracle gets the GPU's actual input to that stage (the GPU's SwiGLU
output h for the down-site RAC, the oracle's quantized operands for each
GEMM), so the bit-exact checks stay meaningful down the chain.

Config 5 (64 experts, hidden 4096, intermediate 1536, 16384 tokens, uniform
routing, Student-t(2.5) body with 82 outlier channels x32): the gate/up RAC
bit-exact at full size, then the gate/up GEMM (131072 packed rows) for
k = 0, 64, 256 and 2048 (half the channels; this k takes the kernel that
gathers the compensation columns) with the oracle checking sampled experts
and every other expert's rows exactly zero.

Weights: sampled experts get the oracle's NVFP4 QDQ of N(0, 0.02) bf16
weights.  In config 3 every other expert gets a sampled expert's codes with
their rows (codes and block scales together) in a random order of its own;
in configs 4 and 5 the other experts get all-zero codes, scales and tensor
scale, so their outputs must be exactly 0.  Tolerances as in test_gpu_gemm."""

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


def _np_bits(t):
    return t.cpu().numpy().view(np.uint16)


def _assert_rac_equal(g, e):
    assert g["ts"].item() == e["ts"]
    assert np.array_equal(g["scale"].cpu().numpy(), e["scale"])
    assert np.array_equal(g["nib"].cpu().numpy(), e["nib"])
    assert np.array_equal(g["sel"].cpu().numpy(), e["sel"])
    assert g["r_ts"].item() == e["r_ts"]
    assert np.array_equal(g["r_scale"].cpu().numpy(), e["r_scale"])
    assert np.array_equal(g["r_nib"].cpu().numpy(), e["r_nib"])


def _assert_close(got, exp, bound, bf16=False):
    err = np.abs(got - exp)
    lim = TOL * bound
    if bf16:
        lim = lim + np.abs(exp) * 2.0 ** -8
    bad = err > lim
    assert not bad.any(), (np.argwhere(bad)[:5], err[bad][:5], lim[bad][:5])


def _sampled_weights(rng, E, N, K, experts):
    """[E, N, K] NVFP4 weights: oracle QDQ of N(0, 0.02) for `experts`, zero elsewhere."""
    wp = np.zeros((E, N, K // 2), np.uint8)
    ws = np.zeros((E, N, K // 16), np.uint8)
    wt = np.zeros(E, np.float32)
    for e in experts:
        wp[e], ws[e], wt[e] = ON.quantize_bf16(synth.weights(rng, 1, N, K)[0])
    return wp, ws, wt


def _ops(out, k):
    a = (_t(out["nib"]), _t(out["scale"]), _t(np.array([out["ts"]], np.float32)))
    r = (_t(out["r_nib"]), _t(out["r_scale"]), _t(np.array([out["r_ts"]], np.float32))) \
        if k else None
    return a, r, (_t(out["sel"]) if k else None)


def _check_rows(y, out, k, w, off, rt, experts, bf16=False):
    """Sampled experts against the oracle; every other expert's rows exactly 0."""
    E = len(off) - 1
    r = (out["r_nib"], out["r_scale"], out["r_ts"]) if k else None
    for e in range(E):
        rows = slice(off[e], off[e + 1])
        if e not in experts:
            assert np.all(y[rows] == 0), e
            continue
        sub_off = np.array([0, off[e + 1] - off[e]])
        # packed A rows of the expert (identity order when there is no row_token)
        sub_rt = np.arange(off[e], off[e + 1], dtype=np.int32) if rt is None \
            else rt[off[e]:off[e + 1]]
        exp, bound = OM.grouped_gemm((out["nib"], out["scale"], out["ts"]), r, out["sel"],
                                     (w[0][e:e + 1], w[1][e:e + 1], w[2][e:e + 1]), sub_off,
                                     sub_rt)
        _assert_close(y[rows], exp, bound, bf16)


def test_config4_decode_layer(Q):
    d = synth.make(4, with_weights=False)
    T, E, H, I, TOPK, K = 64, 128, 2048, 768, 8, 64
    x, ids, tw = d["x"], d["topk_ids"], d["topk_w"]
    print("config4: rac(x)", flush=True)
    g = Q.quads_rac_quantize(_t(x), K)
    e = OR.rac_quantize(F.bf16_to_f64(x), K)
    torch.cuda.synchronize()
    _assert_rac_equal(g, e)

    print("config4: pack", flush=True)
    off_g, rt_g, pos_g = Q.quads_moe_pack(_t(ids), E)
    off, rt, pos = OM.pack_routes(ids, E)
    assert np.array_equal(off_g.cpu().numpy(), off)
    assert np.array_equal(rt_g.cpu().numpy(), rt)
    assert np.array_equal(pos_g.cpu().numpy(), pos)

    counts = np.diff(off)
    active = np.nonzero(counts)[0]
    by_load = active[np.argsort(counts[active], kind="stable")]
    experts = sorted({int(by_load[0]), int(by_load[len(by_load) // 2]), int(by_load[-1]),
                      int(by_load[-2])})
    rng = np.random.default_rng(44)
    w13 = _sampled_weights(rng, E, 2 * I, H, experts)
    w2 = _sampled_weights(rng, E, H, I, experts)
    w13_t = tuple(_t(v) for v in w13)
    w2_t = tuple(_t(v) for v in w2)
    rows = T * TOPK

    print("config4: gate/up gemm", flush=True)
    a, r, sel = _ops(e, K)
    y1 = Q.quads_moe_w4a4_gemm(a, w13_t, 2 * I, rows=rows, r=r, sel=sel, offsets=_t(off),
                               row_token=_t(rt))
    h, hmax = Q.quads_moe_w4a4_gemm_amax(a, w13_t, 2 * I, rows=rows, r=r, sel=sel,
                                         offsets=_t(off), row_token=_t(rt))
    torch.cuda.synchronize()
    y1 = y1.cpu().numpy()
    _check_rows(y1, e, K, w13, off, rt, experts)
    ref = F.bf16_to_f64(OM.swiglu(y1.astype(np.float64)))
    got = F.bf16_to_f64(_np_bits(h))
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126))) - 7)
    assert np.all(np.abs(got - ref) <= ulp * 1.0001)

    print("config4: rac(h)", flush=True)
    hb = _np_bits(h)
    gh = Q.quads_rac_quantize_partials(h, K, hmax)       # max|h| from the GEMM's maxima
    eh = OR.rac_quantize(F.bf16_to_f64(hb), K)
    torch.cuda.synchronize()
    _assert_rac_equal(gh, eh)

    print("config4: down gemm", flush=True)
    a2, r2, sel2 = _ops(eh, K)
    y2 = Q.quads_moe_w4a4_gemm(a2, w2_t, H, rows=rows, r=r2, sel=sel2, offsets=_t(off),
                               out_dtype=Q.OUT_BF16)
    torch.cuda.synchronize()
    y2b = _np_bits(y2)
    _check_rows(F.bf16_to_f64(y2b), eh, K, w2, off, None, experts, bf16=True)

    print("config4: combine", flush=True)
    out = Q.quads_moe_combine(y2, pos_g, _t(tw), y_dtype=Q.OUT_BF16)
    torch.cuda.synchronize()
    yv = F.bf16_to_f64(y2b)
    exp = OM.combine(yv, pos, tw, T, TOPK)
    bound = OM.combine(np.abs(yv), pos, np.abs(tw), T, TOPK)
    assert np.all(np.abs(out.cpu().numpy() - exp) <= 8 * 2.0 ** -24 * bound + 1e-30)


def _layer_weights(rng, E, N, K, experts):
    """[E, N, K] NVFP4 weights in every expert: the oracle's QDQ of N(0, 0.02)
    for `experts`; each other expert takes a sampled expert's codes, block
    scales and tensor scale with its rows in a random order of its own."""
    wp, ws, wt = _sampled_weights(rng, E, N, K, experts)
    for e in range(E):
        if e in experts:
            continue
        src = experts[e % len(experts)]
        perm = rng.permutation(N)
        wp[e], ws[e], wt[e] = wp[src][perm], ws[src][perm], wt[src]
    return wp, ws, wt


def _check_expert_rows(y, out, k, w, off, rt, experts, bf16=False):
    """All rows of `experts`, and the first and last packed row of every other
    non-empty expert, against the oracle."""
    r = (out["r_nib"], out["r_scale"], out["r_ts"]) if k else None
    for e in range(len(off) - 1):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        picks = list(range(lo, hi)) if e in experts else sorted({lo, hi - 1})
        src = np.array(picks, np.int32) if rt is None else rt[picks]
        exp, bound = OM.grouped_gemm((out["nib"], out["scale"], out["ts"]), r, out["sel"],
                                     (w[0][e:e + 1], w[1][e:e + 1], w[2][e:e + 1]),
                                     np.array([0, len(picks)]), src)
        _assert_close(y[picks], exp, bound, bf16)


def test_config3_layer(Q):
    d = synth.make(3, with_weights=False)
    T, E, H, I, TOPK, K = 4096, 128, 2048, 768, 8, 64
    x, ids, tw = d["x"], d["topk_ids"], d["topk_w"]
    rows = T * TOPK
    print("config3: rac(x)", flush=True)
    g = Q.quads_rac_quantize(_t(x), K)
    e = OR.rac_quantize(F.bf16_to_f64(x), K)
    torch.cuda.synchronize()
    _assert_rac_equal(g, e)

    print("config3: pack", flush=True)
    off_g, rt_g, pos_g = Q.quads_moe_pack(_t(ids), E)
    off, rt, pos = OM.pack_routes(ids, E)
    assert np.array_equal(off_g.cpu().numpy(), off)
    assert np.array_equal(rt_g.cpu().numpy(), rt)
    assert np.array_equal(pos_g.cpu().numpy(), pos)

    counts = np.diff(off)
    order = np.argsort(counts, kind="stable")
    mid = len(order) // 2
    experts = sorted({int(v) for v in np.concatenate([order[-8:], order[:4],
                                                      order[mid - 2:mid + 2]])})
    assert len(experts) == 16
    # experts above 256 rows span two row tiles of the tiled kernel
    assert (counts[experts] > 256).sum() >= 4
    rng = np.random.default_rng(33)
    w13 = _layer_weights(rng, E, 2 * I, H, experts)
    w2 = _layer_weights(rng, E, H, I, experts)
    w13_t = tuple(_t(v) for v in w13)
    w2_t = tuple(_t(v) for v in w2)

    print("config3: gate/up gemm", flush=True)
    a, r, sel = _ops(e, K)
    y1 = Q.quads_moe_w4a4_gemm(a, w13_t, 2 * I, rows=rows, r=r, sel=sel, offsets=_t(off),
                               row_token=_t(rt))
    h, hmax = Q.quads_moe_w4a4_gemm_amax(a, w13_t, 2 * I, rows=rows, r=r, sel=sel,
                                         offsets=_t(off), row_token=_t(rt))
    torch.cuda.synchronize()
    y1 = y1.cpu().numpy()
    _check_expert_rows(y1, e, K, w13, off, rt, experts)
    # the SwiGLU bf16 epilogue on every row: within 1 bf16 ulp of the oracle's
    # SwiGLU of the same fp32 gate and up values
    ref = F.bf16_to_f64(OM.swiglu(y1.astype(np.float64)))
    got = F.bf16_to_f64(_np_bits(h))
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126))) - 7)
    assert np.all(np.abs(got - ref) <= ulp * 1.0001)
    del y1, ref, got

    print("config3: rac(h)", flush=True)
    hb = _np_bits(h)
    gh = Q.quads_rac_quantize_partials(h, K, hmax)       # max|h| from the GEMM's maxima
    eh = OR.rac_quantize(F.bf16_to_f64(hb), K)
    torch.cuda.synchronize()
    _assert_rac_equal(gh, eh)

    print("config3: down gemm", flush=True)
    a2, r2, sel2 = _ops(eh, K)
    y2 = Q.quads_moe_w4a4_gemm(a2, w2_t, H, rows=rows, r=r2, sel=sel2, offsets=_t(off),
                               out_dtype=Q.OUT_BF16)
    torch.cuda.synchronize()
    y2b = _np_bits(y2)
    yv = F.bf16_to_f64(y2b)
    _check_expert_rows(yv, eh, K, w2, off, None, experts, bf16=True)

    print("config3: combine", flush=True)
    out = Q.quads_moe_combine(y2, pos_g, _t(tw), y_dtype=Q.OUT_BF16)
    torch.cuda.synchronize()
    exp = OM.combine(yv, pos, tw, T, TOPK)
    bound = OM.combine(np.abs(yv), pos, np.abs(tw), T, TOPK)
    assert np.all(np.abs(out.cpu().numpy() - exp) <= 8 * 2.0 ** -24 * bound + 1e-30)


@pytest.fixture(scope="module")
def cfg5(Q):
    """Config 5 gate/up input, its GPU RAC (k = 256) checked bit-exact, routes."""
    d = synth.make(5, with_weights=False)
    x = d["x"]
    print("config5: rac(x), k=256", flush=True)
    g = Q.quads_rac_quantize(_t(x), 256)
    e = OR.rac_quantize(F.bf16_to_f64(x), 256)
    torch.cuda.synchronize()
    _assert_rac_equal(g, e)
    off, rt, pos = OM.pack_routes(d["topk_ids"], 64)
    experts = [3, 41]
    w13 = _sampled_weights(np.random.default_rng(55), 64, 2 * 1536, 4096, experts)
    return dict(e=e, off=off, rt=rt, x=x, experts=experts, w13=w13)


def _oracle_rac_k(e, k):
    """RAC outputs for k channels from a larger run: the scores do not depend
    on k, so S(k) and its second pass come from the same residual."""
    sel = OR.select_channels(e["score"], k)
    out = dict(e)
    out["sel"] = sel
    out["r_nib"], out["r_scale"], out["r_ts"] = ON.quantize(e["r"][:, sel].astype(np.float64))
    return out


@pytest.mark.parametrize("k", [0, 64, 256, 2048])
def test_config5_gate_up_sampled(Q, cfg5, k):
    I = 1536
    out = _oracle_rac_k(cfg5["e"], k)
    if k != 256:                          # the GPU RAC for this k, bit-exact
        g = Q.quads_rac_quantize(_t(cfg5["x"]), k)
        torch.cuda.synchronize()
        assert np.array_equal(g["sel"].cpu().numpy(), out["sel"])
        if k:
            assert g["r_ts"].item() == out["r_ts"]
            assert np.array_equal(g["r_nib"].cpu().numpy(), out["r_nib"])
            assert np.array_equal(g["r_scale"].cpu().numpy(), out["r_scale"])
    off, rt = cfg5["off"], cfg5["rt"]
    experts, w13 = cfg5["experts"], cfg5["w13"]
    print(f"config5: gate/up gemm k={k}", flush=True)
    a, r, sel = _ops(out, k)
    y = Q.quads_moe_w4a4_gemm(a, tuple(_t(v) for v in w13), 2 * I, rows=int(off[-1]), r=r,
                              sel=sel, offsets=_t(off), row_token=_t(rt))
    torch.cuda.synchronize()
    _check_rows(y.cpu().numpy(), out, k, w13, off, rt, experts)
