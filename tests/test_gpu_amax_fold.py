"""The producer-fed tensor maximum (the down-site input's max|h| from the gate/up GEMM).

quads_moe_w4a4_gemm_amax writes one partial maximum of |h| per work-group of
its launches; the maximum over the slots must be the largest bf16 magnitude
of the h it stored, bit for bit, on every kernel path of the SwiGLU GEMM
(decode kernel alone, experts' tails plus the long-chain tiled kernel, the
single-chain 256 x 256 kernel, the small-tile kernel, and the gathered
compensation), every slot must be written (no stale value from an earlier
call), and h itself must equal the plain call's.  The quantizer and RAC fed
with those partials must then give the outputs of their dynamic-scale forms
bit for bit, and RAC(h) the oracle's (Eq. (9) / section 3.3 with max|h| from
the producer instead of a max pass).

Weights are random valid NVFP4 codes (random nibbles, block-scale codes in
[40, 70], a tensor scale of 2^-6), activations NVFP4 of seeded N(0, 1)
bf16: the checks concern where the maximum is taken, not the products
(whose parity is tested in test_gpu_gemm and test_gpu_configs)."""

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import rac as OR

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def Q():
    import nvfp4_w4a4_quantized_act_amd as lib
    lib.lib()
    return lib


def _weights(rng, E, N, K):
    nib = torch.from_numpy(rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)).to(DEV)
    sc = torch.from_numpy(rng.integers(40, 71, (E, N, K // 16), dtype=np.uint8)).to(DEV)
    ts = torch.full((E,), 2.0 ** -6, dtype=torch.float32, device=DEV)
    return nib, sc, ts


def _acts(Q, rng, T, K, k):
    x = torch.from_numpy(rng.standard_normal((T, K)).astype(np.float32)).to(DEV)
    x = x.to(torch.bfloat16)
    if k:
        g = Q.quads_rac_quantize(x, k)
        return (g["nib"], g["scale"], g["ts"]), (g["r_nib"], g["r_scale"], g["r_ts"]), g["sel"]
    n, s, t = Q.quads_nvfp4_quantize(x)[:3]
    return (n, s, t), None, None


def _routes(rng, T, topk, E, skew):
    """Offsets and row tokens of T tokens routed top-k over E experts (expert
    weights ~ Zipf(skew) when skew > 0, else uniform)."""
    p = np.ones(E) if skew == 0 else 1.0 / np.arange(1, E + 1) ** skew
    p = p / p.sum()
    ids = np.stack([rng.choice(E, topk, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    flat = ids.reshape(-1)
    order = np.argsort(flat, kind="stable")
    rt = (order // topk).astype(np.int32)
    off = np.zeros(E + 1, np.int32)
    off[1:] = np.cumsum(np.bincount(flat, minlength=E))
    return torch.from_numpy(off).to(DEV), torch.from_numpy(rt).to(DEV)


def _h_max_bits(h):
    b = h.view(torch.int16).cpu().numpy().view(np.uint16) & 0x7FFF
    return int(b.max()) if b.size else 0


CASES = [
    # name, T, topk, E, K, N, k, skew
    ("decode kernel", 64, 8, 128, 2048, 1536, 64, 1.2),
    ("tails + long-chain tiles", 4096, 8, 128, 2048, 1536, 64, 0.0),
    ("single chain 256x256", 272, 4, 4, 768, 768, 64, 0.0),
    ("small tiles", 150, 2, 2, 80, 64, 16, 0.0),
    ("gathered compensation", 512, 2, 4, 2048, 256, 1024, 0.0),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_gemm_amax_slots(Q, case):
    name, T, topk, E, K, N, k, skew = case
    print("amax:", name, flush=True)
    rng = np.random.default_rng(7)
    w = _weights(rng, E, N, K)
    a, r, sel = _acts(Q, rng, T, K, k)
    off, rt = _routes(rng, T, topk, E, skew)
    rows = T * topk
    groups = Q.quads_moe_w4a4_gemm_amax_groups(rows, K, k, E, N)
    assert groups > 0
    part = torch.full((groups + 3,), -1, dtype=torch.int32, device=DEV)   # sentinel
    h, _ = Q.quads_moe_w4a4_gemm_amax(a, w, N, rows=rows, r=r, sel=sel, offsets=off,
                                      row_token=rt, amax_part=part[:groups])
    h0 = Q.quads_moe_w4a4_gemm(a, w, N, rows=rows, r=r, sel=sel, offsets=off, row_token=rt,
                               epilogue=Q.EPI_SWIGLU, out_dtype=Q.OUT_BF16)
    torch.cuda.synchronize()
    assert torch.equal(h, h0), name
    p = part.cpu().numpy().view(np.uint32)
    assert np.all(p[:groups] <= 0x7FFF), name              # every slot written
    assert np.all(p[groups:] == 0xFFFFFFFF), name           # nothing past the slots
    hm = _h_max_bits(h)
    assert hm > 0
    assert int(p[:groups].max()) == hm, (name, int(p[:groups].max()), hm)


def test_gemm_amax_second_call_smaller(Q):
    """A second call with fewer rows into the same slots leaves nothing of the first."""
    rng = np.random.default_rng(11)
    E, K, N, k = 4, 768, 768, 64
    w = _weights(rng, E, N, K)
    groups = Q.quads_moe_w4a4_gemm_amax_groups(272 * 4, K, k, E, N)
    part = torch.empty(groups, dtype=torch.int32, device=DEV)
    for T, scale in ((272, 4.0), (40, 1.0)):
        a, r, sel = _acts(Q, rng, T, K, k)
        if scale != 1.0:
            a = (a[0], a[1], a[2] * scale)
        off, rt = _routes(rng, T, 4, E, 0.0)
        h, _ = Q.quads_moe_w4a4_gemm_amax(a, w, N, rows=T * 4, r=r, sel=sel, offsets=off,
                                          row_token=rt, amax_part=part)
        torch.cuda.synchronize()
        p = part.cpu().numpy().view(np.uint32)
        assert int(p.max()) == _h_max_bits(h), T


def _assert_same(g, e, keys):
    for key in keys:
        assert torch.equal(g[key], e[key]), key


@pytest.mark.parametrize("case", [CASES[0], CASES[2]], ids=["decode h", "single-chain h"])
def test_partials_consumers(Q, case):
    name, T, topk, E, K, N, k, skew = case
    rng = np.random.default_rng(5)
    w = _weights(rng, E, N, K)
    a, r, sel = _acts(Q, rng, T, K, k)
    off, rt = _routes(rng, T, topk, E, skew)
    rows = T * topk
    h, part = Q.quads_moe_w4a4_gemm_amax(a, w, N, rows=rows, r=r, sel=sel, offsets=off,
                                         row_token=rt)
    # the quantizer: the dynamic form bit for bit
    qn, qs, qt = Q.quads_nvfp4_quantize_partials(h, part)
    dn, ds, dt = Q.quads_nvfp4_quantize(h)[:3]
    torch.cuda.synchronize()
    assert torch.equal(qn, dn) and torch.equal(qs, ds) and torch.equal(qt, dt), name
    # RAC: the workspace form and the oracle bit for bit
    kr = 64
    g = Q.quads_rac_quantize_partials(h, kr, part, want_score=True)
    e = Q.quads_rac_quantize(h, kr, want_score=True)
    torch.cuda.synchronize()
    _assert_same(g, e, ("nib", "scale", "ts", "sel", "r_nib", "r_scale", "r_ts", "score"))
    o = OR.rac_quantize(F.bf16_to_f64(h.view(torch.int16).cpu().numpy().view(np.uint16)), kr)
    assert g["ts"].item() == o["ts"] and g["r_ts"].item() == o["r_ts"]
    assert np.array_equal(g["sel"].cpu().numpy(), o["sel"])
    assert np.array_equal(g["nib"].cpu().numpy(), o["nib"])
    assert np.array_equal(g["r_nib"].cpu().numpy(), o["r_nib"])
    assert np.array_equal(g["r_scale"].cpu().numpy(), o["r_scale"])
