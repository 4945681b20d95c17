"""GPU parity: NVFP4 activation quantizer and weight QDQ against the oracle,
bit-exact on nibbles, scale bytes and tensor scales."""

import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from oracle import nvfp4 as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def Q():
    import nvfp4_w4a4_quantized_act_amd as lib
    lib.lib()
    return lib


def _up(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda:0")


def _check(Q, bits, ts=None):
    print(f"quantize shape={bits.shape} ts={ts}", flush=True)
    ts_t = None if ts is None else torch.tensor([ts], dtype=torch.float32, device="cuda:0")
    nib, sc, t = Q.quads_nvfp4_quantize(_up(bits), ts_t)
    torch.cuda.synchronize()
    en, es, et = O.quantize_bf16(bits, ts)
    gn, gs, gt = nib.cpu().numpy(), sc.cpu().numpy(), t.cpu().numpy()[0]
    assert gt == et, (gt, et)
    assert np.array_equal(gs, es), np.argwhere(gs != es)[:5]
    assert np.array_equal(gn, en), np.argwhere(gn != en)[:5]
    return nib, sc, t


@pytest.mark.parametrize("cfg", [1, 2])
def test_quantize_dense_configs(Q, cfg):
    d = synth.make(cfg, with_weights=False) if cfg > 2 else synth.make(cfg)
    _check(Q, d["x"])


def test_quantize_moe_inputs(Q):
    d = synth.make(3, with_weights=False)
    _check(Q, d["x"])
    d = synth.make(5, t=2048, with_weights=False)          # heavy tails, x32 outliers
    _check(Q, d["x"])


@pytest.mark.parametrize("m,k", [(1, 16), (37, 48), (3, 4096), (515, 272)])
def test_quantize_ragged(Q, m, k):
    rng = np.random.default_rng(m * 1000 + k)
    x = (rng.standard_t(2.5, (m, k)) * np.exp2(rng.integers(-3, 3, (m, 1)))).astype(np.float32)
    _check(Q, synth.f32_to_bf16_bits(x))


def test_quantize_ties_and_grid(Q):
    """Every element sits exactly on an E2M1 midpoint or grid point of its block
    scale: all ties, resolved to even codes."""
    rng = np.random.default_rng(11)
    m, k = 64, 256
    sb = rng.integers(0x08, 0x7F, size=(m, k // 16))
    sb[0, 0] = 0x7E
    pts = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0])
    v = rng.choice(pts, size=(m, k)) * np.where(rng.random((m, k)) < 0.5, -1, 1)
    v[:, ::16] = 6.0
    x = v * np.repeat(F.E4M3_GRID[sb], 16, -1) * 2.0 ** -4
    bits = F.f64_to_bf16_rne(x)
    assert np.array_equal(F.bf16_to_f64(bits), x)
    _check(Q, bits)


def test_quantize_special_values(Q):
    rng = np.random.default_rng(12)
    x = np.zeros((8, 64), np.float32)
    x[0, :] = rng.standard_normal(64)
    x[1, :16] = 1e-38                                     # subnormal-ish fp32 -> bf16
    x[2, 5] = -0.0
    x[3, :] = rng.standard_normal(64) * 1e-6              # subnormal block scales
    x[4, :16] = 3e38                                      # near the bf16 maximum
    x[5, 3] = -3e38
    bits = synth.f32_to_bf16_bits(x)
    bits[2, 5] = 0x8000
    bits[6, :] = 0x0001                                   # smallest bf16 subnormal
    bits[7, ::2] = 0x8001
    _check(Q, bits)
    # a tensor of tiny values only: scales in the subnormal fp32 range
    tiny = np.full((2, 32), 0x0003, np.uint16)
    tiny[1, 7] = 0x807F
    _check(Q, tiny)
    _check(Q, np.zeros((4, 32), np.uint16))


def test_quantize_static_scale(Q):
    d = synth.make(1)
    _check(Q, d["x"], ts=np.float32(0.003))               # saturates some blocks
    _check(Q, d["x"], ts=np.float32(1.0))


def _all_magnitudes():
    """Every finite bf16 magnitude, each block of 16 holding one of them at
    its maximum (both signs), so every block maximum occurs."""
    mags = np.arange(0x0000, 0x7F80, dtype=np.uint16)         # 0 .. largest finite
    rows = len(mags) // 16 * 16
    blk = np.zeros((len(mags), 16), np.uint16)
    blk[:, 0] = mags
    blk[:, 1] = mags | 0x8000
    blk[:, 2:] = (mags[:, None] >> 1) + np.arange(14, dtype=np.uint16)[None, :] % 3
    return blk[:rows].reshape(-1, 256)


@pytest.mark.parametrize("ts", [2.0 ** -126, 2.0 ** -101, 2.0 ** -100, 3.1e-27, 1.0 / 2688,
                                0.0371, 1.0, 447.0, 6.0e9, 2.0 ** 100, 1.3e35])
def test_quantize_scale_codes_every_magnitude(Q, ts):
    """Caller-given tensor scales across the fp32 range, on blocks whose
    maxima run through every finite bf16 magnitude: block-scale codes and
    element codes bit-exact (the block-scale code comes from an fp32 quotient
    corrected against exact thresholds for s_t >= 2^-100, from the fp64
    quotient below)."""
    _check(Q, _all_magnitudes(), ts=np.float32(ts))


def test_quantize_empty(Q):
    x = torch.zeros((0, 64), dtype=torch.int16, device="cuda:0")
    nib, sc, t = Q.quads_nvfp4_quantize(x)
    torch.cuda.synchronize()
    assert nib.shape == (0, 32) and t.item() == 0.0


def test_quantize_deterministic(Q):
    d = synth.make(2, m=1024, k_dim=1024)
    x = _up(d["x"])
    a = Q.quads_nvfp4_quantize(x)
    b = Q.quads_nvfp4_quantize(x)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


@pytest.mark.parametrize("e,n,k", [(3, 40, 96), (1, 128, 256), (5, 7, 16)])
def test_weight_qdq(Q, e, n, k):
    rng = np.random.default_rng(e * 100 + n)
    w = synth.weights(rng, e, n, k)
    print(f"weight_qdq {e}x{n}x{k}", flush=True)
    nib, sc, ts, dq = Q.quads_nvfp4_weight_qdq(_up(w), want_dq=True)
    torch.cuda.synchronize()
    en, es, et, edq = O.weight_qdq(w)
    assert np.array_equal(ts.cpu().numpy(), et)
    assert np.array_equal(sc.cpu().numpy(), es)
    assert np.array_equal(nib.cpu().numpy(), en)
    assert np.array_equal(dq.cpu().numpy().view(np.uint16), edq)


def test_weight_qdq_moe_shapes(Q):
    """Weight QDQ at the gate/up shape of the 128-expert layer (a sample of
    experts checked against the oracle)."""
    rng = np.random.default_rng(3)
    w = synth.weights(rng, 16, 1536, 2048)
    nib, sc, ts, _ = Q.quads_nvfp4_weight_qdq(_up(w))
    torch.cuda.synchronize()
    for e in (0, 7, 15):
        en, es, et = O.quantize_bf16(w[e])
        assert ts[e].item() == et
        assert np.array_equal(sc[e].cpu().numpy(), es)
        assert np.array_equal(nib[e].cpu().numpy(), en)
