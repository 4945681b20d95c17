"""GPU parity: Residual Activation Compensation against the oracle -- main
NVFP4, channel scores (bitwise), selected channels, and the second-pass
nibbles, scale bytes and tensor scale, all bit-exact."""

import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from oracle import rac as OR

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


def _check(Q, bits, k):
    print(f"rac shape={bits.shape} k={k}", flush=True)
    g = Q.quads_rac_quantize(_up(bits), k, want_score=True)
    torch.cuda.synchronize()
    e = OR.rac_quantize(F.bf16_to_f64(bits), k)
    assert g["ts"].item() == e["ts"]
    assert np.array_equal(g["scale"].cpu().numpy(), e["scale"])
    assert np.array_equal(g["nib"].cpu().numpy(), e["nib"])
    gs = g["score"].cpu().numpy()
    assert np.array_equal(gs.view(np.uint64), e["score"].view(np.uint64)), \
        np.argwhere(gs != e["score"])[:5]
    assert np.array_equal(g["sel"].cpu().numpy(), e["sel"])
    assert g["r_ts"].item() == e["r_ts"]
    assert np.array_equal(g["r_scale"].cpu().numpy(), e["r_scale"])
    assert np.array_equal(g["r_nib"].cpu().numpy(), e["r_nib"])
    return g, e


def test_rac_config1(Q):
    d = synth.make(1)
    _check(Q, d["x"], d["rac_k"])


def test_rac_config2(Q):
    d = synth.make(2)
    _check(Q, d["x"], d["rac_k"])


def test_rac_moe_gate_up_site(Q):
    d = synth.make(3, with_weights=False)
    _check(Q, d["x"], 64)


def test_rac_moe_down_site_shape(Q):
    """Down-site shape of the 128-expert layer (packed rows x 768), heavy tails,
    several tree levels (32768 rows -> 512 -> 8 -> 1)."""
    rng = np.random.default_rng(21)
    x = rng.standard_t(3.0, (32768, 768)).astype(np.float32)
    x[:, rng.choice(768, 8, replace=False)] *= 20
    _check(Q, synth.f32_to_bf16_bits(x), 64)


@pytest.mark.parametrize("m,kd,k", [(1, 16, 16), (37, 48, 16), (65, 272, 32), (300, 1040, 256),
                                    (64, 256, 0), (5, 64, 64), (64, 2048, 64), (63, 1040, 32),
                                    (17, 2048, 0), (8, 2048, 32), (64, 256, 256), (4, 2064, 16)])
def test_rac_ragged(Q, m, kd, k):
    """Ragged shapes on both paths: one work-group for at most 64 rows, K <=
    2048 and at most 16384 elements (8 x 2048, 64 x 256), the launches
    otherwise (65 rows; 64 x 2048, the decode step's gate/up input; K = 2064)."""
    rng = np.random.default_rng(m + kd + k)
    x = (rng.standard_normal((m, kd)) * np.exp2(rng.integers(-2, 3, (1, kd)))).astype(np.float32)
    _check(Q, synth.f32_to_bf16_bits(x), k)


def test_rac_ties_in_score(Q):
    """Channels with identical residual columns tie exactly; the lower index wins."""
    rng = np.random.default_rng(22)
    base = rng.standard_normal((96, 16)).astype(np.float32)
    x = np.tile(base, (1, 8))                    # 8 identical 16-channel groups
    x[:, 40] *= 7.0
    _check(Q, synth.f32_to_bf16_bits(x), 32)


def test_rac_on_grid_input(Q):
    """Zero residual everywhere: all scores 0, S = {0..k-1}, r_ts = 0."""
    rng = np.random.default_rng(23)
    sb = rng.integers(0x30, 0x7F, size=(70, 8))
    sb[0, 0] = 0x7E
    mag = rng.integers(0, 8, size=(70, 128))
    mag[:, ::16] = 7
    x = F.E2M1_MAG[mag] * np.repeat(F.E4M3_GRID[sb], 16, -1)
    g, e = _check(Q, F.f64_to_bf16_rne(x), 48)
    assert list(e["sel"]) == list(range(48)) and e["r_ts"] == 0


def test_rac_all_zero_and_empty(Q):
    _check(Q, np.zeros((10, 64), np.uint16), 16)
    g = Q.quads_rac_quantize(torch.zeros((0, 64), dtype=torch.int16, device="cuda:0"), 32,
                             want_score=True)
    torch.cuda.synchronize()
    assert g["sel"].cpu().tolist() == list(range(32)) and g["r_ts"].item() == 0


def test_rac_full_k(Q):
    d = synth.make(1)
    _check(Q, d["x"], 256)


def test_rac_deterministic(Q):
    d = synth.make(2, m=2048, k_dim=2048)
    x = _up(d["x"])
    a = Q.quads_rac_quantize(x, 128, want_score=True)
    b = Q.quads_rac_quantize(x, 128, want_score=True)
    torch.cuda.synchronize()
    for key in a:
        assert torch.equal(a[key], b[key]), key
