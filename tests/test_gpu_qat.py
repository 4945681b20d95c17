"""Trainer-side W4A16 QAT op (QUADS section 3.2, Eq. (12), (13), (16)) on the GPU.

* The learner's W_hat equals, bit for bit, the oracle's bf16 weight QDQ and
  the bf16 image of the exact decode of the codes the rollout quantizer
  writes for the same master weights (Eq. (16): ||dW_q|| = 0 on the bf16 grid).
* With a power-of-two tensor scale the learner's bf16 values are the
  rollout's exact values.
* Backward is straight-through (Eq. (13)); dL/dX = dY W_hat.
"""

import numpy as np
import pytest
import torch

import synth
from nvfp4_w4a4_quantized_act_amd import qat
from oracle import formats as F
from oracle import nvfp4 as ON

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def Q():
    import nvfp4_w4a4_quantized_act_amd as lib
    lib.lib()
    return lib


def _bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda:0").view(
        torch.bfloat16)


def test_qat_qdq_equals_rollout_codes(Q):
    w_bits = synth.weights(np.random.default_rng(7), 3, 96, 256)
    w = _bf16(w_bits)
    w_hat = qat.weight_qdq(w)
    # the rollout's own quantization of the same master weights
    nib, scale, ts, _ = Q.quads_nvfp4_weight_qdq(w.view(torch.int16))
    torch.cuda.synchronize()
    got = w_hat.view(torch.int16).cpu().numpy().view(np.uint16)
    wp, ws, wt, wdq = ON.weight_qdq(w_bits)
    assert np.array_equal(got, wdq)
    assert np.array_equal(nib.cpu().numpy(), wp) and np.array_equal(scale.cpu().numpy(), ws)
    assert np.array_equal(ts.cpu().numpy(), wt)
    for e in range(3):                       # bf16 of the exact rollout decode
        exact = ON.dequantize(nib[e].cpu().numpy(), scale[e].cpu().numpy(), ts[e].item())
        assert np.array_equal(got[e], F.f64_to_bf16_rne(exact))
    # a 2-D master weight gives the same as its one-expert 3-D form
    assert torch.equal(qat.weight_qdq(w[1]).view(torch.int16), w_hat[1].view(torch.int16))


def test_qat_power_of_two_scale_is_exact(Q):
    # amax = 2688 * 2^-12 gives s_t = 2^-12: every decode v * s_b * s_t has at
    # most 6 significant bits, so the bf16 QDQ is the exact rollout value
    rng = np.random.default_rng(8)
    w = rng.uniform(-0.6, 0.6, size=(64, 128)).astype(np.float32)
    w[0, 0] = 2688.0 * 2.0 ** -12
    w_bits = synth.f32_to_bf16_bits(w)
    assert F.bf16_to_f64(w_bits).max() == 2688.0 * 2.0 ** -12
    w_hat = qat.weight_qdq(_bf16(w_bits))
    torch.cuda.synchronize()
    wp, ws, wt = ON.quantize_bf16(w_bits)
    assert wt == np.float32(2.0 ** -12)
    exact = ON.dequantize(wp, ws, wt)
    assert np.array_equal(F.bf16_to_f64(w_hat.view(torch.int16).cpu().numpy().view(np.uint16)),
                          exact)


def test_qat_linear_forward_and_ste_backward(Q):
    rng = np.random.default_rng(9)
    w_bits = synth.weights(rng, 1, 64, 128)[0]
    x_bits = synth.f32_to_bf16_bits(rng.standard_normal((2, 8, 128)).astype(np.float32))
    w = _bf16(w_bits).requires_grad_(True)
    x = _bf16(x_bits).requires_grad_(True)
    y = qat.qat_linear(x, w)
    assert y.shape == (2, 8, 64) and y.dtype == torch.bfloat16
    gy = torch.ones_like(y)
    y.backward(gy)
    torch.cuda.synchronize()
    w_hat = F.bf16_to_f64(ON.weight_qdq(w_bits[None])[3][0])
    xf = F.bf16_to_f64(x_bits).reshape(-1, 128)
    # forward: the learner's product with W_hat (bf16 inputs, fp32 accumulation)
    y_ref = xf @ w_hat.T
    y_got = y.detach().float().cpu().numpy().reshape(-1, 64)
    assert np.allclose(y_got, y_ref, rtol=2 ** -7, atol=1e-3)
    # STE: dL/dW = dL/dW_hat = gy^T x; dL/dX = gy W_hat
    gw_ref = np.ones((16, 64)).T @ xf
    gx_ref = np.ones((16, 64)) @ w_hat
    assert np.allclose(w.grad.float().cpu().numpy(), gw_ref, rtol=2 ** -7, atol=1e-2)
    assert np.allclose(x.grad.float().cpu().numpy().reshape(-1, 128), gx_ref, rtol=2 ** -7,
                       atol=1e-3)
