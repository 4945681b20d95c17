"""GPU parity: token packing (bit-exact) and the MoE combine (fp32 within a
rounding bound) against the oracle."""

import numpy as np
import pytest
import torch

import synth
from oracle import moe as OM

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def Q():
    import nvfp4_w4a4_quantized_act_amd as lib
    lib.lib()
    return lib


def _pack_check(Q, ids, e):
    print(f"pack T={ids.shape[0]} topk={ids.shape[1]} E={e}", flush=True)
    off, rt, pos = Q.quads_moe_pack(torch.from_numpy(ids).to("cuda:0"), e)
    torch.cuda.synchronize()
    eo, er, ep = OM.pack_routes(ids, e)
    assert np.array_equal(off.cpu().numpy(), eo)
    assert np.array_equal(rt.cpu().numpy(), er)
    assert np.array_equal(pos.cpu().numpy(), ep)
    return off, rt, pos


@pytest.mark.parametrize("cfg", [3, 4, 5])
def test_pack_configs(Q, cfg):
    d = synth.make(cfg, with_weights=False)
    _pack_check(Q, d["topk_ids"], synth.CONFIGS[cfg]["e"])


@pytest.mark.parametrize("t,e,topk", [(1, 1, 1), (3, 5, 2), (1000, 7, 3), (513, 4096, 8),
                                      (2000, 1, 1), (512, 128, 8), (455, 300, 9), (513, 128, 8),
                                      (4000, 256, 4), (65536, 4, 2), (4100, 6, 2)])
def test_pack_small_and_edge(Q, t, e, topk):
    """Every packing path: one work-group up to 4096 pairs and 512 experts
    (512 x 8 is the largest such case, 455 x 9 has 300 experts); the count
    and the scatter that sums the counts itself for up to 16384 per-chunk
    counts with E % 4 == 0 (513 x 8 over 128 experts with a ragged last
    chunk, 4000 x 4 over 256, 65536 x 2 over 4 experts: 512 chunks); three
    launches otherwise (4096 experts; 6 experts)."""
    rng = np.random.default_rng(t + e)
    ids = np.stack([rng.choice(e, topk, replace=False) for _ in range(t)]).astype(np.int32)
    _pack_check(Q, ids, e)


def test_pack_skewed_and_empty(Q):
    ids = np.zeros((3000, 2), np.int32)
    ids[:, 1] = 5                      # two experts take everything, others empty
    _pack_check(Q, ids, 64)
    off, rt, pos = Q.quads_moe_pack(torch.zeros((0, 8), dtype=torch.int32, device="cuda:0"), 16)
    torch.cuda.synchronize()
    assert off.cpu().tolist() == [0] * 17


@pytest.mark.parametrize("bf16", [False, True])
def test_combine(Q, bf16):
    d = synth.make(3, t=512, with_weights=False)
    ids, w = d["topk_ids"], d["topk_w"]
    off, rt, pos = _pack_check(Q, ids, 128)
    rng = np.random.default_rng(9)
    n = 2048
    y = rng.standard_normal((512 * 8, n)).astype(np.float32)
    if bf16:
        yb = synth.f32_to_bf16_bits(y)
        ty = torch.from_numpy(yb.view(np.int16)).to("cuda:0")
        y = (yb.astype(np.uint32) << 16).view(np.float32)
    else:
        ty = torch.from_numpy(y).to("cuda:0")
    out = Q.quads_moe_combine(ty, pos, torch.from_numpy(w).to("cuda:0"),
                              y_dtype=Q.OUT_BF16 if bf16 else Q.OUT_F32)
    torch.cuda.synchronize()
    exp = OM.combine(y, OM.pack_routes(ids, 128)[2], w, 512, 8)
    bound = OM.combine(np.abs(y), OM.pack_routes(ids, 128)[2], np.abs(w), 512, 8)
    err = np.abs(out.cpu().numpy() - exp)
    assert np.all(err <= 8 * 2.0 ** -24 * bound + 1e-30)


def test_empty_layer_calls(Q):
    """Size-0 inputs through the bindings (null data pointers): a GEMM over no
    rows, the SwiGLU GEMM with partial maxima, and a combine over no tokens
    return empty outputs without error."""
    dev = "cuda:0"
    e, n, kd = 4, 64, 256
    rng = np.random.default_rng(3)
    w = (torch.from_numpy(rng.integers(0, 256, (e, n, kd // 2), dtype=np.uint8)).to(dev),
         torch.from_numpy(rng.integers(40, 71, (e, n, kd // 16), dtype=np.uint8)).to(dev),
         torch.full((e,), 2.0 ** -6, dtype=torch.float32, device=dev))
    a = (torch.empty((0, kd // 2), dtype=torch.uint8, device=dev),
         torch.empty((0, kd // 16), dtype=torch.uint8, device=dev),
         torch.ones(1, dtype=torch.float32, device=dev))
    off = torch.zeros(e + 1, dtype=torch.int32, device=dev)
    rt = torch.empty(0, dtype=torch.int32, device=dev)
    y = Q.quads_moe_w4a4_gemm(a, w, n, rows=0, offsets=off, row_token=rt)
    h, part = Q.quads_moe_w4a4_gemm_amax(a, w, n, rows=0, offsets=off, row_token=rt)
    out = Q.quads_moe_combine(torch.empty((0, n), dtype=torch.float32, device=dev),
                              torch.empty((0, 2), dtype=torch.int32, device=dev),
                              torch.empty((0, 2), dtype=torch.float32, device=dev))
    torch.cuda.synchronize()
    assert tuple(y.shape) == (0, n) and tuple(h.shape) == (0, n // 2)
    assert tuple(out.shape) == (0, n)
