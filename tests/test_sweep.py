"""Accuracy sweep (QUADS section 4.3.3, Table 3; section 3.3, Fig. 4(b)) on the
CPU: the channel-count rule of nvfp4_w4a4_quantized_act_amd.sweep, and the
trend the sweep reports, computed with the oracle on a small dense layer:
the output distance to the W4A16-QAT trainer's product X Wq^T (Wq the bf16
decode of the NVFP4 weights) falls at every step of k, and the distance to the bf16 product stays above the weight error
alone (the part RAC cannot remove)."""

import numpy as np

import synth
from nvfp4_w4a4_quantized_act_amd import sweep as S
from oracle import formats as F
from oracle import moe as OM
from oracle import nvfp4 as ON
from oracle import rac as OR


def test_channels_for():
    assert [S.channels_for(f, 4096) for f in S.FRACTIONS] == [0, 512, 1024, 2048, 3072, 4096]
    assert [S.channels_for(f, 2048) for f in S.FRACTIONS] == [0, 256, 512, 1024, 1536, 2048]
    assert S.channels_for(0.01, 1024) == 64          # never below one 64-channel stage
    assert S.channels_for(1.0, 768) == 768


def test_bf16_decode():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x4049, 0x7F7F], np.uint16)
    assert list(S._f64(bits)[:4]) == [1.0, -1.0, 0.0, 3.140625]
    assert S._f64(bits)[4] == (2 - 2 ** -7) * 2.0 ** 127          # largest finite bf16


def test_output_error_falls_with_k():
    d = synth.make(2, m=256, k_dim=1024, n=256)
    x = F.bf16_to_f64(d["x"])
    wp, ws, wt, wdq = ON.weight_qdq(d["w"])
    wp, ws, wt = wp[0], ws[0], wt[0]
    y_qat = x @ F.bf16_to_f64(wdq[0]).T              # the W4A16-QAT trainer's product
    y_16 = x @ F.bf16_to_f64(d["w"][0]).T
    w = (wp[None], ws[None], np.array([wt], np.float32))
    off = np.array([0, x.shape[0]])
    rel_qat, rel_16 = [], []
    for f in S.FRACTIONS:
        k = S.channels_for(f, x.shape[1])
        o = OR.rac_quantize(x, k)
        r = (o["r_nib"], o["r_scale"], o["r_ts"]) if k else None
        y, _ = OM.grouped_gemm((o["nib"], o["scale"], o["ts"]), r, o["sel"], w, off)
        e = S._errors(y, y_qat, y_16)
        rel_qat.append(e["rel_qat"])
        rel_16.append(e["rel_bf16"])
    assert all(a > b for a, b in zip(rel_qat, rel_qat[1:])), rel_qat
    weight_only = np.linalg.norm(y_qat - y_16) / np.linalg.norm(y_16)
    assert all(v > 0.9 * weight_only for v in rel_16), (rel_16, weight_only)
    assert rel_qat[-1] < 0.2 * rel_qat[0]
