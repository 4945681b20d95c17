"""GPU accuracy sweep (QUADS section 4.3.3, Table 3; section 3.3, Fig. 4(b))
at reduced sizes: the error figures the sweep reports from the library's RAC
and GEMM equal the oracle's figures for the same inputs, for every k, and
fall with k; the figures of the approximate MX modes (FP4 and FP8 elements,
E8M0 per 32, and MX FP4 with RAC for every k) equal the oracle's MX figures,
and MX FP4's error falls with k too."""

import numpy as np
import pytest
import torch

import synth
from nvfp4_w4a4_quantized_act_amd import sweep as S
from oracle import formats as F
from oracle import moe as OM
from oracle import mx as OX
from oracle import nvfp4 as ON
from oracle import rac as OR

pytestmark = pytest.mark.gpu

DENSE = dict(m=256, k_dim=1024, n=256)
MOE = dict(t=128, e=16, h=512, i=256)


@pytest.fixture(scope="module")
def Q():
    import nvfp4_w4a4_quantized_act_amd as lib
    lib.lib()
    return lib


def _oracle_rows(x_bits, w_bits, offsets, row_token, kdim):
    """The sweep's figures computed with the oracle (fp64 throughout)."""
    x = F.bf16_to_f64(x_bits)
    e = w_bits.shape[0]
    wp, ws, wt, wdq = ON.weight_qdq(w_bits)       # wdq: the trainer's bf16 weights
    w = (wp, ws, wt)
    rows = int(offsets[-1])
    xa = x[row_token] if row_token is not None else x
    y_qat = np.empty((rows, w_bits.shape[1]))
    y_16 = np.empty_like(y_qat)
    for j in range(e):
        sl = slice(offsets[j], offsets[j + 1])
        y_qat[sl] = xa[sl] @ F.bf16_to_f64(wdq[j]).T
        y_16[sl] = xa[sl] @ F.bf16_to_f64(w_bits[j]).T
    out = []
    for f in S.FRACTIONS:
        k = S.channels_for(f, kdim)
        o = OR.rac_quantize(x, k)
        r = (o["r_nib"], o["r_scale"], o["r_ts"]) if k else None
        y, _ = OM.grouped_gemm((o["nib"], o["scale"], o["ts"]), r, o["sel"], w, offsets,
                               row_token)
        out.append(S._errors(y, y_qat, y_16))
    return out


def _oracle_mx(x_bits, w_bits, offsets, row_token):
    """rel_bf16 and max_bf16 of the MX modes, with the oracle's MX quantizer
    and GEMM (fp64)."""
    x = F.bf16_to_f64(x_bits)
    e, n, kdim = w_bits.shape
    wf = F.bf16_to_f64(w_bits)
    rows = int(offsets[-1])
    xa = x[row_token] if row_token is not None else x
    y_16 = np.empty((rows, n))
    for j in range(e):
        sl = slice(offsets[j], offsets[j + 1])
        y_16[sl] = xa[sl] @ wf[j].T
    out = {}
    for fmt in ("fp4", "fp8"):
        a = OX.quantize(x, fmt)
        wc, wsc = OX.quantize(wf.reshape(e * n, kdim), fmt)
        y, _ = OX.grouped_gemm(a, (wc.reshape(e, n, -1), wsc.reshape(e, n, -1)), offsets,
                               row_token, fmt)
        out["mx" + fmt] = (np.linalg.norm(y - y_16) / np.linalg.norm(y_16),
                           np.abs(y - y_16).max() / np.abs(y_16).max())
    wc, wsc = OX.quantize(wf.reshape(e * n, kdim), "fp4")
    wq = (wc.reshape(e, n, -1), wsc.reshape(e, n, -1))
    for f in S.FRACTIONS:
        k = S.channels_for(f, kdim)
        if k == 0:
            continue
        o = OX.rac_quantize(x, k, "fp4")
        y, _ = OX.grouped_gemm_rac((o["codes"], o["scales"]), (o["r_codes"], o["r_scales"]),
                                   o["sel"], wq, offsets, row_token, "fp4")
        out[("mxfp4+rac", k)] = (np.linalg.norm(y - y_16) / np.linalg.norm(y_16),
                                 np.abs(y - y_16).max() / np.abs(y_16).max())
    return out


def _compare_mx(got, exp):
    rows = [g for g in got if g["format"] in ("mxfp4", "mxfp8")]
    assert [g["format"] for g in rows] == ["mxfp4", "mxfp8"]
    rac = [g for g in got if g["format"] == "mxfp4+rac"]
    assert len(rac) == len(S.FRACTIONS) - 1
    for g in rows + rac:
        rel, mx = exp[g["format"] if g["format"] != "mxfp4+rac" else (g["format"], g["k"])]
        assert abs(g["rel_bf16"] - rel) <= 1e-3 * rel + 1e-6, (g, rel)
        assert abs(g["max_bf16"] - mx) <= 1e-3 * mx + 1e-6, (g, mx)
    # RAC lowers the MX FP4 error as k grows
    errs = [rows[0]["rel_bf16"]] + [g["rel_bf16"] for g in rac]
    assert all(a > b for a, b in zip(errs, errs[1:])), errs
    # the exact NVFP4 path without RAC, against the same bf16 product
    nv = [g for g in got if g["format"] == "nvfp4" and g["k"] == 0][0]
    print("rel. error vs bf16: nvfp4 %.5f, mxfp4 %.5f, mxfp8 %.5f"
          % (nv["rel_bf16"], rows[0]["rel_bf16"], rows[1]["rel_bf16"]))


def _compare(got, exp):
    got = [g for g in got if g["format"] == "nvfp4"]
    assert len(got) == len(exp)
    for g, e in zip(got, exp):
        for key in ("rel_qat", "rel_bf16", "max_qat"):
            assert abs(g[key] - e[key]) <= 2e-5 * max(1.0, e[key]), (g, e)
    rel = [g["rel_qat"] for g in got]
    assert all(a > b for a, b in zip(rel, rel[1:])), rel


def test_sweep_dense_matches_oracle(Q):
    print("sweep: dense", DENSE, flush=True)
    got = S.sweep_dense(Q, torch, synth, torch.device("cuda:0"), **DENSE)
    d = synth.make(2, **DENSE)
    exp = _oracle_rows(d["x"], d["w"], np.array([0, DENSE["m"]]), None, DENSE["k_dim"])
    assert [g["k"] for g in got if g["format"] == "nvfp4"] == [0, 128, 256, 512, 768, 1024]
    _compare(got, exp)
    _compare_mx(got, _oracle_mx(d["x"], d["w"], np.array([0, DENSE["m"]]), None))


def test_sweep_moe_matches_oracle(Q):
    print("sweep: moe", MOE, flush=True)
    got = S.sweep_moe(Q, torch, synth, torch.device("cuda:0"), **MOE)
    d = synth.make(3, **MOE)
    off, rt, _ = OM.pack_routes(d["topk_ids"], MOE["e"])
    exp = _oracle_rows(d["x"], d["w13"], off, rt, MOE["h"])
    assert got[0]["rows"] == MOE["t"] * 8
    _compare(got, exp)
    _compare_mx(got, _oracle_mx(d["x"], d["w13"], off, rt))
