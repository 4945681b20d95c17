"""GPU accuracy sweep (QUADS section 4.3.3, Table 3; section 3.3, Fig. 4(b))
at reduced sizes: the error figures the sweep reports from the library's RAC
and GEMM equal the oracle's figures for the same inputs, for every k, and
fall with k."""

import numpy as np
import pytest
import torch

import synth
from nvfp4_w4a4_quantized_act_amd import sweep as S
from oracle import formats as F
from oracle import moe as OM
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


def _compare(got, exp):
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
    assert [g["k"] for g in got] == [0, 128, 256, 512, 768, 1024]
    _compare(got, exp)


def test_sweep_moe_matches_oracle(Q):
    print("sweep: moe", MOE, flush=True)
    got = S.sweep_moe(Q, torch, synth, torch.device("cuda:0"), **MOE)
    d = synth.make(3, **MOE)
    off, rt, _ = OM.pack_routes(d["topk_ids"], MOE["e"])
    exp = _oracle_rows(d["x"], d["w13"], off, rt, MOE["h"])
    assert got[0]["rows"] == MOE["t"] * 8
    _compare(got, exp)
