"""Accuracy sweep: the output error of W4A4 and W4A4+RAC as the number of
compensated channels grows (QUADS, arXiv 2607.15810: section 4.3.3 with
Table 3, and section 3.3 with Fig. 4(b)).

The pages measure the training/inference gap on a model: the largest
log-probability difference (Table 3, residual ratios 12.5 % to 100 %) and the
per-layer MoE output distance (Fig. 4(b)).  With no model here, the same
quantity is taken at one GEMM on the synthetic workloads, every step on the
GPU through the library:

  Y(k)   W4A4 GEMM (fp32 out) of RAC(X, k) with the NVFP4 weights;
  Y_qat  X Wq^T in fp64, Wq = the library's NVFP4 QDQ of W in bf16: what the
         learner computes under asymmetric W4A16 QAT (section 3.2, Eq. (12)),
         so the gap left is the rollout's activation error that RAC targets
         (and the bf16 rounding of Wq);
  Y_16   X W^T in fp64 with the bf16 weights: no weight alignment.

Reported per k (0, 12.5, 25, 50, 75 and 100 % of K, rounded to 64 channels):
relative Frobenius distances |Y(k) - Y_qat| / |Y_qat| and |Y(k) - Y_16| /
|Y_16|, and the largest element error relative to max |Y_qat| (and to
max |Y_16|).

Beside them, the approximate MX modes of gfx950's block-scaled MFMA (one
power-of-two E8M0 scale per 32 elements instead of an E4M3 scale per 16; FP4
E2M1 and FP8 E4M3 elements, both operands quantized by quads_mx_quantize, the
product by quads_moe_mx_gemm): their distance to Y_16, the same product
format-for-format, with no trainer-side reference of their own; and MX FP4
with RAC (quads_mx_rac_quantize and quads_moe_mx_rac_gemm) for each k > 0.

Workloads: dense = X [4096, 4096] Student-t(3) with 41 outlier channels x20,
W [4096, 4096] N(0, 0.02); moe = the gate/up GEMM of the MoE layer, X [4096,
2048] with 20 outlier channels x20, 128 experts, top-8 softmax routing, W13
[128, 1536, 2048].  The fp64 references run on the host CPU (numpy).

    python -m nvfp4_w4a4_quantized_act_amd.sweep [--workloads dense,moe] [--tokens T]
"""

import argparse
import json
import os
import sys

import numpy as np

FRACTIONS = (0.0, 0.125, 0.25, 0.5, 0.75, 1.0)


def _f64(bits):
    """bf16 bit patterns (uint16 / int16) -> float64."""
    b = np.ascontiguousarray(bits).view(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def channels_for(frac, kdim):
    """k for a ratio of K: a multiple of 64 (the GEMM's stage), at least 64 when frac > 0."""
    if frac <= 0:
        return 0
    return int(min(kdim, max(64, round(frac * kdim / 64) * 64)))


def _errors(y, y_qat, y_16):
    d_qat = y - y_qat
    return dict(rel_qat=float(np.linalg.norm(d_qat) / np.linalg.norm(y_qat)),
                rel_bf16=float(np.linalg.norm(y - y_16) / np.linalg.norm(y_16)),
                max_qat=float(np.abs(d_qat).max() / np.abs(y_qat).max()),
                max_bf16=float(np.abs(y - y_16).max() / np.abs(y_16).max()))


def _mx_errors(y, y_16):
    return dict(rel_qat=None, rel_bf16=float(np.linalg.norm(y - y_16) / np.linalg.norm(y_16)),
                max_qat=None, max_bf16=float(np.abs(y - y_16).max() / np.abs(y_16).max()))


def _mx_rows(Q, torch, x_t, w_t, n, rows, y_16, meta, offsets=None, row_token=None,
             fractions=FRACTIONS):
    """Rows of the MX modes: x and w quantized to MX, the block-scaled GEMM
    (fp32 out), its distance to the bf16 product; then MX FP4 with RAC
    (quads_mx_rac_quantize, quads_moe_mx_rac_gemm) for every k > 0."""
    out = []
    e, _, kdim = w_t.shape
    for name, fmt in (("mxfp4", Q.MX_FP4), ("mxfp8", Q.MX_FP8)):
        a = Q.quads_mx_quantize(x_t, fmt)
        wc, wsc = Q.quads_mx_quantize(w_t.reshape(e * n, kdim), fmt)
        y = Q.quads_moe_mx_gemm(a, (wc.view(e, n, -1), wsc.view(e, n, -1)), n, rows=rows,
                                offsets=offsets, row_token=row_token, fmt=fmt,
                                out_dtype=Q.OUT_F32)
        torch.cuda.synchronize()
        out.append(dict(meta, format=name, frac=0.0, k=0,
                        **_mx_errors(y.cpu().numpy().astype(np.float64), y_16)))
    wc, wsc = Q.quads_mx_quantize(w_t.reshape(e * n, kdim), Q.MX_FP4)
    wq = (wc.view(e, n, -1), wsc.view(e, n, -1))
    for f in fractions:
        k = channels_for(f, kdim)
        if k == 0:
            continue
        a = Q.quads_mx_rac_quantize(x_t, k)
        y = Q.quads_moe_mx_rac_gemm((a["codes"], a["scales"]), (a["r_codes"], a["r_scales"]),
                                    a["sel"], wq, n, rows=rows, offsets=offsets,
                                    row_token=row_token, out_dtype=Q.OUT_F32)
        torch.cuda.synchronize()
        out.append(dict(meta, format="mxfp4+rac", frac=f, k=k,
                        **_mx_errors(y.cpu().numpy().astype(np.float64), y_16)))
    return out


def _gpu_gemm(Q, torch, x_t, k, wq, n, rows, offsets=None, row_token=None):
    a = Q.quads_rac_quantize(x_t, k)
    r = (a["r_nib"], a["r_scale"], a["r_ts"]) if k else None
    y = Q.quads_moe_w4a4_gemm((a["nib"], a["scale"], a["ts"]), wq, n, rows=rows, r=r,
                              sel=a["sel"] if k else None, offsets=offsets,
                              row_token=row_token, out_dtype=Q.OUT_F32)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


def sweep_dense(Q, torch, synth, dev, fractions=FRACTIONS, **overrides):
    """Rows of the sweep for the dense workload (synth config 2, sizes overridable)."""
    d = synth.make(2, **overrides)
    x, w = d["x"], d["w"]                         # bf16 bits [M, K], [1, N, K]
    m, kdim = x.shape
    n = w.shape[1]
    x_t = torch.from_numpy(x.view(np.int16)).to(dev)
    w_t = torch.from_numpy(w.view(np.int16)).to(dev)
    nib, scale, ts, dq = Q.quads_nvfp4_weight_qdq(w_t, want_dq=True)
    torch.cuda.synchronize()
    xf = _f64(x)
    y_qat = xf @ _f64(dq[0].cpu().numpy()).T
    y_16 = xf @ _f64(w[0]).T
    out = []
    for f in fractions:
        k = channels_for(f, kdim)
        y = _gpu_gemm(Q, torch, x_t, k, (nib, scale, ts), n, m)
        out.append(dict(workload="dense", M=m, K=kdim, N=n, format="nvfp4", frac=f, k=k,
                        **_errors(y, y_qat, y_16)))
    out += _mx_rows(Q, torch, x_t, w_t, n, m, y_16, dict(workload="dense", M=m, K=kdim, N=n),
                    fractions=fractions)
    return out


def sweep_moe(Q, torch, synth, dev, fractions=FRACTIONS, **overrides):
    """Rows of the sweep for the MoE gate/up GEMM (synth config 3, sizes overridable)."""
    d = synth.make(3, **overrides)
    x, ids, w13 = d["x"], d["topk_ids"], d["w13"]   # [T, H], [T, top_k], [E, 2I, H]
    t, kdim = x.shape
    e, n, _ = w13.shape
    x_t = torch.from_numpy(x.view(np.int16)).to(dev)
    ids_t = torch.from_numpy(ids).to(dev)
    w_t = torch.from_numpy(w13.view(np.int16)).to(dev)
    nib, scale, ts, dq = Q.quads_nvfp4_weight_qdq(w_t, want_dq=True)
    off_t, rt_t, _pos = Q.quads_moe_pack(ids_t, e)
    torch.cuda.synchronize()
    off = off_t.cpu().numpy()
    rt = rt_t.cpu().numpy()
    rows = int(off[-1])
    xf = _f64(x)
    y_qat = np.empty((rows, n))
    y_16 = np.empty((rows, n))
    for j in range(e):                             # packed rows of expert j
        sl = slice(off[j], off[j + 1])
        if off[j] == off[j + 1]:
            continue
        xa = xf[rt[sl]]
        y_qat[sl] = xa @ _f64(dq[j].cpu().numpy()).T
        y_16[sl] = xa @ _f64(w13[j]).T
    del dq
    out = []
    for f in fractions:
        k = channels_for(f, kdim)
        y = _gpu_gemm(Q, torch, x_t, k, (nib, scale, ts), n, rows, off_t, rt_t)
        out.append(dict(workload="moe_gate_up", T=t, E=e, K=kdim, N=n, rows=rows, format="nvfp4",
                        frac=f, k=k, **_errors(y, y_qat, y_16)))
    out += _mx_rows(Q, torch, x_t, w_t, n, rows, y_16,
                    dict(workload="moe_gate_up", T=t, E=e, K=kdim, N=n, rows=rows),
                    offsets=off_t, row_token=rt_t, fractions=fractions)
    return out


def table(rows):
    def f5(v):
        return "—" if v is None else f"{v:.5f}"
    lines = ["| workload | format | k / K | k | rel. Frobenius vs QAT ref. | rel. Frobenius vs bf16 | "
             "max element vs QAT ref. | max element vs bf16 |", "|---|---|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| {r['workload']} | {r.get('format', 'nvfp4')} | {100 * r['frac']:.1f} % | "
                     f"{r['k']} | {f5(r['rel_qat'])} | {f5(r['rel_bf16'])} | {f5(r['max_qat'])} | "
                     f"{f5(r.get('max_bf16'))} |")
    return "\n".join(lines)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--workloads", default="dense,moe")
    ap.add_argument("--tokens", type=int, default=0,
                    help="override the token count (0: the workloads' own)")
    args = ap.parse_args(argv)
    import torch

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    if root not in sys.path:
        sys.path.insert(0, root)
    import synth

    import nvfp4_w4a4_quantized_act_amd as Q
    Q.lib()
    dev = torch.device("cuda:0")
    rows = []
    for wl in args.workloads.split(","):
        if wl == "dense":
            kw = dict(m=args.tokens) if args.tokens else {}
            got = sweep_dense(Q, torch, synth, dev, **kw)
        elif wl == "moe":
            kw = dict(t=args.tokens) if args.tokens else {}
            got = sweep_moe(Q, torch, synth, dev, **kw)
        else:
            raise SystemExit(f"unknown workload {wl}")
        for r in got:
            print(json.dumps(r), flush=True)
        rows += got
    print(table(rows))


if __name__ == "__main__":
    main()
