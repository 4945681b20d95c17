#!/usr/bin/env python3
"""Benchmark of the QUADS rollout hot path on one MI355X.

Workload (the MoE expert FFN layer the GEMM target is quoted on): 128
experts, hidden 2048, expert intermediate 768, top-8 routing, 4096 tokens,
RAC with k = 64 channels at both GEMM inputs.  One step is one forward pass of
the layer through the library:

  quads_rac_quantize(hidden)            NVFP4 + RAC at the gate/up input
  quads_moe_pack(topk_ids)              token -> expert packing
  quads_moe_w4a4_gemm(gate/up, SwiGLU)  grouped W4A4 GEMM + compensation, bf16 h
  quads_rac_quantize(h)                 NVFP4 + RAC at the down input
  quads_moe_w4a4_gemm(down)             grouped W4A4 GEMM + compensation, bf16 out
  quads_moe_combine                     routing-weighted sum per token

The weight QDQ (quads_nvfp4_weight_qdq) runs once per weight refresh, not per
forward pass; it is timed on its own and reported as `weight_qdq_ms`.

Inputs are seeded synthetic tensors (synth.py) already resident in HBM when
the timed region starts.  `value` is the step's algorithmic GEMM work,
2 * rows * N * (K + k) summed over both GEMMs, divided by the step time.
`roofline` is for the dominant kernel, the gate/up GEMM: its algorithmic
flops per launch over its mean launch time (a pair of HIP events on the
launch stream around it in every timed step; an event record leaves the GPU
idle for a few microseconds, so the other per-op times in `ops` come from
extra steps after the timed region), against the dense fp16 MFMA peak (the GEMM's operands are exact fp16);
`traffic` is its HBM-side bytes per launch from the FETCH_SIZE / WRITE_SIZE
counter summary under profiles/ (null when that summary was taken on other
GEMM sources).  `cpu_baseline` times the NumPy oracle on a bounded sample of
the same layer.  `comparator` times the same gate/up GEMM as an MX
block-scaled GEMM with FP8 and with FP4 elements (quads_moe_mx_gemm), the
FP8 W8A8 baseline the paper's speed claim is measured against, next to the
W4A4+RAC GEMM.  `decode` runs the same layer at the decode step (64 tokens,
Zipf routing, most experts with 0-2 rows), where the GEMMs are bound by the
active experts' weight bytes.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]
"""

import argparse
import json
import os
import sys
import time

PEAK_FP16_TFLOPS = 2500.0        # MI355X dense fp16/bf16 MFMA
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E

ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "moe_ffn_e128_t4096_gemm_gate_up_traffic.md")
GEMM_SOURCES = [os.path.join(ROOT, "nvfp4_w4a4_quantized_act_amd", "csrc", f)
                for f in ("gemm.hip", "gemm_tiles.h", "common.h")]
GEMM_KERNEL_KEY = "k_gemm_w4a4_v2<1>"     # the gate/up (SwiGLU) GEMM kernel


def _parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=2048)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run a device copy of this size (for counter calibration)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU: turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of "
                         "`bench.py --copy-probe-mib N` into the traffic summary under profiles/")
    return ap.parse_args()


def _gemm_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _counter_per_dispatch(directory, counter):
    """{kernel name: [(grid size, value) per dispatch]} from a rocprofv3
    counter_collection.csv."""
    import csv
    import glob
    out = {}
    for f in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        per = {}
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                key = (r["Dispatch_Id"], r["Kernel_Name"], int(r["Grid_Size"]))
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
        for (_, name, grid), v in per.items():
            out.setdefault(name, []).append((grid, v))
    return out


def traffic_summary(fetch_dir, write_dir, copy_mib):
    """HBM-side bytes per launch of the gate/up GEMM: FETCH_SIZE and WRITE_SIZE
    (KiB per dispatch), each scaled by bytes / counter of a plain device copy of
    copy_mib MiB (which reads and writes copy_mib MiB)."""
    fetch = _counter_per_dispatch(fetch_dir, "FETCH_SIZE")
    write = _counter_per_dispatch(write_dir, "WRITE_SIZE")

    def pick(d, key):
        # the prefill layer's launches: the largest grid of that kernel (the
        # decode layer launches the same kernel on a small grid)
        vals = [gv for n, vs in d.items() if key in n for gv in vs]
        if not vals:
            raise SystemExit(f"no dispatch of a kernel matching {key!r}")
        big = max(g for g, _ in vals)
        return [v for g, v in vals if g == big]

    def copy_val(d):
        vals = [v for n, vs in d.items() if "copy" in n.lower() for _, v in vs]
        if not vals:
            raise SystemExit("no copy kernel dispatch found (run with --copy-probe-mib)")
        return max(vals)

    g_f = sum(pick(fetch, GEMM_KERNEL_KEY)) / len(pick(fetch, GEMM_KERNEL_KEY))
    g_w = sum(pick(write, GEMM_KERNEL_KEY)) / len(pick(write, GEMM_KERNEL_KEY))
    c_f, c_w = copy_val(fetch), copy_val(write)
    copy_bytes = copy_mib * (1 << 20)
    f_scale, w_scale = copy_bytes / c_f, copy_bytes / c_w
    traffic = g_f * f_scale + g_w * w_scale
    lines = [
        "# HBM traffic of the gate/up GEMM: MoE FFN, 128 experts, T=4096, hidden 2048, "
        "intermediate 768, top-8, RAC k=64",
        "",
        "Commands (repository root, one MI355X), then this summary on any host:",
        "",
        "```",
        f"cd /tmp && export TMPDIR=/tmp && timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE "
        f"--output-format csv -d $REPO/gpurun_out/pmc_fetch -o f -- python -u $REPO/bench.py "
        f"--steps 2 --warmup 1 --no-cpu-baseline --copy-probe-mib {copy_mib}",
        f"cd /tmp && export TMPDIR=/tmp && timeout -s KILL 120 rocprofv3 --pmc WRITE_SIZE "
        f"--output-format csv -d $REPO/gpurun_out/pmc_write -o w -- python -u $REPO/bench.py "
        f"--steps 2 --warmup 1 --no-cpu-baseline --copy-probe-mib {copy_mib}",
        f"python bench.py --traffic-from gpurun_out/pmc_fetch gpurun_out/pmc_write "
        f"--copy-probe-mib {copy_mib}",
        "```",
        "",
        "| quantity | value |",
        "|---|---|",
        f"| GEMM FETCH_SIZE per dispatch (KiB) | {g_f:.1f} |",
        f"| GEMM WRITE_SIZE per dispatch (KiB) | {g_w:.1f} |",
        f"| copy of {copy_mib} MiB: FETCH_SIZE (KiB) | {c_f:.1f} |",
        f"| copy of {copy_mib} MiB: WRITE_SIZE (KiB) | {c_w:.1f} |",
        f"| scale, read bytes per FETCH_SIZE unit | {f_scale:.2f} |",
        f"| scale, written bytes per WRITE_SIZE unit | {w_scale:.2f} |",
        f"| GEMM read bytes per launch | {g_f * f_scale:.0f} |",
        f"| GEMM written bytes per launch | {g_w * w_scale:.0f} |",
        "",
        f"traffic_bytes_per_launch: {traffic:.0f}",
        f"gemm_source_sha256: {_gemm_source_hash()}",
        "",
    ]
    with open(TRAFFIC_FILE, "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))


def measured_traffic():
    """Traffic bytes per launch from the committed counter summary, or None when
    it is missing or was taken on a different GEMM source."""
    try:
        with open(TRAFFIC_FILE) as fh:
            text = fh.read()
    except OSError:
        return None
    vals = dict(l.split(": ", 1) for l in text.splitlines() if l.startswith(
        ("traffic_bytes_per_launch: ", "gemm_source_sha256: ")))
    if vals.get("gemm_source_sha256") != _gemm_source_hash():
        return None
    return float(vals["traffic_bytes_per_launch"])


def main():
    args = _parse()
    if args.traffic_from:
        traffic_summary(args.traffic_from[0], args.traffic_from[1], args.copy_probe_mib or 512)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build measures one GPU only; multi-GPU runs are not "
                                   "part of it", "n_gpus": args.gpus}))
        sys.exit(2)
    cores = len(os.sched_getaffinity(0))
    os.environ.setdefault("OPENBLAS_NUM_THREADS", str(cores))
    import numpy as np
    import torch

    import nvfp4_w4a4_quantized_act_amd as Q
    import synth

    cfg = synth.CONFIGS[3]
    T, E, H, I, TOPK, KR = cfg["t"], cfg["e"], cfg["h"], cfg["i"], cfg["topk"], cfg["rac_k"]
    rows = T * TOPK
    dev = torch.device("cuda:0")
    Q.lib()

    data = synth.make(3)

    def up(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)

    x = up(data["x"])
    ids = up(data["topk_ids"])
    tw = up(data["topk_w"])
    w13 = up(data["w13"])
    w2 = up(data["w2"])
    del data["w13"], data["w2"]

    # weight QDQ, once per refresh (timed on its own)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    w13q = Q.quads_nvfp4_weight_qdq(w13)[:3]
    w2q = Q.quads_nvfp4_weight_qdq(w2)[:3]
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(3):
        w13q = Q.quads_nvfp4_weight_qdq(w13)[:3]
        w2q = Q.quads_nvfp4_weight_qdq(w2)[:3]
    ev[1].record()
    torch.cuda.synchronize()
    weight_qdq_ms = ev[0].elapsed_time(ev[1]) / 3
    # the MX comparator's weights (FP8 and FP4 elements, E8M0 per 32), quantized
    # once like the NVFP4 ones
    w13_2d = w13.view(E * 2 * I, H)
    w13_mx = {}
    for fmt_name, fmt in (("mxfp8", Q.MX_FP8), ("mxfp4", Q.MX_FP4)):
        c, sc = Q.quads_mx_quantize(w13_2d, fmt)
        w13_mx[fmt_name] = (c.view(E, 2 * I, -1), sc.view(E, 2 * I, -1), fmt)
    del w13, w2, w13_2d

    # Each event record costs the GPU a few microseconds of idle time, so the
    # timed steps bracket only the gate/up GEMM (the roofline kernel); the
    # per-op breakdown comes from extra steps after the timed region.
    nev = 7
    timers, gemm_timers = [], []

    def step(mode):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(nev)] if mode else None

        def mark(i):
            if mode == "all" or (mode == "gemm" and i in (2, 3)):
                evs[i].record()
        mark(0)
        a = Q.quads_rac_quantize(x, KR)
        mark(1)
        off, rt, pos = Q.quads_moe_pack(ids, E)
        mark(2)
        h = Q.quads_moe_w4a4_gemm((a["nib"], a["scale"], a["ts"]), w13q, 2 * I, rows=rows,
                                  r=(a["r_nib"], a["r_scale"], a["r_ts"]), sel=a["sel"],
                                  offsets=off, row_token=rt, epilogue=Q.EPI_SWIGLU,
                                  out_dtype=Q.OUT_BF16)
        mark(3)
        b = Q.quads_rac_quantize(h, KR)
        mark(4)
        y2 = Q.quads_moe_w4a4_gemm((b["nib"], b["scale"], b["ts"]), w2q, H, rows=rows,
                                   r=(b["r_nib"], b["r_scale"], b["r_ts"]), sel=b["sel"],
                                   offsets=off, out_dtype=Q.OUT_BF16)
        mark(5)
        out = Q.quads_moe_combine(y2, pos, tw, y_dtype=Q.OUT_BF16)
        mark(6)
        if mode == "all":
            timers.append(evs)
        elif mode == "gemm":
            gemm_timers.append(evs)
        return out

    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step("gemm")
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    for _ in range(max(3, min(args.steps, 10))):
        step("all")
    torch.cuda.synchronize()

    names = ["rac_gate_up", "pack", "gemm_gate_up_swiglu", "rac_down", "gemm_down", "combine"]
    per_op = {n: 0.0 for n in names}
    for evs in timers:
        for i, n in enumerate(names):
            per_op[n] += evs[i].elapsed_time(evs[i + 1]) / len(timers)
    # the roofline kernel's duration: events of the timed steps
    per_op["gemm_gate_up_swiglu"] = sum(e[2].elapsed_time(e[3]) for e in gemm_timers) / len(
        gemm_timers)

    fl_gu = 2.0 * rows * (2 * I) * (H + KR)
    fl_dn = 2.0 * rows * H * (I + KR)
    value = (fl_gu + fl_dn) / (ms_per_step * 1e-3) / 1e12
    gu_tflops = fl_gu / (per_op["gemm_gate_up_swiglu"] * 1e-3) / 1e12
    dn_tflops = fl_dn / (per_op["gemm_down"] * 1e-3) / 1e12
    q_bytes_gu = 2.5625 * T * H + 0.5625 * T * KR
    q_bytes_dn = 2.5625 * rows * I + 0.5625 * rows * KR
    ops = {
        "rac_gate_up": {"ms": per_op["rac_gate_up"],
                        "GB/s": q_bytes_gu / (per_op["rac_gate_up"] * 1e-3) / 1e9},
        "rac_down": {"ms": per_op["rac_down"],
                     "GB/s": q_bytes_dn / (per_op["rac_down"] * 1e-3) / 1e9},
        "pack": {"ms": per_op["pack"]},
        "gemm_gate_up_swiglu": {"ms": per_op["gemm_gate_up_swiglu"], "TFLOP/s": gu_tflops},
        "gemm_down": {"ms": per_op["gemm_down"], "TFLOP/s": dn_tflops},
        "combine": {"ms": per_op["combine"]},
    }
    for k in ("rac_gate_up", "rac_down"):
        ops[k]["hbm_frac"] = ops[k]["GB/s"] / PEAK_HBM_GBS

    quant = quantizer_rate(np, torch, Q, synth, dev)
    decode = decode_layer(np, torch, Q, synth, dev, w13q, w2q)
    comparator = mx_comparator(torch, Q, x, ids, E, I, rows, w13_mx,
                               per_op["gemm_gate_up_swiglu"], fl_gu)
    per_expert = per_expert_down(torch, Q, x, ids, E, I, H, KR, rows, w13q, w2q)

    if args.copy_probe_mib:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(np, torch, data, w13q, w2q, cfg, args.cpu_sample_tokens, cores)

    line = {
        "metric": "MoE W4A4+RAC grouped-GEMM TFLOP/s & quantizer GB/s, % of MI355X roofline",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": "moe_ffn_e128_h2048_i768_top8_t4096_rac64",
                   "tokens": T, "experts": E, "hidden": H, "intermediate": I, "top_k": TOPK,
                   "rac_k": KR, "packed_rows": rows, "gemm_operands": "nvfp4 -> exact fp16",
                   "accumulate": "fp32", "parallelism": "single_gpu"},
        "roofline": {"bound": "mfma", "kernel": "v2::k_gemm_w4a4_v2<1> (gate/up GEMM, SwiGLU epilogue)",
                     "achieved": gu_tflops, "peak": PEAK_FP16_TFLOPS, "unit": "TFLOP/s",
                     "frac": gu_tflops / PEAK_FP16_TFLOPS, "traffic": measured_traffic()},
        "cpu_baseline": cpu,
        "ops": ops,
        "quantizer": quant,
        "comparator": comparator,
        "decode": decode,
        "per_expert_selection": per_expert,
        "weight_qdq_ms": weight_qdq_ms,
    }
    print(json.dumps(line), flush=True)


def per_expert_down(torch, Q, x, ids, E, I, H, KR, rows, w13q, w2q, reps=20):
    """The variant with one channel selection per expert, at the layer's down
    site (the packed [32768, 768] SwiGLU output, 128 experts, k = 64): RAC
    and the down GEMM with per-expert compensation, each timed over `reps`
    back-to-back calls beside the shared-selection calls on the same input."""
    a = Q.quads_rac_quantize(x, KR)
    off, rt, pos = Q.quads_moe_pack(ids, E)
    h = Q.quads_moe_w4a4_gemm((a["nib"], a["scale"], a["ts"]), w13q, 2 * I, rows=rows,
                              r=(a["r_nib"], a["r_scale"], a["r_ts"]), sel=a["sel"], offsets=off,
                              row_token=rt, epilogue=Q.EPI_SWIGLU, out_dtype=Q.OUT_BF16)
    keep = {}

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(reps):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / reps

    def rac_shared():
        keep["b"] = Q.quads_rac_quantize(h, KR)

    def rac_experts():
        keep["be"] = Q.quads_rac_quantize_experts(h, KR, off)

    ms = {"rac_shared_ms": timed(rac_shared), "rac_per_expert_ms": timed(rac_experts)}
    b, be = keep["b"], keep["be"]
    ms["gemm_down_shared_ms"] = timed(lambda: Q.quads_moe_w4a4_gemm(
        (b["nib"], b["scale"], b["ts"]), w2q, H, rows=rows,
        r=(b["r_nib"], b["r_scale"], b["r_ts"]), sel=b["sel"], offsets=off,
        out_dtype=Q.OUT_BF16))
    ms["gemm_down_per_expert_ms"] = timed(lambda: Q.quads_moe_w4a4_gemm_sel_experts(
        (be["nib"], be["scale"], be["ts"]), w2q, H, r=(be["r_nib"], be["r_scale"], be["r_ts"]),
        sel=be["sel"], offsets=off, out_dtype=Q.OUT_BF16))
    ms["site"] = "down projection input: 32768 packed rows x 768, 128 experts, k = 64"
    return ms


def quantizer_rate(np, torch, Q, synth, dev, reps=20):
    """quads_nvfp4_quantize on the large-prefill gate/up input (16384 x 4096
    bf16, Student-t body with outlier channels): algorithmic bytes (2 read +
    0.5625 written per element) per call, with the dynamic tensor scale (a max
    pass, then the quantize pass) and with a given tensor scale (one pass).
    Calls go straight to the C ABI with buffers allocated once, so the rate is
    the device's; a device-to-device copy of the same input is timed alongside
    as context (it moves 4 bytes per element)."""
    import ctypes
    lib = Q.lib()
    d = synth.make(5, with_weights=False)
    x = torch.from_numpy(d["x"].view(np.int16)).to(dev)
    m, k = x.shape
    nbytes = 2.5625 * m * k
    nib = torch.empty((m, k // 2), dtype=torch.uint8, device=dev)
    sc = torch.empty((m, k // 16), dtype=torch.uint8, device=dev)
    ts = torch.empty(4, dtype=torch.float32, device=dev)
    ts_given = torch.empty(4, dtype=torch.float32, device=dev)
    nws = lib.quads_nvfp4_quantize_ws(m, k)
    ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)

    def P(t):
        return ctypes.c_void_p(t.data_ptr())

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    def call(ts_in):
        st = lib.quads_nvfp4_quantize(P(x), m, k, ts_in, P(nib), P(sc), P(ts), P(ws), nws, stream)
        if st != 0:
            raise RuntimeError(f"quads_nvfp4_quantize failed with status {st}")

    call(None)
    ts_given.copy_(ts)
    out = {"shape": [m, k], "algorithmic_bytes": nbytes}
    for name, ts_in in (("dynamic_scale", None), ("given_scale", P(ts_given))):
        us = timed(lambda: call(ts_in))
        gbs = nbytes / (us * 1e-6) / 1e9
        out[name] = {"us": us, "GB/s": gbs, "hbm_frac": gbs / PEAK_HBM_GBS}
    y = torch.empty_like(x)
    us = timed(lambda: y.copy_(x))
    out["device_copy"] = {"us": us, "GB/s": 4.0 * m * k / (us * 1e-6) / 1e9,
                          "hbm_frac": 4.0 * m * k / (us * 1e-6) / 1e9 / PEAK_HBM_GBS}
    return out


def decode_layer(np, torch, Q, synth, dev, w13q, w2q, reps=50):
    """The decode-step layer (64 tokens, Zipf(1.2) routing over the same 128
    experts, hidden 2048, intermediate 768, top-8, RAC k = 64 at both GEMM
    inputs): the same six library calls as the prefill step, here in the
    few-rows-per-expert regime (512 packed rows, most experts with 0-2 rows).
    The weights are the prefill layer's NVFP4 weights (same shapes and
    distribution).  Reported: the layer time (back-to-back layers, no events
    inside), the per-op times from a separate pass with events, and the two
    GEMMs' rates as the bytes of the active experts' NVFP4 weights (0.5625 B
    per weight) per second against the 8 TB/s HBM peak."""
    d = synth.make(4, with_weights=False)
    x = torch.from_numpy(d["x"].view(np.int16)).to(dev)
    ids = torch.from_numpy(d["topk_ids"]).to(dev)
    tw = torch.from_numpy(d["topk_w"]).to(dev)
    T, TOPK, KR = x.shape[0], ids.shape[1], d["rac_k"]
    E, N13, H = w13q[0].shape[0], w13q[0].shape[1], w13q[0].shape[2] * 2
    I = N13 // 2
    rows = T * TOPK
    keep = {}

    def layer(evs=None):
        def mark(i):
            if evs is not None:
                evs[i].record()
        mark(0)
        a = Q.quads_rac_quantize(x, KR)
        mark(1)
        off, rt, pos = Q.quads_moe_pack(ids, E)
        mark(2)
        h = Q.quads_moe_w4a4_gemm((a["nib"], a["scale"], a["ts"]), w13q, N13, rows=rows,
                                  r=(a["r_nib"], a["r_scale"], a["r_ts"]), sel=a["sel"],
                                  offsets=off, row_token=rt, epilogue=Q.EPI_SWIGLU,
                                  out_dtype=Q.OUT_BF16)
        mark(3)
        b = Q.quads_rac_quantize(h, KR)
        mark(4)
        y2 = Q.quads_moe_w4a4_gemm((b["nib"], b["scale"], b["ts"]), w2q, H, rows=rows,
                                   r=(b["r_nib"], b["r_scale"], b["r_ts"]), sel=b["sel"],
                                   offsets=off, out_dtype=Q.OUT_BF16)
        mark(5)
        out = Q.quads_moe_combine(y2, pos, tw, y_dtype=Q.OUT_BF16)
        mark(6)
        keep.update(a=a, b=b, off=off, rt=rt)
        return out

    for _ in range(5):
        layer()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        layer()
    torch.cuda.synchronize()
    layer_ms = (time.perf_counter() - t0) * 1e3 / reps
    names = ["rac_gate_up", "pack", "gemm_gate_up_swiglu", "rac_down", "gemm_down", "combine"]
    per_op = np.zeros(len(names))
    n_ev = 10
    for _ in range(n_ev):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(7)]
        layer(evs)
        torch.cuda.synchronize()
        per_op += [evs[i].elapsed_time(evs[i + 1]) for i in range(len(names))]
    per_op /= n_ev
    a, b, off, rt = keep["a"], keep["b"], keep["off"], keep["rt"]
    counts = np.diff(off.cpu().numpy())
    active = int((counts > 0).sum())
    wb_gu = 0.5625 * active * N13 * H
    wb_dn = 0.5625 * active * H * I
    ops = {n: {"ms": float(v)} for n, v in zip(names, per_op)}
    # each GEMM alone, back to back on the last layer's inputs (no event
    # between launches): its rate on the active experts' weight bytes
    gemms = {
        "gemm_gate_up_swiglu": (wb_gu, lambda: Q.quads_moe_w4a4_gemm(
            (a["nib"], a["scale"], a["ts"]), w13q, N13, rows=rows,
            r=(a["r_nib"], a["r_scale"], a["r_ts"]), sel=a["sel"], offsets=off, row_token=rt,
            epilogue=Q.EPI_SWIGLU, out_dtype=Q.OUT_BF16)),
        "gemm_down": (wb_dn, lambda: Q.quads_moe_w4a4_gemm(
            (b["nib"], b["scale"], b["ts"]), w2q, H, rows=rows,
            r=(b["r_nib"], b["r_scale"], b["r_ts"]), sel=b["sel"], offsets=off,
            out_dtype=Q.OUT_BF16)),
    }
    for n, (wb, fn) in gemms.items():
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(20):
            fn()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / 20
        gbs = wb / (us * 1e-6) / 1e9
        ops[n].update({"alone_us": us, "weight_bytes": wb, "GB/s": gbs,
                       "hbm_frac": gbs / PEAK_HBM_GBS})
    return {"workload": "moe_decode_e128_h2048_i768_top8_t64_zipf1.2_rac64", "tokens": T,
            "packed_rows": rows, "active_experts": active,
            "max_rows_per_expert": int(counts.max()), "layer_ms": layer_ms,
            "tokens_per_s": T / (layer_ms * 1e-3), "ops": ops,
            "note": "per-op ms carry an event record each (a few microseconds of idle GPU); "
                    "layer_ms has none; the GEMM rates use alone_us (20 back-to-back calls)"}


def mx_comparator(torch, Q, x, ids, E, I, rows, w13_mx, w4a4_ms, w4a4_flops, reps=20):
    """The gate/up GEMM of the same layer (same tokens, routing and SwiGLU bf16
    output) as an MX block-scaled GEMM (quads_moe_mx_gemm): FP8 E4M3 elements,
    the FP8 W8A8 baseline of the paper's speed claim, and FP4 E2M1 elements
    (power-of-two scales per 32: not NVFP4).  Activations are MX-quantized
    from the same bf16 x; timed with events over `reps` launches.  Reported
    beside the W4A4+RAC gate/up GEMM of the timed steps."""
    off, rt, _ = Q.quads_moe_pack(ids, E)
    out = {"workload": "gate/up GEMM, 32768 packed rows x 1536 x 2048, SwiGLU bf16 out",
           "w4a4_rac": {"us": w4a4_ms * 1e3,
                        "TFLOP/s": w4a4_flops / (w4a4_ms * 1e-3) / 1e12}}
    for name, (wc, wsc, fmt) in w13_mx.items():
        ac, asc = Q.quads_mx_quantize(x, fmt)

        def run():
            return Q.quads_moe_mx_gemm((ac, asc), (wc, wsc), 2 * I, rows=rows, offsets=off,
                                       row_token=rt, fmt=fmt, epilogue=Q.EPI_SWIGLU,
                                       out_dtype=Q.OUT_BF16)
        run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            run()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        flops = 2.0 * rows * (2 * I) * x.shape[1]
        out[name] = {"us": us, "TFLOP/s": flops / (us * 1e-6) / 1e12,
                     "w4a4_rac_time_ratio": w4a4_ms * 1e3 / us}
    return out


def cpu_baseline(np, torch, data, w13q, w2q, cfg, t_sample, cores):
    """The oracle, as it stands, on the first t_sample tokens of the same layer
    (weights: the GPU's packed NVFP4 weights, bit-identical to the oracle's
    weight QDQ).  Returns algorithmic GEMM TFLOP/s of the sample."""
    from oracle import formats as OF
    from oracle import moe as OM
    from oracle import rac as OR
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = cores
    E, H, I, TOPK, KR = cfg["e"], cfg["h"], cfg["i"], cfg["topk"], cfg["rac_k"]
    w13 = tuple(t.cpu().numpy() for t in w13q)
    w2 = tuple(t.cpu().numpy() for t in w2q)
    x = data["x"][:t_sample]
    ids = data["topk_ids"][:t_sample]
    tw = data["topk_w"][:t_sample]
    rows = t_sample * TOPK
    t0 = time.perf_counter()
    a = OR.rac_quantize(OF.bf16_to_f64(x), KR)
    off, rt, pos = OM.pack_routes(ids, E)
    y1, _ = OM.grouped_gemm((a["nib"], a["scale"], a["ts"]), (a["r_nib"], a["r_scale"], a["r_ts"]),
                            a["sel"], w13, off, rt, want_bound=False)
    h = OM.swiglu(y1)
    b = OR.rac_quantize(OF.bf16_to_f64(h), KR)
    y2, _ = OM.grouped_gemm((b["nib"], b["scale"], b["ts"]), (b["r_nib"], b["r_scale"], b["r_ts"]),
                            b["sel"], w2, off, None, want_bound=False)
    OM.combine(y2, pos, tw, t_sample, TOPK)
    dt = time.perf_counter() - t0
    flops = 2.0 * rows * (2 * I) * (H + KR) + 2.0 * rows * H * (I + KR)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"first {t_sample} of 4096 tokens ({rows} packed rows), full layer "
                      f"forward through the fp64 NumPy oracle, {dt:.1f} s"}


if __name__ == "__main__":
    main()
