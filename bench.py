#!/usr/bin/env python3
"""Benchmark of the QUADS rollout hot path on one MI355X.

Workload (the MoE expert FFN layer the GEMM target is quoted on): 128
experts, hidden 2048, expert intermediate 768, top-8 routing, 4096 tokens,
RAC with k = 64 channels at both GEMM inputs.  One step is one forward pass of
the layer through the library:

  quads_rac_quantize(hidden)            NVFP4 + RAC at the gate/up input
  quads_moe_pack(topk_ids)              token -> expert packing
  quads_moe_w4a4_gemm_amax(gate/up)     grouped W4A4 GEMM + compensation, SwiGLU bf16 h,
                                        and per-work-group maxima of |h|
  quads_rac_quantize_partials(h)        NVFP4 + RAC at the down input, max|h| from those
                                        maxima (no max pass over h)
  quads_moe_w4a4_gemm(down)             grouped W4A4 GEMM + compensation, bf16 out
  quads_moe_combine                     routing-weighted sum per token

The weight QDQ (quads_nvfp4_weight_qdq) runs once per weight refresh, not per
forward pass; it is timed on its own and reported as `weight_qdq_ms`.

Inputs are seeded synthetic tensors (synth.py) already resident in HBM when
the timed region starts.  `value` is the step's algorithmic GEMM work,
2 * rows * N * (K + k) summed over both GEMMs, divided by the step time of
back-to-back steps.  `roofline` is for the dominant kernel, the gate/up GEMM:
its algorithmic flops per launch over its mean launch time (a pair of HIP
events on the launch stream around it in every timed step; an event record
leaves the GPU idle for a few microseconds, so the other per-op times in
`ops` come from extra steps after the timed region), against the dense fp16
MFMA peak (the GEMM's operands are exact fp16); `traffic` is its HBM-side
bytes per launch from the FETCH_SIZE / WRITE_SIZE counter summary under
profiles/ (null when that summary was taken on other GEMM sources).

Cold figures (`cold`): before each timed call or step a 512 MiB buffer is
written, which evicts the 256 MB last-level cache and the L2s, and an event
pair brackets the call (median and min over the reps).  The quantizer's cold
rate instead cycles through copies of its input spaced at least 512 MiB
apart, back to back, so no event gap enters its 20-50 us calls.

Other workloads: `config2` (dense 4096 x 4096 x 4096 linear, k = 128),
`config5` (64 experts, hidden 4096, intermediate 1536, 16384 tokens: the
gate/up RAC and GEMM at k = 0, 64, 256 and 2048 = 50% of the channels, and
the quantizer on the down-site input, the 131072 x 1536 SwiGLU output),
`rac_overhead` (the step with plain NVFP4 at both sites, k = 0, beside the
RAC step), `decode` (the same layer at the decode step: 64 tokens, Zipf
routing), `comparator` (the gate/up GEMM as MXFP8 and MXFP4),
`per_expert_selection`, and `cpu_baseline` (the NumPy oracle on a bounded
sample of the layer).

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--layer-only]
    python bench.py --traffic-from FETCH_DIR WRITE_DIR --copy-probe-mib N
    python bench.py --trace-from TRACE_DIR
    python bench.py --pmc-from DIR [DIR ...]
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
TRACE_FILE = os.path.join(ROOT, "profiles", "moe_ffn_e128_t4096_kernel_trace.md")
PMC_FILE = os.path.join(ROOT, "profiles", "moe_ffn_e128_t4096_counters.md")
GEMM_SOURCES = [os.path.join(ROOT, "nvfp4_w4a4_quantized_act_amd", "csrc", f)
                for f in ("gemm.hip", "gemm_v3.hip", "gemm_decode.hip", "gemm_tiles.h", "common.h")]
# the gate/up (SwiGLU) GEMM call: the tiled kernel, and the decode kernel that
# takes the rows past 256 of experts of 257 .. 320 rows
GEMM_KERNEL_KEYS = ("k_gemm_w4a4_v3<1, false>", "k_gemm_w4a4_decode<1,")
FLUSH_BYTES = 512 << 20


def _parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=2048)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run a device copy of this size (for counter calibration)")
    ap.add_argument("--layer-only", action="store_true",
                    help="only the prefill layer's steps (for counter runs)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU: turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of "
                         "`bench.py --copy-probe-mib N` into the traffic summary under profiles/")
    ap.add_argument("--trace-from", metavar="TRACE_DIR",
                    help="no GPU: turn a rocprofv3 --kernel-trace run of bench.py into the "
                         "per-kernel, per-launch-shape summary under profiles/")
    ap.add_argument("--pmc-from", nargs="+", metavar="DIR",
                    help="no GPU: turn rocprofv3 --pmc runs of `bench.py --layer-only` into "
                         "the counter summary under profiles/")
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

    # per launch of the call: the mean per dispatch of each of its kernels, summed
    g_f = sum(sum(pick(fetch, key)) / len(pick(fetch, key)) for key in GEMM_KERNEL_KEYS)
    g_w = sum(sum(pick(write, key)) / len(pick(write, key)) for key in GEMM_KERNEL_KEYS)
    c_f, c_w = copy_val(fetch), copy_val(write)
    copy_bytes = copy_mib * (1 << 20)
    f_scale, w_scale = copy_bytes / c_f, copy_bytes / c_w
    traffic = g_f * f_scale + g_w * w_scale
    lines = [
        "# HBM traffic of the gate/up GEMM: MoE FFN, 128 experts, T=4096, hidden 2048, "
        "intermediate 768, top-8, RAC k=64",
        "",
        "The call is two launches: the tiled kernel `v3::k_gemm_w4a4_v3<1, false>` and the decode "
        "kernel `dec::k_gemm_w4a4_decode<1, 2, true, true>` for the rows past 256 of experts of 257 .. "
        "320 rows; the figures below add the two kernels' per-dispatch means.",
        "",
        "Commands (repository root, one MI355X), then this summary on any host:",
        "",
        "```",
        f"cd /tmp && export TMPDIR=/tmp && timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE "
        f"--output-format csv -d $REPO/gpurun_out/pmc_fetch -o f -- python -u $REPO/bench.py "
        f"--steps 2 --warmup 1 --no-cpu-baseline --layer-only --copy-probe-mib {copy_mib}",
        f"cd /tmp && export TMPDIR=/tmp && timeout -s KILL 120 rocprofv3 --pmc WRITE_SIZE "
        f"--output-format csv -d $REPO/gpurun_out/pmc_write -o w -- python -u $REPO/bench.py "
        f"--steps 2 --warmup 1 --no-cpu-baseline --layer-only --copy-probe-mib {copy_mib}",
        f"python bench.py --traffic-from gpurun_out/pmc_fetch gpurun_out/pmc_write "
        f"--copy-probe-mib {copy_mib}",
        "```",
        "",
        "| quantity | value |",
        "|---|---|",
        f"| GEMM FETCH_SIZE per call (KiB) | {g_f:.1f} |",
        f"| GEMM WRITE_SIZE per call (KiB) | {g_w:.1f} |",
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


def _short_name(name):
    """Kernel name without the return type, the library namespace and the
    argument list: `v3::k_gemm_w4a4_v3<1>`."""
    name = name.strip().replace("(anonymous namespace)::", "")
    if name.startswith("void "):
        name = name[5:]
    depth = 0
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            name = name[:i]
            break
    return name.replace("quads::", "")


def trace_summary(trace_dir):
    """Per kernel and launch shape (work-groups in x and y, threads per
    work-group): calls and start-to-end durations from a rocprofv3
    --kernel-trace run of the default benchmark."""
    import csv
    import glob
    groups = {}
    for f in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                wx, wy = int(r["Workgroup_Size_X"]), int(r["Workgroup_Size_Y"])
                wz = int(r["Workgroup_Size_Z"])
                key = (_short_name(r["Kernel_Name"]), int(r["Grid_Size_X"]) // wx,
                       int(r["Grid_Size_Y"]) // wy, wx * wy * wz)
                dt = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3
                groups.setdefault(key, []).append(dt)
    if not groups:
        raise SystemExit(f"no kernel_trace.csv under {trace_dir}")
    total = sum(sum(v) for v in groups.values())
    rows = sorted(groups.items(), key=lambda kv: -sum(kv[1]))
    lines = [
        "# Kernel trace: MoE FFN layer, 128 experts, T=4096, hidden 2048, intermediate 768, "
        "top-8, RAC k=64, with the benchmark's other workloads",
        "",
        "Commands (repository root, one MI355X; `$REPO` is the repository root), then this "
        "summary on any host:",
        "",
        "```",
        "cd /tmp && export TMPDIR=/tmp && timeout -k 10 900 rocprofv3 --kernel-trace --stats "
        "--output-format csv -d $REPO/gpurun_out/prof_trace -o bench -- python -u "
        "$REPO/bench.py --steps 10 --warmup 3 --no-cpu-baseline",
        "python bench.py --trace-from gpurun_out/prof_trace",
        "```",
        "",
        "Durations are the trace's start-to-end times in microseconds, grouped by kernel and "
        "launch shape (work-groups in x and y, threads per work-group), so that launches of one "
        "kernel on different workloads show apart.  The prefill layer's gate/up GEMM is "
        "`v3::k_gemm_w4a4_v3<1, false>` at (3072, 1) x 512 plus "
        "`dec::k_gemm_w4a4_decode<1, 2, true, true>` at (1536, 1) x 128 for the rows past 256 of "
        "experts of 257 .. 320 rows; config 5's gate/up GEMMs are the tiled kernel at (13824, 1) "
        "x 512 (`<1, true>`: k = 2048, with the gathered compensation); the decode layer's "
        "GEMMs are the decode kernel at (1632, 1) and (2176, 1).  The down GEMM (768 + 64 "
        "channels, one accumulator chain) is `v2::k_gemm_w4a4_v2<0>`; config 2's GEMM is "
        "`v3::k_gemm_w4a4_v3<0, false>` at (512, 1).",
        "",
        "| kernel | work-groups (x, y) x threads | calls | total (us) | average (us) | min (us) | "
        "max (us) | % |",
        "|---|---|---|---|---|---|---|---|",
    ]
    for (name, gx, gy, th), v in rows[:60]:
        lines.append(f"| `{name}` | ({gx}, {gy}) x {th} | {len(v)} | {sum(v):.1f} | "
                     f"{sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f} | "
                     f"{100 * sum(v) / total:.1f} |")
    if len(rows) > 60:
        lines.append(f"| ({len(rows) - 60} more groups) | | | "
                     f"{sum(sum(v) for _, v in rows[60:]):.1f} | | | | |")
    lines += ["", f"gemm_source_sha256: {_gemm_source_hash()}", ""]
    with open(TRACE_FILE, "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))


PMC_PASSES = (
    "SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_F16 SQ_INSTS_VALU "
    "SQ_INSTS_MFMA SQ_VALU_MFMA_COEXEC_CYCLES SQ_WAVE_CYCLES SQ_WAIT_INST_ANY GRBM_GUI_ACTIVE",
    "SQ_INSTS_LDS SQ_ACTIVE_INST_LDS SQ_LDS_BANK_CONFLICT SQ_INSTS_VMEM_RD SQ_INSTS_VMEM_WR "
    "SQ_ACTIVE_INST_VALU SQ_WAIT_ANY SQ_INST_LEVEL_VMEM GRBM_GUI_ACTIVE",
)


def pmc_summary(dirs):
    """Per-dispatch counter means for the layer's kernels from rocprofv3 --pmc
    runs of `bench.py --layer-only`, with the derived MFMA-busy fraction and
    LDS conflict rate."""
    import csv
    import glob
    per = {}
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    key = (_short_name(r["Kernel_Name"]), int(r["Grid_Size"]))
                    disp = (f, r["Dispatch_Id"])
                    c = per.setdefault(key, {}).setdefault(r["Counter_Name"], {})
                    c[disp] = c.get(disp, 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit("no counter_collection.csv found")
    n_xcd, n_simd = 8, 1024
    lines = [
        "# Hardware counters: MoE FFN layer (128 experts, T=4096, hidden 2048, intermediate 768, "
        "top-8, RAC k=64) and the quantizer on a [16384, 4096] input",
        "",
        "Commands (repository root, one MI355X; `$REPO` is the repository root), one run per "
        "counter pass, then this summary on any host:",
        "",
        "```",
    ]
    for i, ctrs in enumerate(PMC_PASSES):
        lines.append(f"cd /tmp && export TMPDIR=/tmp && timeout -s KILL 180 rocprofv3 --pmc "
                     f"{ctrs} --output-format csv -d $REPO/gpurun_out/pmc_{'ab'[i]} -o p -- "
                     f"python -u $REPO/bench.py --steps 2 --warmup 1 --no-cpu-baseline "
                     f"--layer-only")
    lines += [
        "python bench.py --pmc-from gpurun_out/pmc_a gpurun_out/pmc_b",
        "```",
        "",
        "Values are means per dispatch over the runs' dispatches of each kernel and grid size "
        "(threads).  `GRBM_GUI_ACTIVE` counts GPU-busy cycles summed over the 8 XCDs; "
        "`SQ_VALU_MFMA_BUSY_CYCLES` counts busy cycles of the MFMA unit summed over the 1024 "
        "SIMDs.  Derived: MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 1024); "
        "f16 MFMA flops = SQ_INSTS_VALU_MFMA_MOPS_F16 x 512; LDS conflict = "
        "SQ_LDS_BANK_CONFLICT / SQ_ACTIVE_INST_LDS (cycles stalled on bank conflicts per cycle "
        "of issued LDS instructions); VALU per MFMA = SQ_INSTS_VALU / SQ_INSTS_MFMA.",
        "",
        "| kernel | grid (threads) | dispatches | MFMA busy | f16 MFMA GFLOP | VALU / MFMA | "
        "LDS conflict | VMEM rd | VMEM wr |",
        "|---|---|---|---|---|---|---|---|---|",
    ]

    def mean(c, name):
        v = c.get(name)
        return sum(v.values()) / len(v) if v else float("nan")

    order = sorted(per.items(), key=lambda kv: -mean(kv[1], "GRBM_GUI_ACTIVE"))
    for (name, grid), c in order:
        gui = mean(c, "GRBM_GUI_ACTIVE")
        busy = mean(c, "SQ_VALU_MFMA_BUSY_CYCLES") / (gui / n_xcd * n_simd)
        mops = mean(c, "SQ_INSTS_VALU_MFMA_MOPS_F16") * 512 / 1e9
        mfma = mean(c, "SQ_INSTS_MFMA")
        valu_per = mean(c, "SQ_INSTS_VALU") / mfma if mfma else float("nan")
        lds_c = mean(c, "SQ_LDS_BANK_CONFLICT") / max(mean(c, "SQ_ACTIVE_INST_LDS"), 1.0)
        nd = max(len(v) for v in c.values())
        lines.append(f"| `{name}` | {grid} | {nd} | {busy:.3f} | {mops:.1f} | "
                     f"{valu_per:.2f} | {lds_c:.3f} | {mean(c, 'SQ_INSTS_VMEM_RD'):.3g} | "
                     f"{mean(c, 'SQ_INSTS_VMEM_WR'):.3g} |")
    lines += ["", "Raw means per dispatch:", ""]
    for (name, grid), c in order:
        lines.append(f"- `{name}` grid {grid}: " + ", ".join(
            f"{k} {mean(c, k):.4g}" for k in sorted(c)))
    lines += ["", f"gemm_source_sha256: {_gemm_source_hash()}", ""]
    with open(PMC_FILE, "w") as fh:
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
    if args.trace_from:
        trace_summary(args.trace_from)
        return
    if args.pmc_from:
        pmc_summary(args.pmc_from)
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
    last = {}
    # the gate/up GEMM's partial maxima of |h|, one slot per work-group
    amax_buf = torch.zeros(Q.quads_moe_w4a4_gemm_amax_groups(rows, H, KR, E, 2 * I),
                           dtype=torch.int32, device=dev)

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
        h, hmax = Q.quads_moe_w4a4_gemm_amax((a["nib"], a["scale"], a["ts"]), w13q, 2 * I,
                                             rows=rows, r=(a["r_nib"], a["r_scale"], a["r_ts"]),
                                             sel=a["sel"], offsets=off, row_token=rt,
                                             amax_part=amax_buf)
        mark(3)
        b = Q.quads_rac_quantize_partials(h, KR, hmax)
        mark(4)
        y2 = Q.quads_moe_w4a4_gemm((b["nib"], b["scale"], b["ts"]), w2q, H, rows=rows,
                                   r=(b["r_nib"], b["r_scale"], b["r_ts"]), sel=b["sel"],
                                   offsets=off, out_dtype=Q.OUT_BF16)
        mark(5)
        out = Q.quads_moe_combine(y2, pos, tw, y_dtype=Q.OUT_BF16)
        mark(6)
        last.update(a=a, off=off, rt=rt)
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

    _progress("timed steps done")
    # cold: a 512 MiB write before each step (and before each lone GEMM call)
    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    la = last["a"]

    def gate_up_alone():
        return Q.quads_moe_w4a4_gemm_amax((la["nib"], la["scale"], la["ts"]), w13q, 2 * I,
                                          rows=rows, r=(la["r_nib"], la["r_scale"], la["r_ts"]),
                                          sel=la["sel"], offsets=last["off"],
                                          row_token=last["rt"], amax_part=amax_buf)
    cold_step = _cold_us(torch, lambda: step(None), flush, 20)
    cold_gemm = _cold_us(torch, gate_up_alone, flush, 20)
    warm_gemm_us = _back_to_back_us(torch, gate_up_alone, 20)
    cold = {
        "protocol": "512 MiB buffer written before each call, event pair around the call",
        "layer_step_ms": {"median": cold_step["median_us"] / 1e3,
                          "min": cold_step["min_us"] / 1e3, "reps": 20},
        "layer_value_TFLOP/s": (fl_gu + fl_dn) / (cold_step["median_us"] * 1e-6) / 1e12,
        "gemm_gate_up_swiglu": {
            "median_us": cold_gemm["median_us"], "min_us": cold_gemm["min_us"],
            "TFLOP/s": fl_gu / (cold_gemm["median_us"] * 1e-6) / 1e12,
            "frac": fl_gu / (cold_gemm["median_us"] * 1e-6) / 1e12 / PEAK_FP16_TFLOPS,
            "warm_back_to_back_us": warm_gemm_us},
    }
    _progress("cold figures done")
    overhead = rac_overhead(torch, Q, x, ids, tw, w13q, w2q, E, I, H, KR, rows, step)

    d5 = synth.make(5, with_weights=False)
    x5 = torch.from_numpy(d5["x"].view(np.int16)).to(dev)
    quant = {"gate_up_input_16384x4096": quantizer_rate(np, torch, Q, x5)}
    cfg2 = cfg5 = None
    if not args.layer_only:
        cfg2 = config2(np, torch, Q, synth, dev, flush)
        _progress("config 2 done")
        cfg5, h5 = config5(np, torch, Q, d5, x5, dev)
        _progress("config 5 done")
        quant["down_input_131072x1536"] = quantizer_rate(np, torch, Q, h5[0], part=h5[1])
        del h5
    del x5
    decode = comparator = per_expert = None
    if not args.layer_only:
        decode = decode_layer(np, torch, Q, synth, dev, w13q, w2q)
        comparator = mx_comparator(torch, Q, x, ids, E, I, rows, w13_mx,
                                   per_op["gemm_gate_up_swiglu"], fl_gu)
        per_expert = per_expert_down(torch, Q, x, ids, E, I, H, KR, rows, w13q, w2q)
        _progress("decode, comparator and per-expert selection done")

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
        "roofline": {"bound": "mfma",
                     "kernel": "gate/up GEMM call, SwiGLU epilogue: v3::k_gemm_w4a4_v3<1, false> "
                               "(256-row tiles) + dec::k_gemm_w4a4_decode<1, 2, true, true> (rows past "
                               "256 of experts of 257..320 rows)",
                     "achieved": gu_tflops, "peak": PEAK_FP16_TFLOPS, "unit": "TFLOP/s",
                     "frac": gu_tflops / PEAK_FP16_TFLOPS, "traffic": measured_traffic()},
        "cpu_baseline": cpu,
        "ops": ops,
        "cold": cold,
        "rac_overhead": overhead,
        "quantizer": quant,
        "config2": cfg2,
        "config5": cfg5,
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


def _progress(msg):
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def _back_to_back_us(torch, fn, reps):
    """Mean time per call of `reps` calls issued back to back (one event pair)."""
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def _cold_us(torch, fn, flush, reps):
    """Each call right after `flush` (512 MiB) is written, an event pair around
    the call: median and min over `reps`, in microseconds."""
    fn()
    torch.cuda.synchronize()
    ts = []
    for i in range(reps):
        flush.fill_(float(i))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3)
    ts.sort()
    return {"median_us": ts[len(ts) // 2], "min_us": ts[0]}


def rac_overhead(torch, Q, x, ids, tw, w13q, w2q, E, I, H, KR, rows, step, reps=20):
    """The layer with plain NVFP4 W4A4 at both GEMM inputs (k = 0: the
    quantizer, no residual pass and no compensation) beside the RAC layer
    (k = 64), both timed as `reps` back-to-back steps with no events inside."""
    buf = torch.zeros(Q.quads_moe_w4a4_gemm_amax_groups(rows, H, 0, E, 2 * I),
                      dtype=torch.int32, device=x.device)

    def plain():
        a = Q.quads_nvfp4_quantize(x)
        off, rt, pos = Q.quads_moe_pack(ids, E)
        h, hmax = Q.quads_moe_w4a4_gemm_amax(a, w13q, 2 * I, rows=rows, offsets=off,
                                             row_token=rt, amax_part=buf)
        b = Q.quads_nvfp4_quantize_partials(h, hmax)
        y2 = Q.quads_moe_w4a4_gemm(b, w2q, H, rows=rows, offsets=off, out_dtype=Q.OUT_BF16)
        return Q.quads_moe_combine(y2, pos, tw, y_dtype=Q.OUT_BF16)

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / reps

    ms_plain = timed(plain)
    ms_rac = timed(lambda: step(None))
    return {"layer_k0_ms": ms_plain, "layer_k64_ms": ms_rac, "ratio": ms_rac / ms_plain,
            "note": "k = 0 is plain NVFP4 W4A4 (quads_nvfp4_quantize at the gate/up input, "
                    "quads_nvfp4_quantize_partials on h with the gate/up GEMM's maxima, GEMMs "
                    "without compensation); k = 64 is the benchmark step; each timed as "
                    "back-to-back layers"}


def quantizer_rate(np, torch, Q, x, reps=20, part=None):
    """quads_nvfp4_quantize on bf16 x [M, K]: algorithmic bytes (2 read + 0.5625
    written per element) per call, with the dynamic tensor scale (a max pass,
    then the quantize pass) and with a given tensor scale (one pass); with
    `part` (the partial maxima of x its producer, the gate/up GEMM, wrote)
    also quads_nvfp4_quantize_partials, the dynamic scale in one pass.  Warm:
    `reps` calls on the same input.  Cold: the calls cycle through copies of
    the input spaced at least 512 MiB apart (each call's input was last read
    before 512 MiB of other inputs), back to back.  Calls go straight to the C
    ABI with buffers allocated once; a device-to-device copy of the input is
    timed the same two ways as context (4 bytes per element)."""
    import ctypes
    lib = Q.lib()
    dev = x.device
    m, k = x.shape
    nbytes = 2.5625 * m * k
    ncopy = -(-FLUSH_BYTES // (2 * m * k)) + 1
    xs = [x] + [x.clone() for _ in range(ncopy - 1)]
    nib = torch.empty((m, k // 2), dtype=torch.uint8, device=dev)
    sc = torch.empty((m, k // 16), dtype=torch.uint8, device=dev)
    ts = torch.empty(4, dtype=torch.float32, device=dev)
    ts_given = torch.empty(4, dtype=torch.float32, device=dev)
    nws = lib.quads_nvfp4_quantize_ws(m, k)
    ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)

    def P(t):
        return ctypes.c_void_p(t.data_ptr())

    def call(xi, ts_in):
        st = lib.quads_nvfp4_quantize(P(xi), m, k, ts_in, P(nib), P(sc), P(ts), P(ws), nws,
                                      stream)
        if st != 0:
            raise RuntimeError(f"quads_nvfp4_quantize failed with status {st}")

    call(x, None)
    ts_given.copy_(ts)
    out = {"shape": [m, k], "algorithmic_bytes": nbytes, "cold_copies": ncopy}

    def rate(us, b=nbytes):
        gbs = b / (us * 1e-6) / 1e9
        return {"us": us, "GB/s": gbs, "hbm_frac": gbs / PEAK_HBM_GBS}

    for name, ts_in in (("dynamic_scale", None), ("given_scale", P(ts_given))):
        out[name] = rate(_back_to_back_us(torch, lambda: call(x, ts_in), reps))
        it = iter(range(10 ** 9))
        out[name + "_cold"] = rate(_back_to_back_us(
            torch, lambda: call(xs[next(it) % ncopy], ts_in), ncopy * max(2, reps // ncopy)))
    if part is not None:
        def call_p(xi):
            st = lib.quads_nvfp4_quantize_partials(P(xi), m, k, P(part), int(part.numel()),
                                                   P(nib), P(sc), P(ts), stream)
            if st != 0:
                raise RuntimeError(f"quads_nvfp4_quantize_partials failed with status {st}")
        call_p(x)
        out["producer_partials"] = rate(_back_to_back_us(torch, lambda: call_p(x), reps))
        it = iter(range(10 ** 9))
        out["producer_partials_cold"] = rate(_back_to_back_us(
            torch, lambda: call_p(xs[next(it) % ncopy]), ncopy * max(2, reps // ncopy)))
    y = torch.empty_like(x)
    out["device_copy"] = rate(_back_to_back_us(torch, lambda: y.copy_(x), reps), 4.0 * m * k)
    it = iter(range(10 ** 9))
    out["device_copy_cold"] = rate(_back_to_back_us(
        torch, lambda: y.copy_(xs[next(it) % ncopy]), ncopy * max(2, reps // ncopy)), 4.0 * m * k)
    del xs
    return out


def config2(np, torch, Q, synth, dev, flush, reps=20):
    """The dense rollout-shaped linear: x [4096, 4096] bf16 (Student-t(3) body,
    41 outlier channels x20), W [4096, 4096] N(0, 0.02) through the weight
    QDQ, RAC k = 128, one W4A4 GEMM with compensation, bf16 output."""
    d = synth.make(2)
    x = torch.from_numpy(d["x"].view(np.int16)).to(dev)
    w = torch.from_numpy(d["w"].view(np.int16)).to(dev)
    m, kd = x.shape
    n = w.shape[1]
    kr = d["rac_k"]
    wq = Q.quads_nvfp4_weight_qdq(w)[:3]
    keep = {}

    def rac():
        keep["a"] = Q.quads_rac_quantize(x, kr)

    rac_us = _back_to_back_us(torch, rac, reps)
    a = keep["a"]

    def gemm():
        return Q.quads_moe_w4a4_gemm((a["nib"], a["scale"], a["ts"]), wq, n,
                                     r=(a["r_nib"], a["r_scale"], a["r_ts"]), sel=a["sel"],
                                     out_dtype=Q.OUT_BF16)
    us = _back_to_back_us(torch, gemm, reps)
    cold = _cold_us(torch, gemm, flush, reps)
    fl = 2.0 * m * n * (kd + kr)
    qb = 2.5625 * m * kd + 0.5625 * m * kr
    return {"workload": "dense_linear_m4096_k4096_n4096_rac128",
            "rac_us": rac_us, "rac_GB/s": qb / (rac_us * 1e-6) / 1e9,
            "gemm_us": us, "gemm_TFLOP/s": fl / (us * 1e-6) / 1e12,
            "gemm_frac": fl / (us * 1e-6) / 1e12 / PEAK_FP16_TFLOPS,
            "gemm_cold_median_us": cold["median_us"],
            "gemm_cold_TFLOP/s": fl / (cold["median_us"] * 1e-6) / 1e12}


def config5(np, torch, Q, d5, x, dev, reps=5):
    """The large-prefill layer's gate/up site: 16384 tokens (Student-t(2.5)
    body, 82 outlier channels x32), 64 experts, uniform top-8 routing (131072
    packed rows), hidden 4096, intermediate 1536.  Weights: N(0, 0.02) drawn
    on the device from a seeded generator, through the weight QDQ.  For
    k = 0 (plain NVFP4), 64, 256 and 2048 (half the channels): the input
    quantization (quads_nvfp4_quantize for k = 0, else quads_rac_quantize)
    and the gate/up GEMM with the SwiGLU bf16 epilogue, each timed back to
    back.  Returns the figures and the k = 64 SwiGLU output (the down site's
    input, [131072, 1536] bf16) with the GEMM's partial maxima of it."""
    E, H, I = 64, 4096, 1536
    ids = torch.from_numpy(d5["topk_ids"]).to(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(20260505)
    w = (torch.randn((E, 2 * I, H), generator=gen, device=dev) * 0.02).to(torch.bfloat16)
    w13q = Q.quads_nvfp4_weight_qdq(w)[:3]
    del w
    off, rt, _ = Q.quads_moe_pack(ids, E)
    rows = int(rt.shape[0])
    out = {"workload": "moe_gate_up_e64_h4096_i1536_top8_t16384_uniform", "packed_rows": rows,
           "k": {}}
    h64 = None
    for k in (0, 64, 256, 2048):
        keep = {}

        def quant():
            keep["a"] = Q.quads_rac_quantize(x, k) if k else Q.quads_nvfp4_quantize(x)
        q_us = _back_to_back_us(torch, quant, reps)
        a = keep["a"]
        if k:
            av, rv, sel = (a["nib"], a["scale"], a["ts"]), (a["r_nib"], a["r_scale"], a["r_ts"]), \
                a["sel"]
        else:
            av, rv, sel = a, None, None

        buf = torch.zeros(Q.quads_moe_w4a4_gemm_amax_groups(rows, H, k, E, 2 * I),
                          dtype=torch.int32, device=dev)

        def gemm():
            keep["h"] = Q.quads_moe_w4a4_gemm_amax(av, w13q, 2 * I, rows=rows, r=rv, sel=sel,
                                                   offsets=off, row_token=rt, amax_part=buf)
        us = _back_to_back_us(torch, gemm, reps)
        fl = 2.0 * rows * 2 * I * (H + k)
        qb = 2.5625 * x.shape[0] * H + 0.5625 * x.shape[0] * k
        out["k"][str(k)] = {"quantize_us": q_us, "quantize_GB/s": qb / (q_us * 1e-6) / 1e9,
                            "gemm_us": us, "gemm_TFLOP/s": fl / (us * 1e-6) / 1e12,
                            "gemm_frac": fl / (us * 1e-6) / 1e12 / PEAK_FP16_TFLOPS}
        if k == 64:
            h64 = keep["h"]
        del keep
    base = out["k"]["0"]
    for k, v in out["k"].items():
        v["time_vs_k0"] = (v["quantize_us"] + v["gemm_us"]) / (base["quantize_us"] +
                                                               base["gemm_us"])
    del w13q
    return out, h64


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
    amax_buf = torch.zeros(Q.quads_moe_w4a4_gemm_amax_groups(rows, H, KR, E, N13),
                           dtype=torch.int32, device=dev)

    def layer(evs=None):
        def mark(i):
            if evs is not None:
                evs[i].record()
        mark(0)
        a = Q.quads_rac_quantize(x, KR)
        mark(1)
        off, rt, pos = Q.quads_moe_pack(ids, E)
        mark(2)
        h, hmax = Q.quads_moe_w4a4_gemm_amax((a["nib"], a["scale"], a["ts"]), w13q, N13,
                                             rows=rows, r=(a["r_nib"], a["r_scale"], a["r_ts"]),
                                             sel=a["sel"], offsets=off, row_token=rt,
                                             amax_part=amax_buf)
        mark(3)
        b = Q.quads_rac_quantize_partials(h, KR, hmax)
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
        "gemm_gate_up_swiglu": (wb_gu, lambda: Q.quads_moe_w4a4_gemm_amax(
            (a["nib"], a["scale"], a["ts"]), w13q, N13, rows=rows,
            r=(a["r_nib"], a["r_scale"], a["r_ts"]), sel=a["sel"], offsets=off, row_token=rt,
            amax_part=amax_buf)),
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


def mx_comparator(torch, Q, x, ids, E, I, rows, w13_mx, w4a4_ms, w4a4_flops, reps=20, kr=64):
    """The gate/up GEMM of the same layer (same tokens, routing and SwiGLU bf16
    output) as an MX block-scaled GEMM (quads_moe_mx_gemm): FP8 E4M3 elements,
    the FP8 W8A8 baseline of the paper's speed claim, and FP4 E2M1 elements
    (power-of-two scales per 32: not NVFP4), and MX FP4 with RAC (k = kr
    channels, the compensation fused into the same GEMM).  Activations are
    MX-quantized from the same bf16 x; timed with events over `reps`
    launches.  Reported beside the W4A4+RAC gate/up GEMM of the timed steps."""
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
    # MX FP4 with RAC (k channels): the MX RAC quantizer and the compensated
    # block-scaled GEMM, beside NVFP4 W4A4+RAC
    if "mxfp4" in w13_mx:
        wc, wsc, _ = w13_mx["mxfp4"]
        keep = {}

        def rac():
            keep["a"] = Q.quads_mx_rac_quantize(x, kr)
        rac()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            rac()
        e1.record()
        torch.cuda.synchronize()
        rac_us = e0.elapsed_time(e1) * 1e3 / reps
        a = keep["a"]

        def run_rac():
            return Q.quads_moe_mx_rac_gemm((a["codes"], a["scales"]), (a["r_codes"], a["r_scales"]),
                                           a["sel"], (wc, wsc), 2 * I, rows=rows, offsets=off,
                                           row_token=rt, epilogue=Q.EPI_SWIGLU,
                                           out_dtype=Q.OUT_BF16)
        run_rac()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            run_rac()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        flops = 2.0 * rows * (2 * I) * (x.shape[1] + kr)
        out["mxfp4_rac"] = {"k": kr, "rac_quantize_us": rac_us, "us": us,
                            "TFLOP/s": flops / (us * 1e-6) / 1e12,
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
