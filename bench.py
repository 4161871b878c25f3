#!/usr/bin/env python3
"""MoE expert-path benchmark on one MI355X.

One step = moe_forward + moe_backward of the DeepSeek-V3-style group-limited
MoE layer (T=8192 tokens, H=7168, I=2048, 256 experts in 8 groups, top-4
groups, top-8 experts, sigmoid scores + selection bias, scale 2.5) on seeded
synthetic inputs that are resident in HBM before the timed region.  Weight
gradients are accumulated into fp32 main-gradient buffers (the training
setting where several micro-batches add into the same gradient).

Prints ONE JSON line on stdout.  Per-stage device times come from HIP events
that the library records on its own stream around each stage
(moe_set_stage_events); the roofline entry is for the slowest grouped GEMM.
The CPU baseline is the oracle, timed on a bounded token sample of the same
workload on the host cores.

The "mxfp8" object times the layer's MXFP8 step (the mxfp8 expert precision:
moe_forward_mx + moe_backward_mx, all six expert GEMMs on block-scaled fp8
MFMA) on the same inputs and buffers, after the bf16 steps: the weight-cache
fill (w1, w2 and their transposes quantised) once, then steps whose grouped
GEMMs are priced against the fp8 MFMA peak.  The cache is dropped once per
optimizer step, so a step without gradient accumulation also pays the fill:
both rates are reported.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE layer fwd+bwd tokens/s; grouped-GEMM TFLOP/s as % of bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA (the MX block-scaled ops run at it)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

GEMM_STAGES = ["up_swiglu", "down", "down_dgrad", "up_dgrad", "down_wgrad", "up_wgrad"]
# a forward workload (the few-large experts one): the forward's stages only
FWD_STAGES = ["router_proj", "router", "permute", "up_swiglu", "down", "combine"]
METRIC_FWD = "MoE layer fwd tokens/s; grouped-GEMM TFLOP/s as % of bf16 MFMA peak"
# kernel-name fragments of each grouped-GEMM op in a rocprofv3 trace (the
# single-shape kernels and the mixed m-tiling ones)
GEMM_KERNELS = {"up_swiglu": ("k_up_swiglu<", "up_swiglu_mixed<"),
                "down": ("k_down<", "down_mixed<"),
                "down_dgrad": ("k_down_dgrad<", "down_dgrad_mixed<"),
                "up_dgrad": ("k_up_dgrad<", "up_dgrad_mixed<"),
                "down_wgrad": ("k_wgrad<",), "up_wgrad": ("k_wgrad<",),
                "up_swiglu_mx": ("k_up_swiglu_mx<",),
                "down_mx": ("k_rows_mx<moe::MxCfg<256, 256, 128, 128>, 1>",),
                "down_dgrad_mx": ("k_down_dgrad_mx<",),
                "up_dgrad_mx": ("k_rows_mx<moe::MxCfg<256, 256, 128, 128>, 3>",),
                "down_wgrad_mx": ("k_wgrad_mx<",), "up_wgrad_mx": ("k_wgrad_mx<",)}


def is_gemm(frags, name):
    return any(f in name for f in frags)
# The measured HBM traffic of the grouped GEMMs lives in this file, next to a
# hash of the kernel sources it was taken with; a changed kernel reports null.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_deepseek_v3.md")
UNIFORM_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_uniform.md")
BUSY_FILE = os.path.join(ROOT, "profiles", "mfma_busy_deepseek_v3.md")
UNIFORM_BUSY_FILE = os.path.join(ROOT, "profiles", "mfma_busy_uniform.md")
TRACE_FILE = os.path.join(ROOT, "profiles", "moe_step_deepseek_v3_kernel_trace.md")
KERNEL_SOURCES = [os.path.join(ROOT, "grouped_gemm_expert_amd", "csrc", f)
                  for f in ("gemm.hip", "tile.h", "common.h", "swiglu_epi.h", "bwd_epi.h", "mxfmt.h",
                            "mx.hip")]
COPY_BYTES = 1 << 30        # plain device copy used to calibrate FETCH_SIZE / WRITE_SIZE


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gemm_flops(w, stage):
    """Algorithmic flops of one grouped-GEMM op (actual routed rows, no padding)."""
    M = w.T * w.k
    two_i = 2 * w.I
    return {"up_swiglu": 2 * M * two_i * w.H, "down": 2 * M * w.H * w.I,
            "down_dgrad": 2 * M * w.H * w.I, "up_dgrad": 2 * M * two_i * w.H,
            "down_wgrad": 2 * M * w.H * w.I, "up_wgrad": 2 * M * two_i * w.H}[stage]


def gemm_bytes(w, stage, counts, dw_accumulate):
    """Algorithmic HBM bytes of one grouped-GEMM op: each operand once (token
    tensors once per token, the weights of the experts that have rows once,
    sorted-row intermediates once per routed row), each output once, and the
    fp32 weight gradient read and written (accumulate) or written (overwrite,
    the zero fill of experts without rows included)."""
    T, H, I, E = w.T, w.H, w.I, w.E
    M = T * w.k
    act = sum(1 for c in counts if c > 0)
    w1b, w2b = act * 2 * I * H * 2, act * H * I * 2
    rmw = 2 if dw_accumulate else 1
    ob = 2 if w.precision == "bf16" else 4   # GEMM2's expert outputs o: bf16 with bf16 intermediates
    dw1 = (act * rmw + (0 if dw_accumulate else E - act)) * 2 * I * H * 4
    dw2 = (act * rmw + (0 if dw_accumulate else E - act)) * H * I * 4
    return {
        "up_swiglu": T * H * 2 + w1b + M * 2 * I * 2 + M * I * 2,
        "down": M * I * 2 + w2b + M * H * ob,
        "down_dgrad": T * H * 2 + w2b + M * 2 * I * 2 + M * I * 2 + M * 2 * I * 2,
        "up_dgrad": M * 2 * I * 2 + w1b + M * H * 2,
        "down_wgrad": M * H * 2 + M * I * 2 + dw2,
        "up_wgrad": M * 2 * I * 2 + M * H * 2 + dw1,
    }[stage]


def stage_bytes(w, stage, with_router_weight):
    """Algorithmic HBM bytes of the memory-bound stages (each operand once)."""
    T, E, k, H = w.T, w.E, w.k, w.H
    M = T * k
    ob = 2 if w.precision == "bf16" else 4   # expert outputs o (bf16 with bf16 intermediates)
    return {
        "router_proj": T * H * 2 + E * H * 4 + T * E * 4,
        "router": T * E * 4 + E * 4 + T * k * 8 + E * 4,
        "permute": 2 * M * 4 + 2 * M * 4 + 2 * (E + 1) * 4,
        "combine": M * H * ob + T * H * 4 + M * 8,
        "router_bwd": T * E * 4 * 2 + M * 12,
        "unpermute": M * H * 2 + T * H * 4 + M * 4,   # dx partials in bf16
    }.get(stage)


def run_gpu(args, w):
    import torch
    from grouped_gemm_expert_amd import inputs, ops

    dev = torch.device("cuda:0")
    log(f"[bench] generating inputs on {dev}: {inputs.describe(w)}")
    d = inputs.make_inputs(w, device=dev, seed=0)
    cfg = ops.config_from_workload(w)
    saved = ops.alloc_saved(cfg, dev)
    if d["logits"] is not None:
        saved["logits"].copy_(d["logits"])
    y = torch.empty((w.T, w.H), dtype=torch.float32, device=dev)
    aux = torch.empty((1,), dtype=torch.float32, device=dev)
    wsf = ops.workspace(cfg, "fwd", dev)
    bwd = w.backward
    wsb = ops.workspace(cfg, "bwd", dev) if bwd else None
    dx = torch.empty((w.T, w.H), dtype=torch.float32, device=dev) if bwd else None
    dl = torch.empty((w.T, w.E), dtype=torch.float32, device=dev) if bwd else None
    dWr = (torch.empty((w.E, w.H), dtype=torch.float32, device=dev)
           if bwd and d["Wr"] is not None else None)
    dW1 = torch.zeros((w.E, 2 * w.I, w.H), dtype=torch.float32, device=dev) if bwd else None
    dW2 = torch.zeros((w.E, w.H, w.I), dtype=torch.float32, device=dev) if bwd else None
    d_aux = torch.ones((1,), dtype=torch.float32, device=dev)
    acc = args.dw_mode == "accumulate"
    stage_list = list(ops.STAGES) if bwd else FWD_STAGES

    def step():
        ops.moe_forward(cfg, d["x"], d["Wr"], d["bias"], d["w1"], d["w2"], y, aux, saved, wsf)
        if bwd:
            ops.moe_backward(cfg, saved, d["x"], d["Wr"], d["w1"], d["w2"], d["dy"], d_aux, dx,
                             dl, dWr, dW1, dW2, wsb, dw_accumulate=acc)

    log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    ev = {s: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(K)] for s in stage_list}
    for pairs in ev.values():          # torch creates its HIP events on first record
        for a, b in pairs:
            a.record()
            b.record()
    log(f"[bench] timing {K} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        for s in stage_list:
            ops.moe_set_stage_events(ops.STAGES[s], *ev[s][i])
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for s in stage_list:
        ops.moe_set_stage_events(ops.STAGES[s], None, None)
    elapsed = t1 - t0

    stage_ms = {}
    for s in stage_list:
        if s == "router_proj" and d["Wr"] is None:
            continue
        if s == "router_grads" and d["Wr"] is None:
            continue
        if s == "mx_quant":               # not part of the bf16 step
            continue
        times = [a.elapsed_time(b) for a, b in ev[s]]
        stage_ms[s] = sum(times) / len(times)
    counts = saved["counts"].cpu()
    log(f"[bench] step {elapsed / K * 1e3:.3f} ms; active experts {(counts > 0).sum().item()}, "
        f"max rows {counts.max().item()}")
    out = dict(elapsed=elapsed, stage_ms=stage_ms, counts=counts.tolist(), d=d, saved=saved,
               bufs=dict(y=y, aux=aux, wsf=wsf, wsb=wsb, dx=dx, dl=dl, dWr=dWr, dW1=dW1, dW2=dW2,
                         d_aux=d_aux))
    if bwd and args.overwrite_steps > 0:
        # the same step with the weight gradients overwritten (exact zeros for
        # experts without rows): the parity tests' dW semantics
        acc = False
        for _ in range(2):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.overwrite_steps):
            step()
        torch.cuda.synchronize()
        out["overwrite_ms"] = (time.perf_counter() - t0) / args.overwrite_steps * 1e3
        log(f"[bench] overwrite-mode step {out['overwrite_ms']:.3f} ms")
    return out


MX_STAGES = ["router_proj", "router", "permute", "mx_quant", "up_swiglu", "down", "combine",
             "operands_bwd2", "down_dgrad", "down_wgrad", "operands_bwd1", "up_dgrad", "up_wgrad",
             "router_bwd", "unpermute", "router_grads"]


def run_mx(args, w, g):
    """The MXFP8 step (moe_forward_mx + moe_backward_mx) on the bf16 run's
    inputs and buffers: the weight-cache fill (all four MX forms) timed once,
    then W warmup and K timed steps with per-stage events."""
    import torch
    from grouped_gemm_expert_amd import ops

    d, b = g["d"], g["bufs"]
    dev = d["x"].device
    cfg = ops.config_from_workload(w)
    saved = g["saved"]
    acc = args.dw_mode == "accumulate"
    cache = ops.MxWeightCache(backward=True)
    log("[bench] mxfp8: quantising w1, w2 and their transposes (weight cache fill)")
    cache.get(d["w1"], d["w2"])      # first fill allocates the cache
    torch.cuda.synchronize()
    cache.drop()                     # the timed fill: the four quantiser launches
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    cache.get(d["w1"], d["w2"])
    c1.record()
    torch.cuda.synchronize()
    fill_ms = c0.elapsed_time(c1)

    def step():
        ops.moe_forward_mx(cfg, d["x"], d["Wr"], d["bias"], cache.w1_mx, cache.w2_mx, b["y"],
                           b["aux"], saved, b["wsf"])
        ops.moe_backward_mx(cfg, saved, d["x"], d["Wr"], cache.w1t_mx, cache.w2t_mx, d["dy"],
                            b["d_aux"], b["dx"], b["dl"], b["dWr"], b["dW1"], b["dW2"], b["wsb"],
                            dw_accumulate=acc)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    stages = [s for s in MX_STAGES if not (s in ("router_proj", "router_grads") and d["Wr"] is None)]
    ev = {s: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(K)] for s in stages}
    for pairs in ev.values():
        for a, z in pairs:
            a.record()
            z.record()
    torch.cuda.synchronize()
    log(f"[bench] mxfp8: timing {K} steps")
    t0 = time.perf_counter()
    for i in range(K):
        for s in stages:
            ops.moe_set_stage_events(ops.STAGES[s], *ev[s][i])
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for s in stages:
        ops.moe_set_stage_events(ops.STAGES[s], None, None)
    st = {s: sum(a.elapsed_time(z) for a, z in ev[s]) / K for s in stages}
    gemm = {s: gemm_flops(w, s) for s in GEMM_STAGES}
    tf = {s: gemm[s] / (st[s] * 1e-3) / 1e12 for s in gemm}
    dom = max(gemm, key=lambda s: st[s])
    gemm_tf = sum(gemm.values()) / (sum(st[s] for s in gemm) * 1e-3) / 1e12
    ms = (t1 - t0) / K * 1e3
    out = {
        "ms_per_step": round(ms, 4),
        "tokens_per_s": round(w.T * K / (t1 - t0), 1),
        "bf16_ms_per_step": round(g["elapsed"] / K * 1e3, 4),
        "weight_cache_fill_ms": round(fill_ms, 3),
        "tokens_per_s_with_cache_fill": round(w.T / ((ms + fill_ms) * 1e-3), 1),
        "stages": {s: {"ms": round(st[s], 4), **({"TFLOP/s": round(tf[s], 1)} if s in tf else {})}
                   for s in stages},
        "grouped_gemm": {"TFLOP/s": round(gemm_tf, 1),
                         "pct_of_fp8_peak": round(100 * gemm_tf / PEAK_FP8_TFLOPS, 2),
                         "ms_per_step": round(sum(st[s] for s in gemm), 4)},
        "roofline": {"bound": "mfma", "kernel": dom + "_mx", "achieved": round(tf[dom], 1),
                     "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf[dom] / PEAK_FP8_TFLOPS, 4),
                     "traffic": measured_traffic(dom + "_mx")},
    }
    log(f"[bench] mxfp8 step {ms:.3f} ms (bf16 {out['bf16_ms_per_step']:.3f} ms); cache fill "
        f"{fill_ms:.2f} ms; GEMMs " + ", ".join(f"{s} {tf[s]:.0f}" for s in GEMM_STAGES))
    return out


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(stage, path=None):
    """HBM bytes per launch of `stage` from the committed PMC record, or None
    when there is none or the kernel sources changed since it was taken."""
    try:
        with open(path or TRAFFIC_FILE) as fh:
            lines = [l for l in fh if l.startswith("traffic-record: ")]
    except OSError:
        return None
    if not lines:
        return None
    rec = json.loads(lines[-1][len("traffic-record: "):])
    if rec.get("source_hash") != kernel_source_hash():
        return None
    e = rec["kernels"].get(stage)
    return None if e is None else e["hbm_bytes"]


def copy_calibration():
    """A plain 1 GiB device copy, three times, as an elementwise kernel (b = a * 1,
    so that it is a kernel and not a DMA transfer): the reference whose
    FETCH_SIZE / WRITE_SIZE calibrate the counters."""
    import torch
    a = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.mul(a, 1.0, out=b)
    torch.cuda.synchronize()
    log(f"[bench] copied {COPY_BYTES} bytes 3 times")


MEM_KERNELS = ["k_router_select", "k_aux_finalize", "k_hist", "k_scan", "k_scatter", "k_schedule",
               "k_combine<float>", "k_combine<unsigned short>", "k_row_weights",
               "k_transpose_segments", "k_router_bwd", "k_mx_quantize(", "k_mx_quantize_cols"]


def counter_rows(d, counter):
    """(dispatch id, kernel name, value, duration us) of one counter in a rocprofv3 --pmc run."""
    import csv
    import glob
    out = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter:
                us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                out.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"]), us))
    out.sort()
    return out


def durations(d, counter):
    return [(n, us) for _, n, _, us in counter_rows(d, counter)]


def wgrad_is_up(name):
    """The UP flag of a weight-gradient kernel's name: the first template
    argument after the tile configuration (k_wgrad<Cfg<...>, UP, SPLIT>,
    k_wgrad_mx<Cfg<...>, UP>)."""
    rest = name.split(">, ", 1)[1] if ">, " in name else ""
    return rest.lstrip().startswith("true")


def pmc_busy_summary(busy_dir, out_path, cmds, workload="deepseek_v3"):
    """MFMA utilisation and clock of the grouped GEMMs from one rocprofv3 --pmc
    run of SQ_VALU_MFMA_BUSY_CYCLES (summed over the 1024 SIMDs) and
    GRBM_GUI_ACTIVE (summed over the 8 XCDs): busy fraction =
    MFMA_BUSY / (GUI_ACTIVE / 8 * 1024), clock = GUI_ACTIVE / 8 / duration."""
    busy = counter_rows(busy_dir, "SQ_VALU_MFMA_BUSY_CYCLES")
    gui = {i: (n, v, us) for i, n, v, us in counter_rows(busy_dir, "GRBM_GUI_ACTIVE")}
    L = [f"# MFMA utilisation of the grouped GEMMs: {TRAFFIC_TITLES[workload]}, MI355X", "",
         "Commands (from the repository root, on an MI355X):",
         "", "```"] + cmds + ["```", "",
         "Busy fraction = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs); "
         "clock = GRBM_GUI_ACTIVE / 8 / launch duration. The MFMA-bound rate at that clock is "
         "4096 bf16 (8192 fp8) flops per CU per clock x 256 CUs; the nominal 2.5 (5.0) PFLOP/s "
         "assume 2.4 GHz.", "",
         "| op | launches | MFMA busy | clock (GHz) | peak at that clock (TFLOP/s) |",
         "|---|---:|---:|---:|---:|"]
    for stage, frag in GEMM_KERNELS.items():
        want_up = stage.startswith("up_wgrad")
        wgrad = stage.startswith(("down_wgrad", "up_wgrad"))
        sel = [(i, v) for i, n, v, _ in busy if is_gemm(frag, n) and
               (not wgrad or wgrad_is_up(n) == want_up)]
        if not sel:
            continue
        fr, ck = [], []
        for i, v in sel:
            if i not in gui:
                continue
            _, g, us = gui[i]
            fr.append(v / (g / 8 * 1024))
            ck.append(g / 8 / (us * 1e3))
        if not fr:
            continue
        f, c = sum(fr) / len(fr), sum(ck) / len(ck)
        per_clk = 8192 if stage.endswith("_mx") else 4096   # fp8 MFMA: twice the bf16 rate
        L.append(f"| {stage} | {len(fr)} | {100 * f:.1f}% | {c:.2f} | {per_clk * 256 * c / 1e3:.0f} |")
    with open(out_path, "w") as fh:
        fh.write("\n".join(L) + "\n")
    print("\n".join(L))


TRAFFIC_TITLES = {
    "deepseek_v3": "DeepSeek-V3-style MoE layer (T=8192 H=7168 I=2048 E=256 G=8 kg=4 k=8)",
    "uniform": "DeepSeek-V3 shapes under `uniform` force load balancing (T=8192 H=7168 I=2048 "
               "E=256 k=8, seeded N(0, 1) logits: every expert gets rows)",
}


def trace_summary(stats_csv, bench_log, out_path, cmds):
    """The per-kernel table of a rocprofv3 --kernel-trace --stats run of the
    bench, with the stage times of the bench line that run printed."""
    import csv
    rows = list(csv.DictReader(open(stats_csv)))
    line = [l for l in open(bench_log) if l.startswith('{"metric"')][-1]
    bench = json.loads(line)
    L = [f"# Kernel trace: {TRAFFIC_TITLES['deepseek_v3']}, MI355X: bf16 fwd+bwd steps, then the "
         "MXFP8 weight-cache fill and MXFP8 fwd+bwd steps", "",
         "Commands (from the repository root, on an MI355X; the CSV lands in the -d folder):",
         "", "```"] + cmds + ["```", "", "| kernel | calls | avg us | total ms | % |",
                              "|---|---:|---:|---:|---:|"]
    for r in rows:
        name = r["Name"]
        if len(name) > 90:
            name = name[:87] + "..."
        L.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                 f"{float(r['TotalDurationNs']) / 1e6:.2f} | {float(r['Percentage']):.1f} |")
    L += ["", f"bench.py stage times (HIP events on the library stream, the same run): "
              f"{bench['ms_per_step']} ms per bf16 step", ""]
    for st, v in bench["stages"].items():
        extra = (f", {v['TFLOP/s']} TFLOP/s" if "TFLOP/s" in v
                 else (f", {v['GB/s']} GB/s" if "GB/s" in v else ""))
        L.append(f"- {st}: {v['ms']} ms{extra}")
    m = bench.get("mxfp8")
    if m:
        L += ["", f"MXFP8 step (moe_forward_mx + moe_backward_mx) stage times, same run: "
                  f"{m['ms_per_step']} ms per step (bf16 step {m['bf16_ms_per_step']} ms); MX grouped "
                  f"GEMMs {m['grouped_gemm']['TFLOP/s']} TFLOP/s ({m['grouped_gemm']['pct_of_fp8_peak']}% "
                  "of the fp8 peak)", ""]
        for st, v in m["stages"].items():
            extra = f", {v['TFLOP/s']} TFLOP/s" if "TFLOP/s" in v else ""
            L.append(f"- {st}: {v['ms']} ms{extra}")
        L.append(f"- weight-cache fill (w1, w2 and their transposes quantised): "
                 f"{m['weight_cache_fill_ms']} ms")
    with open(out_path, "w") as fh:
        fh.write("\n".join(L) + "\n")
    print("\n".join(L[:24]))


def pmc_summary(fetch_dir, write_dir, cfetch_dir, cwrite_dir, out_path, cmds,
                workload="deepseek_v3"):
    """Turn four rocprofv3 --pmc runs (bench FETCH_SIZE, bench WRITE_SIZE, copy
    FETCH_SIZE, copy WRITE_SIZE) into the traffic record bench.py reads."""
    import csv
    import glob

    def rows(d, counter):
        out = []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] == counter:
                    out.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
        out.sort()
        return out

    def copy_kib(d, counter):
        v = [x for _, n, x in rows(d, counter) if "MulFunctor" in n]
        return sorted(v)[len(v) // 2]

    kib = COPY_BYTES / 1024.0
    sf = kib / copy_kib(cfetch_dir, "FETCH_SIZE")
    sw = kib / copy_kib(cwrite_dir, "WRITE_SIZE")
    fetch, write = rows(fetch_dir, "FETCH_SIZE"), rows(write_dir, "WRITE_SIZE")
    kern = {}
    for stage, frag in GEMM_KERNELS.items():
        want_up = stage.startswith("up_wgrad")
        wgrad = stage.startswith(("down_wgrad", "up_wgrad"))
        def pick(rs):
            v = [x for _, n, x in rs if is_gemm(frag, n) and
                 (not wgrad or wgrad_is_up(n) == want_up)]
            return sum(v) / len(v) if v else None
        f, wr = pick(fetch), pick(write)
        if f is None or wr is None:
            continue
        kern[stage] = {"fetch_kib": round(f, 1), "write_kib": round(wr, 1),
                       "hbm_bytes": int(round((f * sf + wr * sw) * 1024))}
    # the memory-bound kernels of the path: measured bytes per launch and the
    # rate over the launch's duration in the counter run
    mem = {}
    for frag in MEM_KERNELS:
        fr = [(x, n) for _, n, x in fetch if frag in n]
        wr_ = [x for _, n, x in write if frag in n]
        dur = [t for n, t in durations(fetch_dir, "FETCH_SIZE") if frag in n]
        if not fr or not wr_ or not dur:
            continue
        b = (sum(x for x, _ in fr) / len(fr) * sf + sum(wr_) / len(wr_) * sw) * 1024
        mem[frag] = (b, sum(dur) / len(dur))
    rec = {"source_hash": kernel_source_hash(), "copy_scale_fetch": round(sf, 4),
           "copy_scale_write": round(sw, 4), "kernels": kern}
    L = [f"# HBM traffic of the grouped GEMMs: {TRAFFIC_TITLES[workload]}, MI355X", "",
         "Commands (from the repository root, on an MI355X):", "", "```"] + cmds + ["```", "",
         f"Calibration: a plain {COPY_BYTES} byte device copy reads FETCH_SIZE x {sf:.4f} and "
         f"WRITE_SIZE x {sw:.4f} of its true size; the per-launch figures below are scaled by "
         "those factors.", "",
         "| op | FETCH_SIZE KiB/launch | WRITE_SIZE KiB/launch | HBM bytes/launch (scaled) |",
         "|---|---:|---:|---:|"]
    for k, v in kern.items():
        L.append(f"| {k} | {v['fetch_kib']:.0f} | {v['write_kib']:.0f} | {v['hbm_bytes']:,} |")
    L += ["", "Memory-bound kernels of the path (bytes per launch as above; GB/s over each "
          "launch's duration in the FETCH_SIZE run, against the 8 TB/s HBM peak):", "",
          "| kernel | HBM bytes/launch | us/launch | GB/s | % of HBM peak |", "|---|---:|---:|---:|---:|"]
    for frag, (b, us) in mem.items():
        L.append(f"| `{frag}` | {b:,.0f} | {us:.1f} | {b / (us * 1e-6) / 1e9:.0f} | "
                 f"{100 * b / (us * 1e-6) / 1e9 / PEAK_HBM_GBS:.1f} |")
    L += ["", "traffic-record: " + json.dumps(rec)]
    with open(out_path, "w") as fh:
        fh.write("\n".join(L) + "\n")
    print("\n".join(L))


def cpu_baseline(w, d, target_s=12.0):
    """The oracle (as it stands) on a bounded sample of the same workload: the
    first S tokens as a batch -- router projection, routing, expert forward,
    backward (dx, dlogits), expert and router weight gradients."""
    import numpy as np
    import torch

    import oracle
    from grouped_gemm_expert_amd import inputs

    score = 0 if w.score == "softmax" else 1
    bias = None if d["bias"] is None else d["bias"].cpu().numpy()
    Wr = None if d["Wr"] is None else d["Wr"].cpu().numpy()

    def prepare(S):
        """Host copies for the first S tokens.  The weight arrays have the full
        [E, ...] shape but are zero-allocated lazily; only the experts these
        tokens route to are filled (and ever touched by the oracle)."""
        x = inputs.bf16_bits(d["x"][:S])
        dy = inputs.bf16_bits(d["dy"][:S])
        if Wr is not None:
            l64 = oracle.logits(x, Wr)
        else:
            l64 = d["logits"][:S].double().cpu().numpy()
        S_sel = oracle.selection_scores(l64.astype(np.float32), score, bias)
        used = np.unique(oracle.topk(S_sel, w.k, w.n_groups, w.topk_groups))
        w1 = np.zeros((w.E, 2 * w.I, w.H), np.uint16)
        w2 = np.zeros((w.E, w.H, w.I), np.uint16)
        for e in used.tolist():
            w1[e] = inputs.bf16_bits(d["w1"][e])
            w2[e] = inputs.bf16_bits(d["w2"][e])
        return x, dy, w1, w2, used

    def run(S, x, dy, w1, w2, used):
        t0 = time.perf_counter()
        if Wr is not None:
            l64 = oracle.logits(x, Wr)
        else:
            l64 = d["logits"][:S].double().cpu().numpy()
        r = oracle.route(l64, score=score, k=w.k, n_groups=w.n_groups, topk_groups=w.topk_groups,
                         bias=bias, renorm=w.renorm, scale=w.scale, coeff=w.aux_coeff)
        oracle.forward(x, w1, w2, r["idx"], r["w"])
        _, dlog = oracle.backward_tokens(x, Wr, l64, w1, w2, r["idx"], r["counts"], dy,
                                         score=score, renorm=w.renorm, scale=w.scale,
                                         coeff=w.aux_coeff)
        oracle.weight_grads(x, w1, w2, r["idx"], r["w"], dy, experts=used)
        if Wr is not None:
            oracle.router_weight_grad(x, dlog)
        return time.perf_counter() - t0

    S0 = 4
    data = prepare(S0)
    t_cal = run(S0, *data)
    S = int(max(S0, min(512, S0 * target_s / max(t_cal, 1e-3))))
    log(f"[bench] cpu baseline: calibration {S0} tokens in {t_cal:.2f} s -> sample {S} tokens")
    data = prepare(S)
    t = run(S, *data)
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": S / t, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {S} tokens of the workload as one batch, fwd+bwd incl. weight "
                      f"gradients of the {len(data[4])} experts they route to; {t:.1f} s",
            "basis": "tokens/s of that sample: an extrapolation to the workload, whose "
                     "8192-token step is not run on the CPU",
            "host_cpu": host_cpu(), "host_logical_cpus": os.cpu_count()}


def host_cpu():
    """The host CPU model name (as lscpu reports it), from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="deepseek_v3")
    ap.add_argument("--dw-mode", choices=["accumulate", "overwrite"], default="accumulate")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-mx", action="store_true", help="skip the MXFP8 leg")
    ap.add_argument("--overwrite-steps", type=int, default=5,
                    help="steps timed again with the weight gradients overwritten (0: skip)")
    ap.add_argument("--uniform-steps", type=int, default=5,
                    help="steps of the `uniform` benchmarking leg (0: skip)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run the 1 GiB copy that calibrates the PMC byte counters")
    ap.add_argument("--pmc-summary", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="write the traffic record from four rocprofv3 --pmc output folders")
    ap.add_argument("--pmc-busy-summary", metavar="DIR",
                    help="write the MFMA-busy profile from a rocprofv3 --pmc run of "
                         "SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE")
    ap.add_argument("--pmc-commands", default="", help="commands recorded with --pmc-summary (;-separated)")
    ap.add_argument("--pmc-workload", default="deepseek_v3", choices=sorted(TRAFFIC_TITLES),
                    help="the workload the --pmc-summary / --pmc-busy-summary runs measured "
                         "(picks the record file)")
    ap.add_argument("--trace-summary", nargs=2, metavar=("STATS_CSV", "BENCH_LOG"),
                    help="write the kernel-trace profile from a rocprofv3 --stats CSV and the "
                         "bench line of the same run")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.pmc_summary:
        out_path = UNIFORM_TRAFFIC_FILE if args.pmc_workload == "uniform" else TRAFFIC_FILE
        pmc_summary(*args.pmc_summary, out_path,
                    [c.strip() for c in args.pmc_commands.split(";") if c.strip()], args.pmc_workload)
        return
    if args.pmc_busy_summary:
        out_path = UNIFORM_BUSY_FILE if args.pmc_workload == "uniform" else BUSY_FILE
        pmc_busy_summary(args.pmc_busy_summary, out_path,
                         [c.strip() for c in args.pmc_commands.split(";") if c.strip()],
                         args.pmc_workload)
        return
    if args.trace_summary:
        trace_summary(*args.trace_summary, TRACE_FILE,
                      [c.strip() for c in args.pmc_commands.split(";") if c.strip()])
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}).", file=sys.stderr)
        sys.exit(2)

    from grouped_gemm_expert_amd import inputs
    w = inputs.WORKLOADS[args.workload]
    g = run_gpu(args, w)
    K = args.steps
    elapsed = g["elapsed"]
    stage_ms = g["stage_ms"]
    # a forward workload reports forward tokens/s (not the headline metric)
    gemm_stages = GEMM_STAGES if w.backward else ["up_swiglu", "down"]

    gemm_ms = {s: stage_ms[s] for s in gemm_stages}
    total_gemm_flops = sum(gemm_flops(w, s) for s in gemm_stages)
    gemm_tflops = total_gemm_flops / (sum(gemm_ms.values()) * 1e-3) / 1e12
    # the weight gradients' operand transposes exist only to feed their GEMMs:
    # the rate with them counted as GEMM time too
    prep_ms = sum(stage_ms.get(s, 0.0) for s in ("operands_bwd1", "operands_bwd2"))
    gemm_tflops_prep = total_gemm_flops / ((sum(gemm_ms.values()) + prep_ms) * 1e-3) / 1e12
    dom = max(gemm_ms, key=gemm_ms.get)
    dom_tflops = gemm_flops(w, dom) / (gemm_ms[dom] * 1e-3) / 1e12

    stages = {}
    for s, ms in stage_ms.items():
        e = {"ms": round(ms, 4)}
        if s in gemm_stages:
            e["TFLOP/s"] = round(gemm_flops(w, s) / (ms * 1e-3) / 1e12, 1)
        else:
            b = stage_bytes(w, s, g["d"]["Wr"] is not None)
            if b:
                e["GB/s"] = round(b / (ms * 1e-3) / 1e9, 1)
        stages[s] = e

    out = {
        "metric": METRIC if w.backward else METRIC_FWD,
        "value": round(w.T * K / elapsed, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "H": w.H, "I": w.I, "E": w.E, "k": w.k,
                   "n_groups": w.n_groups, "topk_groups": w.topk_groups, "score": w.score,
                   "dw": f"fp32 {args.dw_mode}" if w.backward else "none (forward)",
                   "outputs": "fp32 y/dx, bf16 operands"},
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": round(dom_tflops, 1),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(dom_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(dom)},
        "grouped_gemm": {"TFLOP/s": round(gemm_tflops, 1),
                         "pct_of_bf16_peak": round(100 * gemm_tflops / PEAK_BF16_TFLOPS, 2),
                         "flops_per_step": total_gemm_flops,
                         "ms_per_step": round(sum(gemm_ms.values()), 4),
                         "TFLOP/s_with_operand_prep": round(gemm_tflops_prep, 1),
                         "pct_of_bf16_peak_with_operand_prep":
                             round(100 * gemm_tflops_prep / PEAK_BF16_TFLOPS, 2)},
        "stages": stages,
        "active_experts": sum(1 for c in g["counts"] if c > 0),
    }
    if w.precision != "bf16":
        out["config"]["intermediates"] = w.precision
    if "overwrite_ms" in g:
        out["dw_overwrite"] = {"ms_per_step": round(g["overwrite_ms"], 4),
                               "tokens_per_s": round(w.T / (g["overwrite_ms"] * 1e-3), 1),
                               "steps": args.overwrite_steps}
    if not args.no_mx and w.backward and w.precision == "bf16":
        out["mxfp8"] = run_mx(args, w, g)
    if not args.no_cpu_baseline and w.backward:
        out["cpu_baseline"] = cpu_baseline(w, g["d"])
    if args.uniform_steps > 0 and w.name == "deepseek_v3":
        del g
        out["uniform"] = uniform_leg(args)
    print(json.dumps(out), flush=True)


def uniform_leg(args):
    """The pages' benchmarking mode, `uniform` force load balancing: the
    DeepSeek-V3 shapes with seeded i.i.d. N(0, 1) logits in place of the router
    projection, so all 256 experts get rows.  Step time, grouped-GEMM rate,
    and the HBM roofline of the slowest GEMM from its algorithmic bytes (the
    regime is weight- and weight-gradient-streaming bound)."""
    import gc

    import torch
    from grouped_gemm_expert_amd import inputs

    gc.collect()
    torch.cuda.empty_cache()
    wu = inputs.WORKLOADS["uniform"]
    a = argparse.Namespace(**vars(args))
    a.steps, a.warmup, a.overwrite_steps = args.uniform_steps, 2, 0
    g = run_gpu(a, wu)
    st = g["stage_ms"]
    acc = args.dw_mode == "accumulate"
    gemm_ms = {s: st[s] for s in GEMM_STAGES}
    flops = sum(gemm_flops(wu, s) for s in GEMM_STAGES)
    tf = flops / (sum(gemm_ms.values()) * 1e-3) / 1e12
    by = {s: gemm_bytes(wu, s, g["counts"], acc) for s in GEMM_STAGES}
    dom = max(gemm_ms, key=gemm_ms.get)
    gbs = by[dom] / (gemm_ms[dom] * 1e-3) / 1e9
    ms = g["elapsed"] / a.steps * 1e3
    res = {
        "ms_per_step": round(ms, 4),
        "tokens_per_s": round(wu.T / (ms * 1e-3), 1),
        "active_experts": sum(1 for c in g["counts"] if c > 0),
        "rows_per_expert": [min(g["counts"]), max(g["counts"])],
        "grouped_gemm": {"TFLOP/s": round(tf, 1),
                         "pct_of_bf16_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
                         "ms_per_step": round(sum(gemm_ms.values()), 4),
                         "algorithmic_bytes_per_step": sum(by.values()),
                         "GB/s": round(sum(by.values()) / (sum(gemm_ms.values()) * 1e-3) / 1e9, 1)},
        "stages": {s: {"ms": round(st[s], 4),
                       "TFLOP/s": round(gemm_flops(wu, s) / (st[s] * 1e-3) / 1e12, 1),
                       "GB/s": round(by[s] / (st[s] * 1e-3) / 1e9, 1)} for s in GEMM_STAGES},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(gbs, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "algorithmic_bytes": by[dom],
                     "traffic": measured_traffic(dom, UNIFORM_TRAFFIC_FILE)},
    }
    log(f"[bench] uniform step {ms:.3f} ms; GEMMs {tf:.0f} TF/s; {dom} {gbs:.0f} GB/s")
    return res


if __name__ == "__main__":
    main()
