#!/usr/bin/env python3
"""Benchmark of the DCU hot path on one MI355X.

Default workload (synthetic, seeded, LLaDA-8B-shaped, bf16): one full DCU denoising step plus the
end of step. Batch 8, N = 1024 tokens, 32 layers of d = 4096 (32 heads x 128), SwiGLU FFN 12288.
Per step: budgets from the previous step's layer means (B_layer = 32), then for every layer the
token distance against the cached input, top-B plus window selection (B_window = 32 around 4 key
positions per sequence in [512, 1024)), and the selective layer on the selected rows; then
confidence over [8 x 256, 126464] logits with a planted peak and the Frechet commit (delta = 0.1).
Layer inputs drift by N(0, sigma_l^2), sigma_l = 0.01 (1 + l/8), on a random 30% of each
sequence's rows (open loop: every step sees the same drift, so the cache roll, a pointer swap, is
not performed).

Prints ONE JSON line: value = selective layer-steps/s (32 layer-steps per denoising step, end of
step included in the time), plus recomputed tokens/s, per-stage times, the roofline of the
dominant kernel (timed live with HIP events on the library's stream), the dense-recompute layer at
the same shape (this library with every row selected, and a PyTorch reference of the same layer),
and the CPU oracle timed on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--no-cpu-baseline]
                    [--workload step|dist-select|layer-b1|layer-b8-n2048]

The other workloads use the same machinery at other shapes: distance + budget + select only for 32
layers at batch 1; one selective layer at batch 1 (~64 rows: budget 32 + a 32-wide window); the
32-layer step without its end at batch 8, N = 2048, B_layer = 64.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "selective layer-steps/s and recomputed tokens/s at N=1024; % HBM/MFMA peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s

L = 32
D, H, DH, F = 4096, 32, 128, 12288
V, M_CAND = 126464, 256
B_WINDOW, DELTA = 32, 0.1
APD_ALPHA, APD_BETA = 0.1, 0.1
ROPE_THETA = 500000.0           # rotary base of the LLaDA-8B configuration

# name -> shape of the run; sigma(l) is the drift of layer l's inputs
WORKLOADS = {
    "step": dict(B=8, N=1024, L=32, b_layer=32, n_keys=4, key_lo=512, cfg=5, layers=True, end=True,
                 sigma=lambda l: 0.01 * (1 + l / 8),
                 desc="full 32-layer DCU denoising step + end of step (confidence over [8x256, 126464] "
                      "logits, Frechet commit delta=0.1); LLaDA-8B-shaped layers, bf16"),
    "dist-select": dict(B=1, N=1024, L=32, b_layer=32, n_keys=4, key_lo=512, cfg=2, layers=False,
                        end=False, sigma=lambda l: 0.01 * (1 + l / 8),
                        desc="distance + budget + select for 32 layers, batch 1, N=1024, d=4096, bf16"),
    "layer-b1": dict(B=1, N=1024, L=1, b_layer=32, n_keys=1, key_lo=512, cfg=3, layers=True, end=False,
                     sigma=lambda l: 0.01 * (1 + 31 / 8),
                     desc="one selective LLaDA-8B-shaped layer, batch 1, N=1024, budget 32 + window 32"),
    "step-closed": dict(B=8, N=1024, L=32, b_layer=32, n_keys=4, key_lo=512, cfg=5, layers=True,
                        end=True, closed=True, sigma=lambda l: 0.01 * (1 + l / 8),
                        desc="closed-loop 32-layer DCU step + end of step, batch 8, N=1024: layer l+1 "
                             "reads layer l's output, distances of layers >= 1 on the scattered rows "
                             "only (with the cache roll), commits give the next step's key positions"),
    "layer-b8-n2048": dict(B=8, N=2048, L=32, b_layer=64, n_keys=4, key_lo=1024, cfg=4, layers=True,
                           end=False, sigma=lambda l: 0.01 * (1 + l / 8),
                           desc="32-layer DCU step without its end, batch 8, N=2048, B_layer=64, "
                                "LLaDA-8B-shaped layers, bf16"),
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm_gate_up_swiglu.json")
KERNEL_SOURCES = ["selective_token_cache_amd/csrc/layer.hip", "selective_token_cache_amd/csrc/gemm.h",
                  "selective_token_cache_amd/csrc/common.h"]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def stage_flops_bytes(M: int, B: int, N: int):
    """Algorithmic flops and HBM bytes of one layer's stages for M recomputed rows (whole batch)."""
    w = 2  # bf16
    return {
        "distance": dict(bytes=2 * B * N * D * w + B * N * 4),
        "select": dict(bytes=B * N * 4 + B * N * 4),
        "gather_rmsnorm": dict(bytes=2 * M * D * w + B * N * 4),
        "qkv_scatter": dict(flops=2 * M * 3 * D * D, bytes=3 * D * D * w + M * D * w + 3 * M * D * w),
        "attention": dict(flops=4 * M * N * D, bytes=B * 2 * N * D * w + 2 * M * D * w),
        "o_proj_residual": dict(flops=2 * M * D * D, bytes=D * D * w + 2 * M * D * w + M * D * 4),
        "rmsnorm": dict(bytes=M * D * 4 + M * D * w),
        "gate_up_swiglu": dict(flops=2 * M * 2 * F * D, bytes=2 * F * D * w + M * D * w + M * F * w),
        "down_residual_scatter": dict(flops=2 * M * D * F,
                                      bytes=D * F * w + M * F * w + M * D * 4 + M * D * w),
        "qkv_fixup": {}, "o_proj_fixup": {}, "gate_up_fixup": {}, "down_fixup": {},
    }


# kernels of the step as the profiler names them -> (stage, launches per layer-step (1) or per
# step (0)); the algorithmic amounts per launch come from stage_flops_bytes and the end-of-step sizes
PROFILED_KERNELS = [
    ("k_budget", "budget", 0), ("k_distance<", "distance", 1), ("k_select", "select", 1),
    ("k_gather_rmsnorm<", "gather_rmsnorm", 1), ("k_gemm<5>", "qkv_scatter", 1),
    ("k_gemm_fixup<5>", "qkv_fixup", 1), ("k_attn<", "attention", 1),
    ("k_attn_combine", "attention_combine", 1), ("k_gemm<1>", "o_proj_residual", 1),
    ("k_gemm_fixup<1>", "o_proj_fixup", 1), ("k_rmsnorm_f32<", "rmsnorm", 1),
    ("k_resid_rmsnorm<", "rmsnorm", 1),
    ("k_gemm<2>", "gate_up_swiglu", 1), ("k_gemm_fixup<2>", "gate_up_fixup", 1),
    ("k_gemm<3>", "down_residual_scatter", 1), ("k_gemm_fixup<3>", "down_fixup", 1),
    ("k_confidence<", "confidence", 0), ("k_frechet", "commit", 0),
]


def summarize_profiles(ktrace_dir, fetch_dir, write_dir, mfma_dir, bench_json, steps, cmds):
    """Write the committed profile summaries from rocprofv3 outputs of the commands in `cmds`
    (kernel trace, FETCH_SIZE, WRITE_SIZE, MFMA counters; all runs of `bench.py --profile`):
    per kernel of the step, the kernel-trace average over the timed steps' launches, the HBM-side
    bytes per launch from FETCH_SIZE / WRITE_SIZE scaled by what those counters read for a plain
    1 GiB device copy (the runtime's copy kernel) in the same run, the algorithmic bytes and flops
    per launch, and for the MFMA kernels the hardware MFMA flops and busy fraction."""
    import csv
    import glob

    def rows(d, suffix):
        return list(csv.DictReader(open(glob.glob(os.path.join(d, f"*{suffix}"))[0])))

    def match(name, tag):
        return f"::{tag}" in name

    bj = json.loads(open(bench_json).read().strip().splitlines()[-1])
    M_l = bj["rows_per_layer"]
    cfg = bj["config"]
    B, N = cfg["batch"], cfg["seq_len"]
    kt_all = rows(ktrace_dir, "_kernel_trace.csv")
    kt_all.sort(key=lambda r: int(r["Start_Timestamp"]))

    def durations(tag, per_layer):
        ks = [r for r in kt_all if match(r["Kernel_Name"], tag)]
        n = steps * (L if per_layer else 1)
        return [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in ks[-n:]]

    def counters(d):
        rs = rows(d, "_counter_collection.csv")
        by = {}
        for r in rs:
            by.setdefault((r["Counter_Name"], r["Kernel_Name"]), []).append(
                (int(r.get("Dispatch_Id", 0) or 0), float(r["Counter_Value"]), int(r["Grid_Size"])))
        return rs, by

    def counter_avg(by, cname, tag, per_layer):
        vals = []
        for (c, kname), v in by.items():
            if c == cname and match(kname, tag):
                vals += v
        vals.sort()
        n = L if per_layer else 1
        vals = [x[1] for x in vals[-n:]]
        return (sum(vals) / len(vals)) if vals else None

    def copy_cal(by, cname):
        vals = []
        for (c, kname), v in by.items():
            if c == cname and kname.startswith("__amd_rocclr_copyBuffer"):
                vals += [x for x in v if x[2] >= 131072]
        vals.sort()
        vals = [x[1] for x in vals[-3:]]
        return sum(vals) / len(vals)

    _, fby = counters(fetch_dir)
    _, wby = counters(write_dir)
    _, mby = counters(mfma_dir)
    gib_kib = float(1 << 20)
    f_scale = copy_cal(fby, "FETCH_SIZE") / gib_kib
    w_scale = copy_cal(wby, "WRITE_SIZE") / gib_kib
    table = []
    for tag, stage, per_layer in PROFILED_KERNELS:
        durs = durations(tag, per_layer)
        if not durs:
            continue
        avg_us = sum(durs) / len(durs)
        if per_layer:
            amounts = [stage_flops_bytes(int(m), B, N).get(stage, {}) for m in M_l]
            alg_b = sum(a.get("bytes", 0) for a in amounts) / len(amounts)
            alg_f = sum(a.get("flops", 0) for a in amounts) / len(amounts)
        elif stage == "confidence":
            alg_b, alg_f = B * M_CAND * V * 2, 0
        elif stage == "commit":
            alg_b, alg_f = B * M_CAND * 8, 0
        else:
            alg_b, alg_f = 2 * 4 * B * L, 0
        fk = counter_avg(fby, "FETCH_SIZE", tag, per_layer)
        wk = counter_avg(wby, "WRITE_SIZE", tag, per_layer)
        traffic = None
        if fk is not None and wk is not None:
            traffic = fk * 1024 / f_scale + wk * 1024 / w_scale
        hw_f = counter_avg(mby, "MfmaFlopsBF16", tag, per_layer)
        util = counter_avg(mby, "MfmaUtil", tag, per_layer)
        table.append(dict(kernel=tag.rstrip("<"), stage=stage, launches=len(durs), avg_us=avg_us,
                          alg_bytes=alg_b, alg_flops=alg_f, traffic=traffic, hw_mfma_flops=hw_f,
                          mfma_util=util))
    gu = next(t for t in table if t["stage"] == "gate_up_swiglu")
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    traffic = {"kernel": "k_gemm<EPI_SWIGLU> (gate/up projection + SwiGLU), 128x128 tiles",
               "workload": "full 32-layer step, batch 8, N=1024, LLaDA-8B shapes",
               "source_sha256": source_hash(),
               "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
               "traffic_bytes_per_launch": int(gu["traffic"]),
               "algorithmic_bytes_per_launch": int(gu["alg_bytes"]),
               "commands": cmds[1:3]}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(traffic, f, indent=1)
    step_us = sum(t["avg_us"] * (L if dict((k[1], k[2]) for k in PROFILED_KERNELS)[t["stage"]] else 1)
                  for t in table)
    lines = [
        "# Kernels of the full 32-layer DCU step, batch 8, N=1024 (LLaDA-8B-shaped layers, rotary, bf16)",
        "",
        "Commands (run from the repository root; each is `bench.py --profile`: set-up, warm-up and the",
        "timed steps only):",
        "",
        *["    " + c for c in cmds],
        "",
        f"Per launch, averaged over the timed region (kernel trace: last {steps} steps; counters: the",
        "one profiled step). `alg` = the algorithmic amount of the method (rows, weights, caches read",
        "or written once); `HBM` = FETCH_SIZE + WRITE_SIZE scaled by a 1 GiB copy in the same run",
        f"(FETCH_SIZE reads {f_scale:.3f} KiB per KiB copied, WRITE_SIZE {w_scale:.3f}). Rates are algorithmic",
        "amounts over the trace duration; peaks 8 TB/s HBM, 2.5 PFLOP/s dense bf16 MFMA.",
        "",
        "| kernel | stage | launches | avg us | alg MB | HBM MB | HBM/alg | alg GB/s (% of 8 TB/s) "
        "| alg TFLOP/s (% of 2.5 PF) | MFMA busy % | hw MFMA flops / alg |",
        "|---|---|---|---|---|---|---|---|---|---|---|",
    ]
    for t in table:
        gbs = t["alg_bytes"] / (t["avg_us"] * 1e-6) / 1e9 if t["alg_bytes"] else None
        tf = t["alg_flops"] / (t["avg_us"] * 1e-6) / 1e12 if t["alg_flops"] else None
        lines.append(
            f"| `{t['kernel']}` | {t['stage']} | {t['launches']} | {t['avg_us']:.2f} | "
            f"{t['alg_bytes'] / 1e6:.2f} | "
            + (f"{t['traffic'] / 1e6:.2f} | {t['traffic'] / t['alg_bytes']:.2f} | " if t["traffic"] and t["alg_bytes"] >= 1e6 else (f"{t['traffic'] / 1e6:.2f} | - | " if t["traffic"] else "- | - | "))
            + (f"{gbs:.0f} ({100 * gbs / HBM_PEAK_GBS:.1f}%) | " if gbs else "- | ")
            + (f"{tf:.0f} ({100 * tf / MFMA_BF16_PEAK_TFLOPS:.1f}%) | " if tf else "- | ")
            + (f"{t['mfma_util']:.1f} | " if t["mfma_util"] is not None and t["alg_flops"] else "- | ")
            + (f"{t['hw_mfma_flops'] / t['alg_flops']:.3f} |" if t["hw_mfma_flops"] and t["alg_flops"] else "- |"))
    lines += ["", f"Sum of the listed kernels per step: {step_us / 1e3:.2f} ms "
                  f"(bench wall time per step in the trace run: {bj['ms_per_step']:.2f} ms; the rest is "
                  "launch gaps).", ""]
    out = os.path.join(ROOT, "profiles", "kernels_full_step_b8_n1024.md")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    # the roofline kernel's own summary (the bench line's avg_launch_us must agree with it): the
    # timed steps time one gate/up launch each, step i's layer i mod L
    gu_durs = durations(next(t for t, s_, _ in PROFILED_KERNELS if s_ == "gate_up_swiglu"), True)
    sampled = [gu_durs[i * L + (i % L)] for i in range(steps) if i * L + (i % L) < len(gu_durs)]
    sampled_us = sum(sampled) / len(sampled)
    stats = rows(ktrace_dir, "_kernel_stats.csv")
    stats.sort(key=lambda r: -float(r["TotalDurationNs"]))
    g_lines = [
        "# gate/up projection GEMM (k_gemm<EPI_SWIGLU>) -- full 32-layer DCU step, batch 8, N=1024",
        "",
        "Kernel trace command (run from the repository root):",
        "",
        "    " + cmds[0],
        "",
        f"Timed-region launches (last {steps} steps x {L} layers = {gu['launches']} launches):",
        f"  rocprofv3 average duration  {gu['avg_us']:9.2f} us (every launch)",
        f"  rocprofv3, sampled launches {sampled_us:9.2f} us (step i's layer i mod {L}: the launches "
        "the bench line times)",
        f"  bench.py HIP-event average  {bj['roofline']['avg_launch_us']:9.2f} us (the same sampled launches)",
        f"  algorithmic flops / launch  {gu['alg_flops']:.4e}",
        f"  achieved (trace)            {gu['alg_flops'] / (gu['avg_us'] * 1e-6) / 1e12:.1f} TFLOP/s of {MFMA_BF16_PEAK_TFLOPS}",
        f"  achieved (bench events)     {bj['roofline']['achieved']} TFLOP/s",
        f"  HBM-side traffic / launch   {gu['traffic'] / 1e6:.1f} MB against {gu['alg_bytes'] / 1e6:.1f} MB algorithmic",
        "",
        "Whole-run kernel statistics (includes set-up: weight generation and packing, dense cache fill):",
        "",
        f"  {'kernel':90s} {'calls':>6s} {'avg us':>10s} {'pct':>6s}",
    ]
    for r in stats[:16]:
        g_lines.append(f"  {r['Name'][:90]:90s} {r['Calls']:>6s} {float(r['AverageNs']) / 1e3:10.2f} "
                       f"{float(r['Percentage']):6.2f}")
    out2 = os.path.join(ROOT, "profiles", "gemm_gate_up_swiglu_full_step_b8_n1024.md")
    with open(out2, "w") as f:
        f.write("\n".join(g_lines) + "\n")
    print(out)
    print(out2)


def summarize_counters(pmc_dir, cmd, out_name, title, notes):
    """Per-kernel averages of every counter or derived metric of one rocprofv3 --pmc run (all
    launches of each library kernel the run collected), as a table with the command that made it."""
    import collections
    import csv
    import glob
    import re

    rows = list(csv.DictReader(open(glob.glob(os.path.join(pmc_dir, "*_counter_collection.csv"))[0])))
    agg = collections.OrderedDict()
    launches = collections.defaultdict(set)
    for r in rows:
        if "dcu::" not in r["Kernel_Name"]:
            continue
        m = re.search(r"dcu::(?:\(anonymous namespace\)::)?(\w+(?:<[^>]*>)?)", r["Kernel_Name"])
        k = m.group(1) if m else r["Kernel_Name"]
        agg.setdefault(k, collections.OrderedDict()).setdefault(r["Counter_Name"], []).append(
            float(r["Counter_Value"]))
        launches[k].add(r["Dispatch_Id"])
    names = []
    for d in agg.values():
        for c in d:
            if c not in names:
                names.append(c)
    out = [f"# {title}", "", "Command (run from the repository root):", "", "    " + cmd, "",
           "Average over every launch of each kernel in the run.", ""]
    out += notes + [""] if notes else []
    # with SQ_WAVE_CYCLES in the run, the other SQ wave-cycle counters (same quad-cycle units) are
    # shown as fractions of it
    frac = "SQ_WAVE_CYCLES" in names
    shown = [c for c in names if not (frac and c == "SQ_WAVE_CYCLES")]
    heads = [f"{c} / SQ_WAVE_CYCLES" if frac and c.startswith("SQ_") else c for c in shown]
    out.append("| kernel | launches | " + " | ".join(heads) + " |")
    out.append("|---|---|" + "---|" * len(heads))
    for k, d in agg.items():
        cells = []
        for c in shown:
            v = d.get(c)
            if not v:
                cells.append("-")
            elif frac and c.startswith("SQ_"):
                cells.append(f"{sum(v) / max(sum(d['SQ_WAVE_CYCLES']), 1.0):.2f}")
            else:
                cells.append(f"{sum(v) / len(v):.4g}")
        out.append(f"| `{k}` | {len(launches[k])} | " + " | ".join(cells) + " |")
    path = os.path.join(ROOT, "profiles", out_name)
    with open(path, "w") as f:
        f.write("\n".join(out) + "\n")
    print(path)


def summarize_trace(ktrace_dir, bench_json, steps, cmd, out_name, title):
    """Kernel-trace summary of one workload (durations only). Every step starts with the budget
    kernel, so the timed region runs from the start of the last `steps` budget launches to the end
    of the trace (a --profile run stops after the timed steps); per kernel of the library, its
    launches per step and average duration inside that window."""
    import csv
    import glob
    import re

    rows = list(csv.DictReader(open(glob.glob(os.path.join(ktrace_dir, "*_kernel_trace.csv"))[0])))
    rows = [r for r in rows if "dcu::" in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    bj = json.loads(open(bench_json).read().strip().splitlines()[-1])
    budgets = [r for r in rows if "::k_budget" in r["Kernel_Name"]]
    t0 = int(budgets[-steps]["Start_Timestamp"])
    window = [r for r in rows if int(r["Start_Timestamp"]) >= t0]
    t1 = max(int(r["End_Timestamp"]) for r in window)
    by = {}
    for r in window:
        m = re.search(r"::(k_\w+(<[^>]*>)?)", r["Kernel_Name"])
        name = m.group(1) if m else r["Kernel_Name"][:40]
        by.setdefault(name, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    order = []
    for r in window:
        m = re.search(r"::(k_\w+(<[^>]*>)?)", r["Kernel_Name"])
        name = m.group(1) if m else r["Kernel_Name"][:40]
        if name not in order:
            order.append(name)
    lines = [f"# {title}", "", "Kernel trace command (run from the repository root):", "", "    " + cmd, "",
             f"The last {steps} steps of the run (from their first budget launch to the end of the "
             f"trace: {(t1 - t0) / 1e3 / steps:.1f} us per step). Bench line of the traced run: "
             f"{bj['value']} {bj['unit']}, {bj['ms_per_step']} ms per step, rows per layer "
             f"{bj['rows_per_layer_min_max']}.", "",
             "| kernel | launches per step | avg us | us per step |", "|---|---|---|---|"]
    total = 0.0
    for name in order:
        d = by[name]
        per = len(d) / steps
        avg = sum(d) / len(d)
        lines.append(f"| `{name}` | {per:g} | {avg:.2f} | {avg * per:.1f} |")
        total += avg * per
    lines += ["", f"Sum of kernel durations per step: {total:.1f} us; the rest of the step time is the "
                  "gaps between dependent launches.", ""]
    out = os.path.join(ROOT, "profiles", out_name)
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(out)


def torch_dense_layer(w, x, eps):
    """PyTorch reference of the dense layer (every row recomputed), a cross-check outside the
    library: vendor GEMMs (torch.nn.functional.linear on 2-D operands) and attention as two
    batched products on contiguous bf16 operands with an fp32 softmax."""
    import torch
    import torch.nn.functional as Fn

    Bsz, Nseq, d = x.shape
    x2 = x.reshape(Bsz * Nseq, d)

    def rms(t, g):
        t32 = t.float()
        return (t32 * torch.rsqrt(t32.pow(2).mean(-1, keepdim=True) + eps) * g.float()).to(torch.bfloat16)

    qkv = Fn.linear(rms(x2, w["g_attn"]), w["w_qkv"])
    q, k, v = (t.reshape(Bsz, Nseq, H, DH).transpose(1, 2).contiguous() for t in qkv.split(d, dim=1))
    # rotary embedding of q and k (pairs i, i + DH/2), angles in fp32
    half = DH // 2
    inv = ROPE_THETA ** (-torch.arange(half, device=x.device, dtype=torch.float64) * 2 / DH)
    ang = (torch.arange(Nseq, device=x.device, dtype=torch.float64)[:, None] * inv).float()
    cs, sn = torch.cos(ang), torch.sin(ang)

    def rot(t):
        t1, t2 = t[..., :half].float(), t[..., half:].float()
        return torch.cat([t1 * cs - t2 * sn, t2 * cs + t1 * sn], dim=-1).to(torch.bfloat16)

    q, k = rot(q), rot(k)
    s = torch.matmul(q, k.transpose(-1, -2).contiguous()).float() * (1.0 / DH ** 0.5)
    p = torch.softmax(s, dim=-1).to(torch.bfloat16)
    o = torch.matmul(p, v).transpose(1, 2).reshape(Bsz * Nseq, d)
    a = x2.float() + Fn.linear(o, w["w_o"]).float()
    an = rms(a, w["g_ffn"])
    h = (Fn.silu(Fn.linear(an, w["w_gate"]).float()) * Fn.linear(an, w["w_up"]).float()).to(torch.bfloat16)
    return (a + Fn.linear(h, w["w_down"]).float()).to(torch.bfloat16)


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-trace":
        # ktrace_dir bench_json steps cmd out_name title
        a = sys.argv[2:]
        summarize_trace(a[0], a[1], int(a[2]), a[3], a[4], a[5])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-counters":
        # pmc_dir cmd out_name title [note lines...]
        a = sys.argv[2:]
        summarize_counters(a[0], a[1], a[2], a[3], a[4:])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-profiles":
        # ktrace_dir fetch_dir write_dir mfma_dir bench_json steps cmd_trace cmd_fetch cmd_write cmd_mfma
        a = sys.argv[2:]
        summarize_profiles(a[0], a[1], a[2], a[3], a[4], int(a[5]), a[6:10])
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="step", choices=sorted(WORKLOADS))
    ap.add_argument("--dense-layers", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay measurement")
    ap.add_argument("--max-rows", type=int, default=0,
                    help="row bound passed to the layer calls (default: B * min(N, L * b_layer + window))")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also launch a plain 1 GiB device copy (counter calibration runs)")
    ap.add_argument("--profile", action="store_true",
                    help="profiler runs: only set-up, warm-up and the timed steps (no side measurements)")
    args = ap.parse_args()
    if args.profile:
        args.no_cpu_baseline = args.no_graph = True
        args.dense_layers = 0
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (the path is measured on a single MI355X); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    wl = WORKLOADS[args.workload]
    B, N, L_, B_LAYER, N_KEYS, CFG = wl["B"], wl["N"], wl["L"], wl["b_layer"], wl["n_keys"], wl["cfg"]

    import torch

    import selective_token_cache_amd as stc
    from selective_token_cache_amd._lib import LAYER_STAGES
    from workloads import device as wd

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    stc.load()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    # ------------------------------------------------------------------ inputs in HBM
    log(f"generating inputs ({args.workload})")
    layers, x_cur, x_prev, kc, vc, y = [], [], [], [], [], []
    for l in range(L_):
        if wl["layers"]:
            w = wd.layer_weights(D, F, 0.02, CFG, l, device=dev)
            # the layer keeps its own blocked copy; row-major weights stay only for layer 0
            # (the PyTorch dense reference)
            layers.append((stc.Layer(D, H, DH, F, 1e-5, w["w_qkv"], w["w_o"], w["w_gate"], w["w_up"],
                                     w["w_down"], w["g_attn"], w["g_ffn"], rope_theta=ROPE_THETA),
                           w if l == 0 else None))
            del w
            kc.append(torch.empty((B, N, H, DH), dtype=torch.bfloat16, device=dev))
            vc.append(torch.empty((B, N, H, DH), dtype=torch.bfloat16, device=dev))
            y.append(torch.empty((B, N, D), dtype=torch.bfloat16, device=dev))
        xc, xp = wd.drift_inputs(B, N, D, 0.3, wl["sigma"](l), CFG, l, device=dev)
        x_cur.append(xc)
        x_prev.append(xp)
    logits = wd.planted_logits(B * M_CAND, V, CFG, device=dev) if wl["end"] else None
    keys = wd.key_positions(B, N_KEYS, wl["key_lo"], N, CFG, device=dev)
    ws = None
    if wl["layers"]:
        ws = torch.empty((layers[0][0].workspace_bytes(B, N, B * N),), dtype=torch.uint8, device=dev)
    dist = torch.empty((B, N), dtype=torch.float32, device=dev)
    s_buf = [torch.zeros((L_, B), dtype=torch.float32, device=dev) for _ in range(2)]
    budgets = torch.empty((B, L_), dtype=torch.int32, device=dev)
    sel_idx = torch.empty((L_, B, N), dtype=torch.int32, device=dev)
    sel_cnt = torch.empty((L_, B), dtype=torch.int32, device=dev)
    conf = torch.empty((B * M_CAND,), dtype=torch.float32, device=dev)
    tok = torch.empty((B * M_CAND,), dtype=torch.int32, device=dev)
    n_commit = torch.empty((B,), dtype=torch.int32, device=dev)
    order = torch.empty((B, M_CAND), dtype=torch.int32, device=dev)

    closed = wl.get("closed", False)
    # candidate slot j of a sequence is position 512 + j (the first 256 generated positions)
    slot_pos = (torch.arange(M_CAND, dtype=torch.int32, device=dev) + N // 2).repeat(B, 1).contiguous()

    # dense fill of every layer's caches from the cached inputs (setup, untimed); in closed loop the
    # chain runs from the first layer's cached input and each later layer's cached input is a copy
    # of the previous layer's output
    if wl["layers"]:
        log("dense fill")
        for l in range(L_):
            if closed and l > 0:
                x_prev[l].copy_(y[l - 1])
            stc.dcu_selective_layer(layers[l][0], x_prev[l], None, None, kc[l], vc[l], y[l],
                                    max_rows=B * N, workspace=ws)
        torch.cuda.synchronize()

    # host-side bound on the selected rows of one layer call: a sequence's budget for one layer is
    # at most its whole step budget L * b_layer, plus the windows of its keys, and never more than N
    max_rows = args.max_rows if args.max_rows > 0 else B * min(N, L_ * B_LAYER + N_KEYS * B_WINDOW)
    stages = list(LAYER_STAGES) if wl["layers"] else []
    n_ev_layer = 2 + len(stages) + 1 if wl["layers"] else 3

    def rec(e, i):
        if e is not None and e[i] is not None:
            e[i].record()

    def step(s_prev, s_cur, ev=None):
        stc.dcu_budget(s_prev, B, L_, B_LAYER, out=budgets)
        for l in range(L_):
            e = ev[l] if ev is not None else None
            rec(e, 0)
            if closed and l > 0:
                # only the rows layer l-1 scattered can have moved; rolls them into the cache
                stc.dcu_distance_rows(y[l - 1], x_prev[l], sel_idx[l - 1], sel_cnt[l - 1], dist=dist,
                                      roll=True)
            else:
                stc.dcu_distance(x_cur[l], x_prev[l], dist=dist, want_mean=False)
            rec(e, 1)
            # the layer mean s_l (next step's budget input) comes from the select kernel, which
            # reads every distance of the sequence anyway (one launch fewer per layer)
            stc.dcu_select(dist, budgets, l, keys, B_WINDOW, sel_idx=sel_idx[l], sel_count=sel_cnt[l],
                           mean=s_cur[l])
            if wl["layers"]:
                le = e[2:] if e is not None and any(x is not None for x in e[2:]) else None
                x_in = y[l - 1] if closed and l > 0 else x_cur[l]
                stc.dcu_selective_layer(layers[l][0], x_in, sel_idx[l], sel_cnt[l], kc[l], vc[l],
                                        y[l], max_rows=max_rows, workspace=ws, events=le)
            else:
                rec(e, 2)
        if not wl["end"]:
            return
        e = ev[L_] if ev is not None else None
        rec(e, 0)
        stc.dllm_confidence(logits, V, conf=conf, token=tok)
        rec(e, 1)
        stc.frechet_commit(conf.view(B, M_CAND), DELTA, n_commit=n_commit, order=order)
        rec(e, 2)
        if closed:
            # the committed positions place the next step's windows; the first layer's input
            # alternates between its two synthetic states (its cached input is the other one)
            stc.dllm_commit_positions(order, n_commit, slot_pos, N_KEYS, key_pos=keys)
            x_cur[0], x_prev[0] = x_prev[0], x_cur[0]

    def make_events(full, sample=None):
        """Events of one step: every stage boundary (full), or only the two around the roofline
        kernel of layer `sample` (each recorded event costs ~4.5 us of device time, so a timed step
        carries just those two; the sampled layer rotates over the timed steps)."""
        def ev():
            return torch.cuda.Event(enable_timing=True)
        per = []
        for l in range(L_):
            if full:
                per.append([ev() for _ in range(n_ev_layer)])
            elif l != sample:
                per.append([None] * (n_ev_layer if wl["layers"] else 3))
            elif wl["layers"]:
                g = [None] * n_ev_layer
                gi = 2 + stages.index("gate_up_swiglu")
                g[gi], g[gi + 1] = ev(), ev()
                per.append(g)
            else:
                per.append([ev(), ev(), None])
        per.append([ev() for _ in range(3)] if full else [None, None, None])
        for group in per:  # create the event handles before they are passed to the library
            for x in group:
                if x is not None:
                    x.record()
        return per

    # warm-up: the first step has no previous means (uniform budgets)
    log(f"warmup {args.warmup}")
    first = True
    cur = 0
    for _ in range(max(args.warmup, 1)):
        step(None if first else s_buf[cur ^ 1], s_buf[cur])
        first = False
        cur ^= 1
    torch.cuda.synchronize()

    # ------------------------------------------------------------------ timed region
    # K steps with only the roofline kernel's events, then a few instrumented steps with an event
    # at every stage boundary for the per-stage table
    K = args.steps
    evs = [make_events(False, sample=it % L_) for it in range(K)]
    torch.cuda.synchronize()
    log(f"timing {K} steps")
    t0 = time.perf_counter()
    for it in range(K):
        step(s_buf[cur ^ 1], s_buf[cur], evs[it])
        cur ^= 1
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall / K * 1e3
    # roofline kernel: one sampled launch per timed step (layer it mod L), its duration from events
    roof = []                      # (layer, ms) of every sampled launch
    for it in range(K):
        l = it % L_
        e = evs[it][l]
        if wl["layers"]:
            gi = 2 + stages.index("gate_up_swiglu")
            roof.append((l, e[gi].elapsed_time(e[gi + 1])))
        else:
            roof.append((l, e[0].elapsed_time(e[1])))

    KI = 0 if args.profile else min(K, 5)
    ievs = [make_events(True) for _ in range(KI)]
    torch.cuda.synchronize()
    log(f"instrumented {KI} steps")
    for it in range(KI):
        step(s_buf[cur ^ 1], s_buf[cur], ievs[it])
        cur ^= 1
    torch.cuda.synchronize()

    counts = sel_cnt.cpu().numpy()            # same selection every step (open loop)
    M_l = counts.sum(axis=1)                   # rows recomputed per layer (whole batch)
    rows_step = int(M_l.sum())

    # per-stage device times (ms) of the instrumented steps
    names = ["distance", "select"] + stages
    stage_ms = {n: 0.0 for n in names}
    for it in range(KI):
        for l in range(L_):
            e = ievs[it][l]
            for i, n in enumerate(names):
                stage_ms[n] += e[i].elapsed_time(e[i + 1])
    kernels = {}
    for n in names if KI else []:
        per_layer_ms = stage_ms[n] / (KI * L_)
        fb = [stage_flops_bytes(int(m), B, N)[n] for m in M_l]
        flops = sum(x.get("flops", 0) for x in fb) / L_
        byts = sum(x.get("bytes", 0) for x in fb) / L_
        k = {"us_per_layer": round(per_layer_ms * 1e3, 2)}
        if byts:
            k["GBps"] = round(byts / (per_layer_ms * 1e-3) / 1e9, 1)
            k["hbm_frac"] = round(k["GBps"] / HBM_PEAK_GBS, 3)
        if flops:
            k["TFLOPps"] = round(flops / (per_layer_ms * 1e-3) / 1e12, 1)
            k["mfma_frac"] = round(k["TFLOPps"] / MFMA_BF16_PEAK_TFLOPS, 3)
        kernels[n] = k
    end_ms = {"confidence": 0.0, "commit": 0.0}
    if wl["end"] and KI:
        for it in range(KI):
            e = ievs[it][L_]
            end_ms["confidence"] += e[0].elapsed_time(e[1])
            end_ms["commit"] += e[1].elapsed_time(e[2])
        for n in end_ms:
            kernels[n] = {"us_per_step": round(end_ms[n] / KI * 1e3, 2)}
        conf_bytes = B * M_CAND * V * 2
        kernels["confidence"]["GBps"] = round(conf_bytes / (end_ms["confidence"] / KI * 1e-3) / 1e9, 1)
        kernels["confidence"]["hbm_frac"] = round(kernels["confidence"]["GBps"] / HBM_PEAK_GBS, 3)

    # the commit rules compared on the same confidences (the last step's): tokens committed per
    # sequence and device time per call, Frechet at the step's delta and the page's default, the
    # matched factor rule f = 1 - delta, and the threshold rule tau = 0.9
    commit_rules = None
    if wl["end"] and not args.profile:
        c2 = conf.view(B, M_CAND)
        commit_rules = {}
        for name, rule, param in [("frechet_delta_0.1", "frechet", DELTA),
                                  ("factor_f_0.9", "factor", 1.0 - DELTA),
                                  ("frechet_delta_0.25", "frechet", 0.25),
                                  ("factor_f_0.75", "factor", 0.75),
                                  ("threshold_tau_0.9", "threshold", 0.9)]:
            nc = torch.empty((B,), dtype=torch.int32, device=dev)
            oc = torch.empty((B, M_CAND), dtype=torch.int32, device=dev)
            stc.dllm_commit(c2, rule, param, n_commit=nc, order=oc)
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            reps = 20
            e0.record()
            for _ in range(reps):
                stc.dllm_commit(c2, rule, param, n_commit=nc, order=oc)
            e1.record()
            torch.cuda.synchronize()
            commit_rules[name] = {"tokens_per_seq": round(float(nc.float().mean()), 2),
                                  "us_per_call": round(e0.elapsed_time(e1) / reps * 1e3, 2)}

    # the V-feature distance (Value vectors recomputed for every row, compared with the V cache)
    # against the input distance the step uses, on layer 0
    vfeat = None
    if wl["layers"] and not args.profile:
        v_new = torch.empty((B, N, D), dtype=torch.bfloat16, device=dev)
        vcache = vc[0].view(B, N, D)

        def timed(fn, reps=5):
            fn()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps * 1e3

        t_vf = timed(lambda: stc.dcu_v_features(layers[0][0], x_cur[0], v_out=v_new, workspace=ws))
        t_vd = timed(lambda: stc.dcu_distance(v_new, vcache, dist=dist, want_mean=False))
        t_xd = timed(lambda: stc.dcu_distance(x_cur[0], x_prev[0], dist=dist, want_mean=False))
        vfeat = {"v_features_us": round(t_vf, 2), "v_distance_us": round(t_vd, 2),
                 "input_distance_us": round(t_xd, 2),
                 "v_proxy_over_input_proxy": round((t_vf + t_vd) / t_xd, 2),
                 "v_features_TFLOPps": round(2.0 * B * N * D * D / (t_vf * 1e-6) / 1e12, 1)}
        # the attention-context feature (DyLLM style): q of every row and its attention over the
        # caches, then the same distance on the contexts
        t_ac = timed(lambda: stc.dcu_attention_context(layers[0][0], x_cur[0], kc[0], vc[0],
                                                       ctx_out=v_new, workspace=ws))
        vfeat["attention_context_us"] = round(t_ac, 2)
        vfeat["context_proxy_over_input_proxy"] = round((t_ac + t_vd) / t_xd, 2)
        del v_new

    # adaptive parallel decoding on the same positions: the previous step's logits are this step's
    # with N(0, 0.3^2) noise; thresholds start at 0.9 (alpha = beta = 0.1: the page leaves them
    # open); one call streams both [B*256, V] logit matrices
    apd = None
    if wl["end"] and not args.profile:
        R = B * M_CAND
        zprev = wd.drifted_logits(logits, 0.3, CFG)
        tau = torch.empty((R,), dtype=torch.float32, device=dev)
        zmax = torch.empty((R,), dtype=torch.float32, device=dev)
        ca = torch.empty((R,), dtype=torch.float32, device=dev)
        ta = torch.empty((R,), dtype=torch.int32, device=dev)
        hh = torch.empty((R,), dtype=torch.float32, device=dev)

        def apd_pair():
            tau.fill_(0.9)
            stc.dllm_apd(zprev, None, V, APD_ALPHA, APD_BETA, tau, zmax, conf=ca, token=ta)
            stc.dllm_apd(logits, zprev, V, APD_ALPHA, APD_BETA, tau, zmax, conf=ca, token=ta,
                         h_instab=hh)

        apd_pair()
        nc, _ = stc.dllm_commit(ca.view(B, M_CAND), "tau", tau=tau.view(B, M_CAND))
        torch.cuda.synchronize()
        toks = float(nc.float().mean())
        h_mean = float(hh.mean())
        reps = 10
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            stc.dllm_apd(logits, zprev, V, APD_ALPHA, APD_BETA, tau, zmax, conf=ca, token=ta)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / reps * 1e3
        apd_bytes = 2.0 * R * V * 2
        apd = {"kernel": "k_apd (concentration, instability, thresholds; two logit matrices)",
               "us_per_call": round(us, 2), "GBps": round(apd_bytes / (us * 1e-6) / 1e9, 1),
               "hbm_frac": round(apd_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 3),
               "alpha": APD_ALPHA, "beta": APD_BETA, "tau0": 0.9,
               "tokens_per_seq": round(toks, 2), "mean_instability": round(h_mean, 4)}
        del zprev

    # roofline of the dominant kernel, timed with HIP events on the library's stream
    n_roof = len(roof)
    if wl["layers"]:
        gu_flops = sum(2.0 * int(M_l[l]) * 2 * F * D for l, _ in roof)
        gu_time = sum(ms for _, ms in roof) * 1e-3
        gu_bytes = (2.0 * F * D * 2) * n_roof
        if float(M_l.mean()) >= 312:
            # MFMA-bound at these row counts: gate/up projection with the SwiGLU epilogue
            achieved = gu_flops / gu_time / 1e12
            traffic = None
            if args.workload == "step" and os.path.exists(TRAFFIC_FILE):
                try:
                    tj = json.load(open(TRAFFIC_FILE))
                    if tj.get("source_sha256") == source_hash():
                        traffic = tj.get("traffic_bytes_per_launch")
                except Exception:  # pragma: no cover
                    traffic = None
            roofline = {"kernel": "k_gemm<EPI_SWIGLU> (gate/up projection + SwiGLU)", "bound": "mfma",
                        "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                        "traffic": traffic, "algorithmic_flops_per_launch": int(gu_flops / n_roof),
                        "avg_launch_us": round(gu_time / n_roof * 1e6, 2),
                        "launches_timed": n_roof}
        else:
            # few rows: the projection streams its weights once per layer-step (HBM-bound)
            achieved = gu_bytes / gu_time / 1e9
            roofline = {"kernel": "k_gemm<EPI_SWIGLU> (gate/up projection + SwiGLU)", "bound": "hbm",
                        "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                        "algorithmic_bytes_per_launch": int(gu_bytes / n_roof),
                        "avg_launch_us": round(gu_time / n_roof * 1e6, 2),
                        "launches_timed": n_roof}
    else:
        d_ms = sum(ms for _, ms in roof) / n_roof
        d_bytes = 2.0 * B * N * D * 2 + B * N * 4
        roofline = {"kernel": "k_distance (cosine distance)", "bound": "hbm",
                    "achieved": round(d_bytes / (d_ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(d_bytes / (d_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    "traffic": None, "algorithmic_bytes_per_launch": int(d_bytes),
                    "avg_launch_us": round(d_ms * 1e3, 2), "launches_timed": n_roof}

    # ------------------------------------------------------------------ dense recompute, same shape
    dense = None
    n_dense = min(args.dense_layers, L_) if wl["layers"] else 0
    if n_dense > 0:
        log("dense layers")
        kd = torch.empty_like(kc[0])
        vd = torch.empty_like(vc[0])
        yd = torch.empty_like(y[0])
        stc.dcu_selective_layer(layers[0][0], x_cur[0], None, None, kd, vd, yd, max_rows=B * N,
                                workspace=ws)
        torch.cuda.synchronize()
        dev_ev = []
        gi = stages.index("gate_up_swiglu")
        for l in range(n_dense):
            # marks only at the start, around the gate/up projection and at the end
            e = [torch.cuda.Event(enable_timing=True) if i in (0, gi, gi + 1, len(stages)) else None
                 for i in range(len(stages) + 1)]
            for x in e:
                if x is not None:
                    x.record()
            dev_ev.append(e)
        torch.cuda.synchronize()
        for l in range(n_dense):
            stc.dcu_selective_layer(layers[l][0], x_cur[l], None, None, kd, vd, yd, max_rows=B * N,
                                    workspace=ws, events=dev_ev[l])
        torch.cuda.synchronize()
        d_ms = sum(e[0].elapsed_time(e[-1]) for e in dev_ev) / n_dense
        d_gu = sum(e[gi].elapsed_time(e[gi + 1]) for e in dev_ev) / n_dense
        # selective layer-step from the timed (uninstrumented) steps, end of step excluded
        sel_ms = ms_step / L_ - (sum(end_ms.values()) / KI / L_ if wl["end"] and KI else 0.0)
        dense_flops = 2.0 * B * N * (4 * D * D + 3 * D * F) + 4.0 * B * N * N * D
        dense = {"layer_ms": round(d_ms, 3), "selective_layer_step_ms": round(sel_ms, 3),
                 "speedup_selective_vs_dense": round(d_ms / sel_ms, 2),
                 "dense_TFLOPps": round(dense_flops / (d_ms * 1e-3) / 1e12, 1),
                 "dense_gate_up_TFLOPps": round(2.0 * B * N * 2 * F * D / (d_gu * 1e-3) / 1e12, 1),
                 "rows": B * N}
        # the same dense layer written with PyTorch operators (vendor GEMMs), as a cross-check
        log("torch dense reference")
        del kd, vd, yd
        w0 = layers[0][1]
        with torch.no_grad():
            for _ in range(2):
                torch_dense_layer(w0, x_cur[0], 1e-5)
            torch.cuda.synchronize()
            t_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            t_ev[0].record()
            for _ in range(3):
                torch_dense_layer(w0, x_cur[0], 1e-5)
            t_ev[1].record()
            torch.cuda.synchronize()
        t_ms = t_ev[0].elapsed_time(t_ev[1]) / 3
        dense["torch_layer_ms"] = round(t_ms, 3)
        dense["speedup_selective_vs_torch_dense"] = round(t_ms / sel_ms, 2)
        torch.cuda.empty_cache()

    # the batch-1 layer (one sequence, budget 32 + a 32-wide window: ~64 rows) against the dense
    # layer at the same shape, with the step's first-layer weights
    layer_b1 = None
    if wl["layers"] and args.workload == "step" and not args.profile:
        log("batch-1 layer")
        layer_b1 = batch1_layer(stc, torch, wd, layers[0][0], N, dev)
    peaks = None
    if not args.profile:
        log("measured peaks")
        peaks = measure_peaks(stc, torch, dev)

    if args.calib_copy:
        log("calibration copy")
        src = torch.empty((1 << 30,), dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    # ------------------------------------------------------------------ CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline")

        def weights_of(l):
            # row-major weights of layer l: kept for layer 0, regenerated (same seeds) otherwise
            if layers[l][1] is not None:
                return layers[l][1]
            return wd.layer_weights(D, F, 0.02, CFG, l, device=dev)

        cpu = cpu_baseline(wl, weights_of, x_cur, x_prev, kc, vc, y, s_buf[cur ^ 1], keys, logits,
                           torch)

    # the same step replayed from a HIP graph (two steps captured, so the layer-mean buffers
    # alternate as in the eager loop): the library only enqueues kernels, so a whole step captures
    graph = None
    if not args.no_graph:
        try:
            gph = torch.cuda.CUDAGraph()
            torch.cuda.synchronize()
            with torch.cuda.graph(gph):
                step(s_buf[cur ^ 1], s_buf[cur])
                step(s_buf[cur], s_buf[cur ^ 1])
            gph.replay()
            torch.cuda.synchronize()
            reps = max(1, K // 2)
            t0 = time.perf_counter()
            for _ in range(reps):
                gph.replay()
            torch.cuda.synchronize()
            ms_graph = (time.perf_counter() - t0) / (2 * reps) * 1e3
            graph = {"ms_per_step": round(ms_graph, 3), "layer_steps_per_s": round(L_ / (ms_graph * 1e-3), 2),
                     "speedup_vs_eager": round(ms_step / ms_graph, 3)}
            del gph
        except Exception as exc:  # capture is an optional measurement
            graph = {"error": str(exc)[:200]}

    out = {
        "metric": METRIC,
        "value": round(L_ / (ms_step * 1e-3), 2),
        "unit": "layer-steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl["desc"], "batch": B, "seq_len": N, "layers": L_, "d": D, "heads": H,
                   "head_dim": DH, "ffn": F, "rope_theta": ROPE_THETA if wl["layers"] else None, "vocab": V if wl["end"] else None, "b_layer": B_LAYER,
                   "b_window": B_WINDOW, "max_rows": max_rows if wl["layers"] else None,
                   "keys_per_seq": N_KEYS, "drift_rows": 0.3,
                   "parallelism": "single GPU"},
        "recomputed_tokens_per_s": round(rows_step / (ms_step * 1e-3), 1),
        "rows_per_step": rows_step,
        "rows_per_layer_min_max": [int(M_l.min()), int(M_l.max())],
        "rows_per_layer": [int(m) for m in M_l],
        "kernels": kernels,
        "layer_b1": layer_b1,
        "peaks": peaks,
        "commit_rules": commit_rules,
        "apd": apd,
        "v_feature_distance": vfeat,
        "graph": graph,
        "roofline": roofline,
        "dense": dense,
        "cpu_baseline": cpu,
    }
    if not wl["layers"]:
        out["metric"] = "distance+budget+select layer-steps/s at N=1024; % HBM peak"
        out["recomputed_tokens_per_s"] = None
    if peaks is not None and roofline is not None:
        # the same achieved rate against what this device's own peak kernel reaches
        key = "mfma_loop_TFLOPps" if roofline["bound"] == "mfma" else "stream_read_GBps"
        roofline["measured_peak"] = peaks[key]
        roofline["frac_of_measured_peak"] = round(roofline["achieved"] / peaks[key], 4)
    print(json.dumps(out), flush=True)


def _event_time_ms(torch, fn, reps, warm=2):
    """Average device time of fn() over reps back-to-back calls, events on the current stream."""
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def measure_peaks(stc, torch, dev):
    """This device's own peaks: a streaming read of 2 GiB (8x the 256 MB last-level cache, so the
    bytes come from HBM; best of three grid sizes) and a loop of independent bf16 MFMAs."""
    buf = torch.empty((2 << 30,), dtype=torch.uint8, device=dev)
    sink = torch.zeros((256,), dtype=torch.int32, device=dev)
    best = 0.0
    for grid in (1024, 2048, 4096):
        ms = _event_time_ms(torch, lambda: stc.dcu_measure_stream_read(buf, grid, sink), 5)
        best = max(best, buf.numel() / (ms * 1e-3) / 1e9)
    del buf
    fs = torch.zeros((256,), dtype=torch.float32, device=dev)
    best_f = 0.0
    for grid in (1024, 2048):
        flops = [0]

        def run():
            flops[0] = stc.dcu_measure_mfma_loop(grid, 1024, fs)
        ms = _event_time_ms(torch, run, 3)
        best_f = max(best_f, flops[0] / (ms * 1e-3) / 1e12)
    return {"stream_read_GBps": round(best, 1), "hbm_nominal_GBps": HBM_PEAK_GBS,
            "stream_read_frac_of_nominal": round(best / HBM_PEAK_GBS, 3),
            "mfma_loop_TFLOPps": round(best_f, 1), "mfma_bf16_nominal_TFLOPps": MFMA_BF16_PEAK_TFLOPS,
            "mfma_loop_frac_of_nominal": round(best_f / MFMA_BF16_PEAK_TFLOPS, 3),
            "kernels": "dcu_measure_stream_read (2 GiB, 16-byte non-temporal loads, best of grids "
                       "1024/2048/4096 x 256 threads); dcu_measure_mfma_loop (8 independent "
                       "v_mfma_f32_32x32x16_bf16 chains per wave, best of 1024/2048 workgroups)"}


def batch1_layer(stc, torch, wd, layer, N, dev):
    """One sequence of N tokens through one LLaDA-8B-shaped layer with rotary embedding: the
    selective layer-step (distance, select with budget 32 and a 32-wide window around one key in
    [N/2, N), the layer on the ~64 selected rows) against the dense layer (all N rows) at the same
    shape, both this library; eager and replayed from a HIP graph."""
    sigma = 0.01 * (1 + 31 / 8)
    x_cur, x_prev = wd.drift_inputs(1, N, D, 0.3, sigma, 3, 0, device=dev)
    keys = wd.key_positions(1, 1, N // 2, N, 3, device=dev)
    kc = torch.empty((1, N, H, DH), dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    y = torch.empty((1, N, D), dtype=torch.bfloat16, device=dev)
    ws = torch.empty((layer.workspace_bytes(1, N, N),), dtype=torch.uint8, device=dev)
    stc.dcu_selective_layer(layer, x_prev, None, None, kc, vc, y, max_rows=N, workspace=ws)
    budgets = torch.full((1, 1), 32, dtype=torch.int32, device=dev)
    dist = torch.empty((1, N), dtype=torch.float32, device=dev)
    sel = torch.empty((1, N), dtype=torch.int32, device=dev)
    cnt = torch.empty((1,), dtype=torch.int32, device=dev)
    mean = torch.empty((1,), dtype=torch.float32, device=dev)
    max_rows = 32 + B_WINDOW

    def selective():
        stc.dcu_distance(x_cur, x_prev, dist=dist, want_mean=False)
        stc.dcu_select(dist, budgets, 0, keys, B_WINDOW, sel_idx=sel, sel_count=cnt, mean=mean)
        stc.dcu_selective_layer(layer, x_cur, sel, cnt, kc, vc, y, max_rows=max_rows, workspace=ws)

    kd, vd, yd = torch.empty_like(kc), torch.empty_like(vc), torch.empty_like(y)

    def dense():
        stc.dcu_selective_layer(layer, x_cur, None, None, kd, vd, yd, max_rows=N, workspace=ws)

    t_sel = _event_time_ms(torch, selective, 50)
    t_dense = _event_time_ms(torch, dense, 20)
    rows = int(cnt.item())
    out = {"workload": "one LLaDA-8B-shaped layer with rotary embedding, batch 1, N=%d, budget 32 "
                       "+ a 32-wide window around one key" % N,
           "rows": rows, "selective_layer_step_us": round(t_sel * 1e3, 2),
           "dense_layer_us": round(t_dense * 1e3, 2), "speedup": round(t_dense / t_sel, 2),
           "layer_steps_per_s": round(1e3 / t_sel, 1),
           "recomputed_tokens_per_s": round(rows / (t_sel * 1e-3), 1)}
    try:
        gs, gd = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(gs):
            selective()
        with torch.cuda.graph(gd):
            dense()
        tg_sel = _event_time_ms(torch, gs.replay, 50)
        tg_dense = _event_time_ms(torch, gd.replay, 20)
        out.update({"graph_selective_layer_step_us": round(tg_sel * 1e3, 2),
                    "graph_dense_layer_us": round(tg_dense * 1e3, 2),
                    "graph_speedup": round(tg_dense / tg_sel, 2)})
        del gs, gd
    except Exception as exc:  # capture is an optional measurement
        out["graph_error"] = str(exc)[:200]
    return out


def cpu_baseline(wl, weights_of, x_cur, x_prev, kc, vc, y, s_prev_dev, keys, logits, torch):
    """The numpy oracle, untuned, on a bounded sample of the same workload, on this host's cores:
    a subset of the layers for the whole batch (distance, select, and the selective layer when the
    workload has one) plus the end of step on 1/8 of the candidate rows, each timed three times
    (median); scaled to layer-steps/s of the whole step. BLAS threads = the CPUs this process may
    run on (sched_getaffinity). The oracle computes in fp64 only (it has no fp32 path)."""
    import statistics

    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import budget as obud
    from oracle import confidence as oconf
    from oracle import distance as odist
    from oracle import frechet as ofre
    from oracle import layer as olayer
    from oracle import select as osel

    B, L_ = wl["B"], wl["L"]
    n_cpu = len(os.sched_getaffinity(0))
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass

    def h16(t):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    if wl["layers"]:
        sample_layers = list(range(0, L_, 8)) if wl["N"] <= 1024 else [0, 16]
    else:
        sample_layers = list(range(0, L_, 2))
    host = []
    for l in sample_layers:
        w = {k: h16(v) for k, v in weights_of(l).items()} if wl["layers"] else None
        lay = (h16(kc[l]), h16(vc[l]), h16(y[l])) if wl["layers"] else None
        host.append((w, h16(x_cur[l]), h16(x_prev[l]), lay))
    s_prev = s_prev_dev.cpu().numpy().T.copy()     # [B, L]
    kp = keys.cpu().numpy()
    lg = h16(logits[: B * M_CAND // 8]) if wl["end"] else None
    t0 = time.perf_counter()
    per_layer, per_end = [], []
    with threadpool_limits(limits=n_cpu):
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        for rep in range(3):
            t1 = time.perf_counter()
            bud = obud.layer_budget(s_prev, B, L_, wl["b_layer"])
            for (w, xc, xp, lay), l in zip(host, sample_layers):
                d, _ = odist.distance_and_mean(xc, xp)
                sel, cnt = osel.select(d, bud, l, kp, B_WINDOW)
                if lay is not None:
                    olayer.selective_layer(w, H, DH, 1e-5, xc, sel, cnt, *lay, ROPE_THETA)
            per_layer.append((time.perf_counter() - t1) / len(sample_layers))
            if wl["end"]:
                t2 = time.perf_counter()
                c, _ = oconf.confidence(lg, V)
                ofre.frechet_commit(c.reshape(B // 8, M_CAND), None, DELTA)
                per_end.append((time.perf_counter() - t2) * 8)
    t_layer = statistics.median(per_layer)
    t_end = statistics.median(per_end) if per_end else 0.0
    t_step = L_ * t_layer + t_end
    what = "distance, select, selective layer" if wl["layers"] else "distance, select"
    end = " plus confidence/commit on 1/8 of the candidate rows (x8)" if wl["end"] else ""
    return {"value": round(L_ / t_step, 4), "unit": "layer-steps/s", "cores": int(threads),
            "kind": "oracle", "cpu_model": model, "cpus_available": n_cpu,
            "path": "fp64 numpy oracle (its only path)",
            "sample": f"numpy fp64 oracle on layers {sample_layers} of the batch-{B} step ({what})"
                      f"{end}; median of 3 runs, scaled to the whole {L_}-layer step",
            "sample_seconds": round(time.perf_counter() - t0, 2),
            "cpu_layer_step_s": round(t_layer, 3),
            "cpu_layer_step_s_runs": [round(x, 3) for x in per_layer]}


if __name__ == "__main__":
    main()
