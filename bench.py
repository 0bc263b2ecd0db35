#!/usr/bin/env python3
"""Benchmark of one full DCU denoising step plus the end of step, on one MI355X.

Workload (synthetic, seeded, LLaDA-8B-shaped, bf16): batch 8, N = 1024 tokens, 32 layers of
d = 4096 (32 heads x 128), SwiGLU FFN 12288. Per step: budgets from the previous step's layer
means (B_layer = 32), then for every layer the token distance against the cached input, top-B plus
window selection (B_window = 32 around 4 key positions per sequence in [512, 1024)), and the
selective layer on the selected rows; then confidence over [8 x 256, 126464] logits with a planted
peak and the Frechet commit (delta = 0.1). Layer inputs drift by N(0, sigma_l^2),
sigma_l = 0.01 (1 + l/8), on a random 30% of each sequence's rows (open loop: every step sees the
same drift, so the cache roll, a pointer swap, is not performed).

Prints ONE JSON line: value = selective layer-steps/s (32 layer-steps per denoising step, end of
step included in the time), plus recomputed tokens/s, per-stage times, the roofline of the
dominant kernel (timed live with HIP events on the library's stream), the dense-recompute layer at
the same shape, and the CPU oracle timed on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--no-cpu-baseline]
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

B, N, L = 8, 1024, 32
D, H, DH, F = 4096, 32, 128, 12288
V, M_CAND = 126464, 256
B_LAYER, B_WINDOW, N_KEYS, DELTA = 32, 32, 4, 0.1
CFG = 5
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


def stage_flops_bytes(M: int):
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


def summarize_profiles(ktrace_dir, fetch_dir, write_dir, bench_json, steps, cmds):
    """Write the committed profile summaries from rocprofv3 outputs of the commands in `cmds`:
    the kernel-trace average of the gate/up GEMM over the timed steps' launches (the last
    steps*32), and its per-launch HBM-side bytes from FETCH_SIZE / WRITE_SIZE scaled by what those
    counters read for a plain 1 GiB device copy (the runtime's copy kernel) in the same run."""
    import csv
    import glob

    def rows(d, suffix):
        return list(csv.DictReader(open(glob.glob(os.path.join(d, f"*{suffix}"))[0])))

    tag = "k_gemm<2,"
    kt = [r for r in rows(ktrace_dir, "_kernel_trace.csv") if tag in r["Kernel_Name"]]
    kt.sort(key=lambda r: int(r["Start_Timestamp"]))
    timed = kt[-steps * L:]
    durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in timed]
    avg_us = sum(durs) / len(durs)
    bj = json.loads(open(bench_json).read().strip().splitlines()[-1])
    stats = rows(ktrace_dir, "_kernel_stats.csv")
    stats.sort(key=lambda r: -float(r["TotalDurationNs"]))

    def counter(d, name):
        rs = rows(d, "_counter_collection.csv")
        g = [float(r["Counter_Value"]) for r in rs if tag in r["Kernel_Name"]][-L:]
        cp = [float(r["Counter_Value"]) for r in rs
              if r["Kernel_Name"].startswith("__amd_rocclr_copyBuffer") and int(r["Grid_Size"]) >= 131072][-3:]
        return sum(g) / len(g), sum(cp) / len(cp)

    f_k, f_cp = counter(fetch_dir, "FETCH_SIZE")
    w_k, w_cp = counter(write_dir, "WRITE_SIZE")
    gib_kib = float(1 << 20)
    f_scale, w_scale = f_cp / gib_kib, w_cp / gib_kib
    fetch_b = f_k * 1024 / f_scale
    write_b = w_k * 1024 / w_scale
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    traffic = {"kernel": "k_gemm<EPI_SWIGLU> (gate/up projection + SwiGLU), 128x128 tiles",
               "workload": "full 32-layer step, batch 8, N=1024, LLaDA-8B shapes",
               "source_sha256": source_hash(),
               "fetch_size_kib_per_launch": round(f_k, 1), "write_size_kib_per_launch": round(w_k, 1),
               "copy_1GiB_fetch_kib": round(f_cp, 1), "copy_1GiB_write_kib": round(w_cp, 1),
               "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
               "fetch_bytes_per_launch": int(fetch_b), "write_bytes_per_launch": int(write_b),
               "traffic_bytes_per_launch": int(fetch_b + write_b),
               "algorithmic_bytes_per_launch": None,
               "commands": cmds[1:]}
    M_avg = bj["rows_per_step"] / L
    alg = 2 * F * D * 2 + M_avg * D * 2 + M_avg * F * 2
    traffic["algorithmic_bytes_per_launch"] = int(alg)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(traffic, f, indent=1)
    lines = [
        "# gate/up projection GEMM (k_gemm<EPI_SWIGLU>) -- full 32-layer DCU step, batch 8, N=1024",
        "",
        "Kernel trace command (run from the repository root):",
        "",
        "    " + cmds[0],
        "",
        f"Timed-region launches (last {steps} steps x {L} layers = {len(durs)} launches):",
        f"  rocprofv3 average duration  {avg_us:9.2f} us",
        f"  bench.py HIP-event average  {bj['roofline']['avg_launch_us']:9.2f} us",
        f"  algorithmic flops / launch  {bj['roofline']['algorithmic_flops_per_launch']:.4e}",
        f"  achieved (bench)            {bj['roofline']['achieved']} TFLOP/s of {bj['roofline']['peak']}",
        "",
        "Counter runs:",
        "",
        "    " + cmds[1],
        "    " + cmds[2],
        "",
        f"  FETCH_SIZE per launch {f_k:12.1f} KiB; 1 GiB copy reads as {f_cp:12.1f} KiB (scale {f_scale:.4f})",
        f"  WRITE_SIZE per launch {w_k:12.1f} KiB; 1 GiB copy writes as {w_cp:12.1f} KiB (scale {w_scale:.4f})",
        f"  traffic per launch    {(fetch_b + write_b) / 1e6:9.1f} MB (fetch {fetch_b / 1e6:.1f}, write {write_b / 1e6:.1f})",
        f"  algorithmic per launch {alg / 1e6:8.1f} MB (weights 2*F*d*2 B + rows read and written)",
        "",
        "Whole-run kernel statistics (includes setup: weight generation, dense cache fill, warm-up):",
        "",
        f"  {'kernel':90s} {'calls':>6s} {'avg us':>10s} {'pct':>6s}",
    ]
    for r in stats[:16]:
        lines.append(f"  {r['Name'][:90]:90s} {r['Calls']:>6s} {float(r['AverageNs']) / 1e3:10.2f} "
                     f"{float(r['Percentage']):6.2f}")
    out = os.path.join(ROOT, "profiles", "gemm_gate_up_swiglu_full_step_b8_n1024.md")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(out)


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-profiles":
        a = sys.argv[2:]
        summarize_profiles(a[0], a[1], a[2], a[3], int(a[4]), a[5:8])
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--dense-layers", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also launch a plain 1 GiB device copy (counter calibration runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (the path is measured on a single MI355X); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

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
    log("generating inputs")
    layers, x_cur, x_prev, kc, vc, y = [], [], [], [], [], []
    for l in range(L):
        w = wd.layer_weights(D, F, 0.02, CFG, l, device=dev)
        layers.append((stc.Layer(D, H, DH, F, 1e-5, w["w_qkv"], w["w_o"], w["w_gate"], w["w_up"],
                                 w["w_down"], w["g_attn"], w["g_ffn"]), w))
        xc, xp = wd.drift_inputs(B, N, D, 0.3, 0.01 * (1 + l / 8), CFG, l, device=dev)
        x_cur.append(xc)
        x_prev.append(xp)
        kc.append(torch.empty((B, N, H, DH), dtype=torch.bfloat16, device=dev))
        vc.append(torch.empty((B, N, H, DH), dtype=torch.bfloat16, device=dev))
        y.append(torch.empty((B, N, D), dtype=torch.bfloat16, device=dev))
    logits = wd.planted_logits(B * M_CAND, V, CFG, device=dev)
    keys = wd.key_positions(B, N_KEYS, N // 2, N, CFG, device=dev)
    lay0 = layers[0][0]
    ws = torch.empty((lay0.workspace_bytes(B, N, B * N),), dtype=torch.uint8, device=dev)
    dist = torch.empty((B, N), dtype=torch.float32, device=dev)
    s_buf = [torch.zeros((L, B), dtype=torch.float32, device=dev) for _ in range(2)]
    budgets = torch.empty((B, L), dtype=torch.int32, device=dev)
    sel_idx = torch.empty((L, B, N), dtype=torch.int32, device=dev)
    sel_cnt = torch.empty((L, B), dtype=torch.int32, device=dev)
    conf = torch.empty((B * M_CAND,), dtype=torch.float32, device=dev)
    tok = torch.empty((B * M_CAND,), dtype=torch.int32, device=dev)
    n_commit = torch.empty((B,), dtype=torch.int32, device=dev)
    order = torch.empty((B, M_CAND), dtype=torch.int32, device=dev)

    # dense fill of every layer's caches from the cached inputs (setup, untimed)
    log("dense fill")
    for l in range(L):
        stc.dcu_selective_layer(layers[l][0], x_prev[l], None, None, kc[l], vc[l], y[l],
                                max_rows=B * N, workspace=ws)
    torch.cuda.synchronize()

    n_ev_layer = 2 + len(LAYER_STAGES) + 1

    def step(s_prev, s_cur, ev=None):
        stc.dcu_budget(s_prev, B, L, B_LAYER, out=budgets)
        for l in range(L):
            e = ev[l] if ev is not None else None
            if e:
                e[0].record()
            stc.dcu_distance(x_cur[l], x_prev[l], dist=dist, mean=s_cur[l])
            if e:
                e[1].record()
            stc.dcu_select(dist, budgets, l, keys, B_WINDOW, sel_idx=sel_idx[l], sel_count=sel_cnt[l])
            stc.dcu_selective_layer(layers[l][0], x_cur[l], sel_idx[l], sel_cnt[l], kc[l], vc[l], y[l],
                                    max_rows=B * N, workspace=ws, events=e[2:] if e else None)
        e = ev[L] if ev is not None else None
        if e:
            e[0].record()
        stc.dllm_confidence(logits, V, conf=conf, token=tok)
        if e:
            e[1].record()
        stc.frechet_commit(conf.view(B, M_CAND), DELTA, n_commit=n_commit, order=order)
        if e:
            e[2].record()

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
    K = args.steps
    evs = []
    for _ in range(K):
        per = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev_layer)] for _ in range(L)]
        per.append([torch.cuda.Event(enable_timing=True) for _ in range(3)])
        evs.append(per)
    for per in evs:  # create the event handles before they are passed to the library
        for group in per:
            for e in group:
                e.record()
    torch.cuda.synchronize()
    log(f"timing {K} steps")
    t0 = time.perf_counter()
    for it in range(K):
        step(s_buf[cur ^ 1], s_buf[cur], evs[it])
        cur ^= 1
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall / K * 1e3

    counts = sel_cnt.cpu().numpy()            # same selection every step (open loop)
    M_l = counts.sum(axis=1)                   # rows recomputed per layer (whole batch)
    rows_step = int(M_l.sum())

    # per-stage device times (ms), averaged over steps; per layer lists for the GEMM roofline
    names = ["distance", "select"] + list(LAYER_STAGES)
    stage_ms = {n: 0.0 for n in names}
    gateup_ms = [0.0] * L
    for it in range(K):
        for l in range(L):
            e = evs[it][l]
            for i, n in enumerate(names):
                t = e[i].elapsed_time(e[i + 1])
                stage_ms[n] += t
                if n == "gate_up_swiglu":
                    gateup_ms[l] += t
    end_ms = {"confidence": 0.0, "commit": 0.0}
    for it in range(K):
        e = evs[it][L]
        end_ms["confidence"] += e[0].elapsed_time(e[1])
        end_ms["commit"] += e[1].elapsed_time(e[2])

    kernels = {}
    for n in names:
        per_layer_ms = stage_ms[n] / (K * L)
        fb = [stage_flops_bytes(int(m))[n] for m in M_l]
        flops = sum(x.get("flops", 0) for x in fb) / L
        byts = sum(x.get("bytes", 0) for x in fb) / L
        k = {"us_per_layer": round(per_layer_ms * 1e3, 2)}
        if byts:
            k["GBps"] = round(byts / (per_layer_ms * 1e-3) / 1e9, 1)
            k["hbm_frac"] = round(k["GBps"] / HBM_PEAK_GBS, 3)
        if flops:
            k["TFLOPps"] = round(flops / (per_layer_ms * 1e-3) / 1e12, 1)
            k["mfma_frac"] = round(k["TFLOPps"] / MFMA_BF16_PEAK_TFLOPS, 3)
        kernels[n] = k
    for n in end_ms:
        us = end_ms[n] / K * 1e3
        kernels[n] = {"us_per_step": round(us, 2)}
    conf_bytes = B * M_CAND * V * 2
    kernels["confidence"]["GBps"] = round(conf_bytes / (end_ms["confidence"] / K * 1e-3) / 1e9, 1)
    kernels["confidence"]["hbm_frac"] = round(kernels["confidence"]["GBps"] / HBM_PEAK_GBS, 3)

    # roofline of the dominant kernel: gate/up projection with the SwiGLU epilogue
    gu_flops = sum(2.0 * int(M_l[l]) * 2 * F * D for l in range(L)) * K
    gu_time = sum(gateup_ms) * 1e-3
    achieved = gu_flops / gu_time / 1e12
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        try:
            tj = json.load(open(TRAFFIC_FILE))
            if tj.get("source_sha256") == source_hash():
                traffic = tj.get("traffic_bytes_per_launch")
        except Exception:  # pragma: no cover
            traffic = None
    roofline = {"kernel": "k_gemm<EPI_SWIGLU> (gate/up projection + SwiGLU)", "bound": "mfma",
                "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic,
                "algorithmic_flops_per_launch": int(gu_flops / (K * L)),
                "avg_launch_us": round(gu_time / (K * L) * 1e6, 2)}

    # ------------------------------------------------------------------ dense recompute, same shape
    dense = None
    if args.dense_layers > 0:
        log("dense layers")
        kd = torch.empty_like(kc[0])
        vd = torch.empty_like(vc[0])
        yd = torch.empty_like(y[0])
        stc.dcu_selective_layer(layers[0][0], x_cur[0], None, None, kd, vd, yd, max_rows=B * N,
                                workspace=ws)
        torch.cuda.synchronize()
        dev_ev = []
        for l in range(args.dense_layers):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(len(LAYER_STAGES) + 1)]
            for x in e:
                x.record()
            dev_ev.append(e)
        torch.cuda.synchronize()
        for l in range(args.dense_layers):
            stc.dcu_selective_layer(layers[l][0], x_cur[l], None, None, kd, vd, yd, max_rows=B * N,
                                    workspace=ws, events=dev_ev[l])
        torch.cuda.synchronize()
        d_ms = sum(e[0].elapsed_time(e[-1]) for e in dev_ev) / args.dense_layers
        d_gu = sum(e[LAYER_STAGES.index("gate_up_swiglu")].elapsed_time(
            e[LAYER_STAGES.index("gate_up_swiglu") + 1]) for e in dev_ev) / args.dense_layers
        sel_ms = (stage_ms["distance"] + stage_ms["select"] +
                  sum(stage_ms[n] for n in LAYER_STAGES)) / (K * L)
        dense_flops = 2.0 * B * N * (4 * D * D + 3 * D * F) + 4.0 * B * N * N * D
        dense = {"layer_ms": round(d_ms, 3), "selective_layer_step_ms": round(sel_ms, 3),
                 "speedup_selective_vs_dense": round(d_ms / sel_ms, 2),
                 "dense_TFLOPps": round(dense_flops / (d_ms * 1e-3) / 1e12, 1),
                 "dense_gate_up_TFLOPps": round(2.0 * B * N * 2 * F * D / (d_gu * 1e-3) / 1e12, 1),
                 "rows": B * N}

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
        cpu = cpu_baseline(layers, x_cur, x_prev, kc, vc, y, s_buf[cur ^ 1], keys, logits, torch)

    out = {
        "metric": METRIC,
        "value": round(L / (ms_step * 1e-3), 2),
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
        "config": {"workload": "full 32-layer DCU denoising step + end of step (confidence over "
                               "[8x256, 126464] logits, Frechet commit delta=0.1); LLaDA-8B-shaped "
                               "layers, bf16",
                   "batch": B, "seq_len": N, "layers": L, "d": D, "heads": H, "head_dim": DH,
                   "ffn": F, "vocab": V, "b_layer": B_LAYER, "b_window": B_WINDOW,
                   "keys_per_seq": N_KEYS, "drift_rows": 0.3, "parallelism": "single GPU"},
        "recomputed_tokens_per_s": round(rows_step / (ms_step * 1e-3), 1),
        "rows_per_step": rows_step,
        "rows_per_layer_min_max": [int(M_l.min()), int(M_l.max())],
        "kernels": kernels,
        "roofline": roofline,
        "dense": dense,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(layers, x_cur, x_prev, kc, vc, y, s_prev_dev, keys, logits, torch):
    """The numpy oracle, untuned, on a bounded sample of the same step: 8 of the 32 layers for the
    whole batch (distance, select, selective layer) plus the end of step on 1/8 of the candidate
    rows; scaled to layer-steps/s of the full step (32 layers + full end of step)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import budget as obud
    from oracle import confidence as oconf
    from oracle import distance as odist
    from oracle import frechet as ofre
    from oracle import layer as olayer
    from oracle import select as osel

    def h16(t):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    sample_layers = list(range(0, L, 4))
    host = []
    for l in sample_layers:
        w = {k: h16(v) for k, v in layers[l][1].items()}
        host.append((w, h16(x_cur[l]), h16(x_prev[l]), h16(kc[l]), h16(vc[l]), h16(y[l])))
    s_prev = s_prev_dev.cpu().numpy().T.copy()     # [B, L]
    kp = keys.cpu().numpy()
    lg = h16(logits[: B * M_CAND // 8])
    t0 = time.perf_counter()
    bud = obud.layer_budget(s_prev, B, L, B_LAYER)
    for (w, xc, xp, k_, v_, y_), l in zip(host, sample_layers):
        d, _ = odist.distance_and_mean(xc, xp)
        sel, cnt = osel.select(d, bud, l, kp, B_WINDOW)
        olayer.selective_layer(w, H, DH, 1e-5, xc, sel, cnt, k_, v_, y_)
    t_layer = (time.perf_counter() - t0) / len(sample_layers)
    t1 = time.perf_counter()
    c, _ = oconf.confidence(lg, V)
    ofre.frechet_commit(c.reshape(B // 8, M_CAND), None, DELTA)
    t_end = (time.perf_counter() - t1) * 8
    t_step = L * t_layer + t_end
    sample_s = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": round(L / t_step, 4), "unit": "layer-steps/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"numpy fp64 oracle on layers {sample_layers} of the batch-8 step (distance, "
                      f"select, selective layer) plus confidence/commit on 1/8 of the 2048 "
                      f"candidate rows; scaled to a 32-layer step with full end of step",
            "sample_seconds": round(sample_s, 2),
            "cpu_layer_step_s": round(t_layer, 3)}


if __name__ == "__main__":
    main()
