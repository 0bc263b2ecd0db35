"""GPU parity at the real shapes of the batched workloads, end to end through the selection:

* batch 8, N = 2048 (1024 prompt + 1024 generated), B_layer = 64, B_window = 32, LLaDA-8B layer
  shapes: the last layer of the drift workload (sigma = 0.01 (1 + 31/8) on 30% of the rows), whose
  proportional budget reaches ~2.2k selected rows per call, driven through dcu_distance,
  dcu_budget and dcu_select into the layer; two whole sequences recomputed by the oracle;
* three closed-loop LLaDA-8B-shaped layers with rotary embedding at batch 8, N = 1024: layer l+1
  reads layer l's output, distances after the first layer come from the scattered rows only, two
  steps; every layer checked against the oracle on the GPU's own inputs.

Bars as everywhere: selections and budgets bit-exact, distances 1e-5 relative (exact 0 where the
oracle gives 0), layer rows rel-L2 <= 1e-2 per tensor and per row, other rows untouched."""
import numpy as np
import pytest
import torch

import selective_token_cache_amd as stc
from oracle import budget as obud
from oracle import distance as odist
from oracle import layer as olayer
from oracle import select as osel
from tests.util import assert_rel, dev, dev_bf16, host_bf16, rel_l2, row_rel_l2
from workloads import synth

pytestmark = pytest.mark.gpu
TOL = 1e-2


def _log(msg):
    print(msg, flush=True)


def _layer(w, shape, theta):
    t = {k: dev_bf16(v) for k, v in w.items()}
    return stc.Layer(shape.d, shape.n_heads, shape.head_dim, shape.ffn, shape.eps, t["w_qkv"],
                     t["w_o"], t["w_gate"], t["w_up"], t["w_down"], t["g_attn"], t["g_ffn"],
                     rope_theta=theta)


def _check_rows(got_k, got_v, got_y, ref, rows):
    rk, rv, ry = ref
    f = synth.bf16_to_f32
    errs = []
    for g_, r_ in ((got_k, rk), (got_v, rv), (got_y, ry)):
        a = f(g_[rows]).reshape(len(rows), -1)
        b = r_[rows].reshape(len(rows), -1)
        errs.append((rel_l2(a, b), float(row_rel_l2(a, b).max())))
    _log("  rel-L2 K %.2e (row %.2e) V %.2e (row %.2e) Y %.2e (row %.2e)" %
         tuple(x for e in errs for x in e))
    for pooled, row in errs:
        assert pooled <= TOL and row <= TOL


def test_batch8_n2048_budget_64_through_the_selection():
    shape = synth.LLADA8B
    B, N, L, b_layer, bw, layer = 8, 2048, 32, 64, 32, 31
    d = shape.d
    _log("real shape: batch 8, N 2048, B_layer 64, last layer")
    g = synth.rng(990, 0)
    cur = np.empty((B, N, d), np.uint16)
    prev = np.empty_like(cur)
    sigma = 0.01 * (1 + layer / 8)
    for b in range(B):
        cur[b], prev[b], _ = synth.drift_pair(g, N, d, int(0.3 * N), sigma)
    # previous step's layer means: the drift model's depth profile with per-sequence jitter
    prof = (1 + np.arange(L) / 8) ** 2 * 1e-5
    s_prev = (prof[None, :] * (1 + g.uniform(-0.1, 0.1, (B, L)))).astype(np.float32)
    budgets = stc.dcu_budget(dev(s_prev.T.copy()), B, L, b_layer)
    bud = budgets.cpu().numpy()
    assert np.array_equal(bud, obud.layer_budget(s_prev, B, L, b_layer))
    keys = synth.key_positions(g, B, 4, 1024, 2048)
    dist, _ = stc.dcu_distance(dev_bf16(cur), dev_bf16(prev), want_mean=False)
    dh = dist.cpu().numpy()
    rd, _ = odist.distance_and_mean(cur, prev)
    assert_rel(dh, rd)
    sel, cnt = stc.dcu_select(dist, budgets, layer, dev(keys), bw)
    rs, rc = osel.select(dh, bud, layer, keys, bw)
    assert np.array_equal(cnt.cpu().numpy(), rc) and np.array_equal(sel.cpu().numpy(), rs)
    M = int(rc.sum())
    _log(f"  budgets of layer {layer}: {bud[:, layer].tolist()}; {M} rows selected")
    assert M > 2000

    w = synth.layer_weights(g, shape)
    kv_std = 0.02 * np.sqrt(d)
    kc0 = synth.normal_bf16(g, (B, N, shape.n_heads, shape.head_dim), kv_std)
    vc0 = synth.normal_bf16(g, (B, N, shape.n_heads, shape.head_dim), kv_std)
    y0 = synth.normal_bf16(g, (B, N, d))
    lay = _layer(w, shape, 0.0)
    kc, vc, y = dev_bf16(kc0), dev_bf16(vc0), dev_bf16(y0)
    done = torch.empty((B,), dtype=torch.int32, device="cuda")
    max_rows = B * min(N, L * b_layer + 4 * bw)
    stc.dcu_selective_layer(lay, dev_bf16(cur), sel, cnt, kc, vc, y, max_rows=max_rows,
                            rows_done=done)
    torch.cuda.synchronize()
    assert np.array_equal(done.cpu().numpy(), rc)
    gk, gv, gy = host_bf16(kc), host_bf16(vc), host_bf16(y)
    for b in range(B):
        keep = np.setdiff1d(np.arange(N), rs[b, :rc[b]])
        assert np.array_equal(gy[b, keep], y0[b, keep])
        assert np.array_equal(gk[b, keep], kc0[b, keep])
        assert np.array_equal(gv[b, keep], vc0[b, keep])
    w64 = olayer.weights64(w)
    for b in (0, 5):
        _log(f"  oracle sequence {b}: {rc[b]} rows")
        ref = olayer.selective_layer_seq(w64, shape.n_heads, shape.head_dim, shape.eps,
                                         olayer.as64(cur[b]), rs[b, :rc[b]], olayer.as64(kc0[b]),
                                         olayer.as64(vc0[b]), olayer.as64(y0[b]))
        _check_rows(gk[b], gv[b], gy[b], ref, rs[b, :rc[b]])


def test_closed_loop_full_size_with_rotary():
    shape = synth.LLADA8B
    L, B, N, b_layer, bw, theta = 3, 8, 1024, 32, 32, 5e5
    d = shape.d
    _log("closed loop: 3 LLaDA-8B-shaped layers, batch 8, N 1024, rotary")
    ws_host = [synth.layer_weights(synth.rng(991, l), shape) for l in range(L)]
    layers = [_layer(w, shape, theta) for w in ws_host]
    w64 = [olayer.weights64(w) for w in ws_host]
    g = synth.rng(991, 100)
    a, bb, _ = synth.drift_pair(g, B * N, d, int(0.3 * B * N), 0.02)
    x0 = [dev_bf16(a.reshape(B, N, d)), dev_bf16(bb.reshape(B, N, d))]
    kc = [torch.zeros((B, N, shape.n_heads, shape.head_dim), dtype=torch.bfloat16, device="cuda")
          for _ in range(L)]
    vc = [torch.zeros_like(kc[0]) for _ in range(L)]
    y = [torch.zeros((B, N, d), dtype=torch.bfloat16, device="cuda") for _ in range(L)]
    xprev = [None] + [torch.zeros((B, N, d), dtype=torch.bfloat16, device="cuda") for _ in range(L - 1)]
    ws = torch.empty((layers[0].workspace_bytes(B, N, B * N),), dtype=torch.uint8, device="cuda")
    X = x0[0]
    for l in range(L):
        stc.dcu_selective_layer(layers[l], X, None, None, kc[l], vc[l], y[l], workspace=ws)
        if l + 1 < L:
            xprev[l + 1].copy_(y[l])
        X = y[l]
    keys = dev(synth.key_positions(g, B, 4, 512, 1024))
    sel = torch.empty((L, B, N), dtype=torch.int32, device="cuda")
    cnt = torch.empty((L, B), dtype=torch.int32, device="cuda")
    s_prev = None
    # a sequence's rows in one layer: at most its whole step budget plus the four keys' windows
    max_rows = B * min(N, L * b_layer + 4 * bw)
    done = torch.empty((B,), dtype=torch.int32, device="cuda")
    for step in range(2):
        cur, prev0 = x0[(step + 1) % 2], x0[step % 2]
        budgets = stc.dcu_budget(s_prev, B, L, b_layer)
        s_cur = torch.empty((L, B), dtype=torch.float32, device="cuda")
        X = cur
        for l in range(L):
            if l == 0:
                dist, _ = stc.dcu_distance(cur, prev0, want_mean=False)
                ref_in, ref_prev = host_bf16(cur), host_bf16(prev0)
            else:
                ref_in, ref_prev = host_bf16(y[l - 1]), host_bf16(xprev[l])
                dist = stc.dcu_distance_rows(y[l - 1], xprev[l], sel[l - 1], cnt[l - 1], roll=True)
                assert np.array_equal(host_bf16(xprev[l]), ref_in)
            rd, _ = odist.distance_and_mean(ref_in, ref_prev)
            dh = dist.cpu().numpy()
            assert_rel(dh, rd)
            if l > 0:
                sp, cp = sel[l - 1].cpu().numpy(), cnt[l - 1].cpu().numpy()
                for b in range(B):
                    moved = np.zeros(N, bool)
                    moved[sp[b, :cp[b]]] = True
                    assert np.all(dh[b, ~moved] == 0.0)          # stuck in the mud, exactly
            stc.dcu_select(dist, budgets, l, keys, bw, sel_idx=sel[l], sel_count=cnt[l],
                           mean=s_cur[l])
            rs, rc = osel.select(dh, budgets.cpu().numpy(), l, keys.cpu().numpy(), bw)
            assert np.array_equal(sel[l].cpu().numpy(), rs) and np.array_equal(cnt[l].cpu().numpy(), rc)
            k0, v0, y0 = host_bf16(kc[l]), host_bf16(vc[l]), host_bf16(y[l])
            stc.dcu_selective_layer(layers[l], X, sel[l], cnt[l], kc[l], vc[l], y[l],
                                    max_rows=max_rows, workspace=ws, rows_done=done)
            torch.cuda.synchronize()
            assert np.array_equal(done.cpu().numpy(), rc)
            gk, gv, gy = host_bf16(kc[l]), host_bf16(vc[l]), host_bf16(y[l])
            _log(f"  step {step} layer {l}: {int(rc.sum())} rows")
            for b in range(B):
                keep = np.setdiff1d(np.arange(N), rs[b, :rc[b]])
                assert np.array_equal(gy[b, keep], y0[b, keep])
                assert np.array_equal(gk[b, keep], k0[b, keep])
            for b in (1, 6):
                r = rs[b, :rc[b]]
                ref = olayer.selective_layer_seq(w64[l], shape.n_heads, shape.head_dim, shape.eps,
                                                 olayer.as64(ref_in[b]), r, olayer.as64(k0[b]),
                                                 olayer.as64(v0[b]), olayer.as64(y0[b]), theta)
                _check_rows(gk[b], gv[b], gy[b], ref, r)
            X = y[l]
        s_prev = s_cur
