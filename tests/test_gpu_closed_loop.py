"""Closed-loop DCU steps on the GPU: layer l+1's input is layer l's output buffer, the distances of
layers after the first read only the rows the previous layer scattered (dcu_distance_rows, with the
cache roll), and the commits of a step give the next step's key positions. Checked per layer against
the oracle on the same GPU inputs: distances, the stuck-in-the-mud zeros of Key design 2 (a row the
previous layer did not update has distance 0 exactly), the selections (bit for bit) and the layer
outputs."""
import numpy as np
import pytest
import torch

import selective_token_cache_amd as stc
from oracle import distance as odist
from oracle import layer as olayer
from oracle import select as osel
from oracle import step as ostep
from tests.util import assert_rel, dev, dev_bf16, host_bf16, rel_l2
from workloads import synth

pytestmark = pytest.mark.gpu
THETA = 1e4  # rotary embedding on, as in the models the chain stands for


def test_closed_loop_steps_against_the_oracle():
    g = synth.rng(980, 0)
    shape = synth.LayerShape(d=128, n_heads=2, head_dim=64, ffn=192)
    L, B, N, MC, V = 3, 2, 64, 16, 512
    d = shape.d
    ws_host = [synth.layer_weights(g, shape, std=0.05, gain_jitter=0.1) for _ in range(L)]
    layers = []
    for w in ws_host:
        t = {k: dev_bf16(v) for k, v in w.items()}
        layers.append(stc.Layer(d, shape.n_heads, shape.head_dim, shape.ffn, shape.eps, t["w_qkv"],
                                t["w_o"], t["w_gate"], t["w_up"], t["w_down"], t["g_attn"], t["g_ffn"],
                                rope_theta=THETA))
    # two alternating first-layer inputs that differ on a third of the rows
    a, bb, _ = synth.drift_pair(g, B * N, d, (B * N) // 3, 0.1)
    x0 = [dev_bf16(a.reshape(B, N, d)), dev_bf16(bb.reshape(B, N, d))]
    kc = [torch.zeros((B, N, shape.n_heads, shape.head_dim), dtype=torch.bfloat16, device="cuda")
          for _ in range(L)]
    vc = [torch.zeros_like(kc[0]) for _ in range(L)]
    y = [torch.zeros((B, N, d), dtype=torch.bfloat16, device="cuda") for _ in range(L)]
    xprev = [None] + [torch.zeros((B, N, d), dtype=torch.bfloat16, device="cuda") for _ in range(L - 1)]
    ws = torch.empty((layers[0].workspace_bytes(B, N, B * N),), dtype=torch.uint8, device="cuda")
    # dense fill of the chain from x0[0]; the cached inputs of layers >= 1 are copies of the outputs
    X = x0[0]
    for l in range(L):
        stc.dcu_selective_layer(layers[l], X, None, None, kc[l], vc[l], y[l], workspace=ws)
        if l + 1 < L:
            xprev[l + 1].copy_(y[l])
        X = y[l]
    s_prev = None
    keys = dev(np.array([[20, -1], [40, 41]], np.int32))
    slot_pos = dev(np.tile(np.arange(N - MC, N, dtype=np.int32), (B, 1)))
    sel = torch.empty((L, B, N), dtype=torch.int32, device="cuda")
    cnt = torch.empty((L, B), dtype=torch.int32, device="cuda")
    for step in range(3):
        cur, prev0 = x0[(step + 1) % 2], x0[step % 2]
        budgets = stc.dcu_budget(s_prev, B, L, 10)
        s_cur = torch.empty((L, B), dtype=torch.float32, device="cuda")
        X = cur
        for l in range(L):
            if l == 0:
                dist, _ = stc.dcu_distance(cur, prev0, want_mean=False)
                ref_in, ref_prev = host_bf16(cur), host_bf16(prev0)
            else:
                ref_in, ref_prev = host_bf16(y[l - 1]), host_bf16(xprev[l])
                dist = stc.dcu_distance_rows(y[l - 1], xprev[l], sel[l - 1], cnt[l - 1], roll=True)
                # the roll left the cached input equal to this step's input
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
            stc.dcu_select(dist, budgets, l, keys, 8, sel_idx=sel[l], sel_count=cnt[l], mean=s_cur[l])
            rs, rc = osel.select(dh, budgets.cpu().numpy(), l, keys.cpu().numpy(), 8)
            assert np.array_equal(sel[l].cpu().numpy(), rs) and np.array_equal(cnt[l].cpu().numpy(), rc)
            k0, v0, y0 = host_bf16(kc[l]), host_bf16(vc[l]), host_bf16(y[l])
            stc.dcu_selective_layer(layers[l], X, sel[l], cnt[l], kc[l], vc[l], y[l], workspace=ws)
            rk, rv, ry = olayer.selective_layer(ws_host[l], shape.n_heads, shape.head_dim, shape.eps,
                                                ref_in, rs, rc, k0, v0, y0, THETA)
            gy = synth.bf16_to_f32(host_bf16(y[l]))
            for b in range(B):
                r = rs[b, :rc[b]]
                if len(r):
                    assert rel_l2(gy[b, r], ry[b, r]) <= 1e-2
                keep = np.setdiff1d(np.arange(N), r)
                assert np.array_equal(host_bf16(y[l])[b, keep], y0[b, keep])
            X = y[l]
        s_prev = s_cur
        # the commits of this step place the next step's windows
        logits = dev_bf16(synth.planted_logits(g, B * MC, V)[0])
        conf, _ = stc.dllm_confidence(logits, V)
        n, order = stc.frechet_commit(conf.view(B, MC), 0.1)
        keys = stc.dllm_commit_positions(order, n, slot_pos, 2)
        kh, oh, nh = keys.cpu().numpy(), order.cpu().numpy(), n.cpu().numpy()
        for b in range(B):
            k = min(int(nh[b]), 2)
            assert kh[b, :k].tolist() == [N - MC + int(oh[b, j]) for j in range(k)]


def test_full_budget_closed_loop_step_equals_the_oracle_step():
    """A closed-loop step in which every row of the first input moves and the budget covers every
    row: every layer then recomputes all rows (the step equals the dense step), on the GPU chain
    and in the oracle's own step driver (dcu_step, closed loop, rotary layers) alike, so the two
    chains are compared layer by layer: selections of all N rows, outputs within rel-L2 1e-2."""
    g = synth.rng(980, 1)
    shape = synth.LayerShape(d=128, n_heads=2, head_dim=64, ffn=192)
    L, B, N, bw = 3, 2, 64, 8
    d = shape.d
    ws_host = [synth.layer_weights(g, shape, std=0.05, gain_jitter=0.1) for _ in range(L)]
    layers = []
    for w in ws_host:
        t = {k: dev_bf16(v) for k, v in w.items()}
        layers.append(stc.Layer(d, shape.n_heads, shape.head_dim, shape.ffn, shape.eps, t["w_qkv"],
                                t["w_o"], t["w_gate"], t["w_up"], t["w_down"], t["g_attn"], t["g_ffn"],
                                rope_theta=THETA))
    x_prev0 = synth.normal_bf16(g, (B, N, d))
    x1 = synth.f32_to_bf16(synth.bf16_to_f32(x_prev0) +
                           g.standard_normal((B, N, d), dtype=np.float32) * np.float32(0.1))
    kc = [torch.zeros((B, N, shape.n_heads, shape.head_dim), dtype=torch.bfloat16, device="cuda")
          for _ in range(L)]
    vc = [torch.zeros_like(kc[0]) for _ in range(L)]
    y = [torch.zeros((B, N, d), dtype=torch.bfloat16, device="cuda") for _ in range(L)]
    xprev = [dev_bf16(x_prev0)] + [torch.zeros((B, N, d), dtype=torch.bfloat16, device="cuda")
                                   for _ in range(L - 1)]
    X = xprev[0]
    for l in range(L):
        stc.dcu_selective_layer(layers[l], X, None, None, kc[l], vc[l], y[l])
        if l + 1 < L:
            xprev[l + 1].copy_(y[l])
        X = y[l]
    # the oracle's state: the same cached inputs (the GPU's dense chain), its own dense fill
    st = ostep.dense_fill(ws_host, shape.n_heads, shape.head_dim, shape.eps,
                          [host_bf16(t) for t in xprev], THETA)
    keys = np.array([[20, -1], [40, 41]], np.int32)
    rec = ostep.dcu_step(st, ws_host, shape.n_heads, shape.head_dim, shape.eps, N, bw, keys,
                         x0=x1, rope_theta=THETA)
    budgets = stc.dcu_budget(None, B, L, N)
    X = dev_bf16(x1)
    for l in range(L):
        if l == 0:
            dist, _ = stc.dcu_distance(X, xprev[0], want_mean=False)
        else:
            dist = stc.dcu_distance_rows(y[l - 1], xprev[l], sel, cnt, roll=True)
        sel, cnt = stc.dcu_select(dist, budgets, l, dev(keys), bw)
        assert np.all(cnt.cpu().numpy() == N) and np.all(rec[l]["sel_count"] == N)
        stc.dcu_selective_layer(layers[l], X, sel, cnt, kc[l], vc[l], y[l])
        e = rel_l2(synth.bf16_to_f32(host_bf16(y[l])), st.y[l])
        print(f"  layer {l}: rel-L2 against the oracle step {e:.2e}", flush=True)
        assert e <= 1e-2
        X = y[l]
