"""A whole DCU step (budget, per-layer distance / select / selective layer, end-of-step confidence
and commit) captured in a HIP graph and replayed: every replay, with eager work and state resets
in between, reproduces the eager step bit for bit (the library only enqueues kernels)."""
import numpy as np
import pytest
import torch

import selective_token_cache_amd as stc
from tests.util import dev, dev_bf16
from workloads import synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B,max_rows", [(2, 0), (1, 64)])
def test_graph_replay_matches_eager_step(B, max_rows):
    """max_rows 0: every row may be selected (the 128-row tile kernels); 64: the single-sequence
    kernels of a row bound of at most 64 (the fused QKV weight stream, the row-workgroup RMSNorm)."""
    g = synth.rng(960, B)
    shape = synth.LayerShape(d=128, n_heads=2, head_dim=64, ffn=192)
    L, N, V, MC = 2, 96, 1000, 16
    max_rows = max_rows or B * N
    layers, kc0, vc0, y0, xc, xp = [], [], [], [], [], []
    for _ in range(L):
        w = synth.layer_weights(g, shape, std=0.05, gain_jitter=0.1)
        t = {k: dev_bf16(v) for k, v in w.items()}
        layers.append(stc.Layer(shape.d, shape.n_heads, shape.head_dim, shape.ffn, shape.eps,
                                t["w_qkv"], t["w_o"], t["w_gate"], t["w_up"], t["w_down"],
                                t["g_attn"], t["g_ffn"], rope_theta=1e4 if B == 1 else 0.0))
        kc0.append(dev_bf16(synth.normal_bf16(g, (B, N, shape.n_heads, shape.head_dim))))
        vc0.append(dev_bf16(synth.normal_bf16(g, (B, N, shape.n_heads, shape.head_dim))))
        y0.append(dev_bf16(synth.normal_bf16(g, (B, N, shape.d))))
        cur, prev, _ = synth.drift_pair(g, N * B, shape.d, N // 3, 0.05)
        xc.append(dev_bf16(cur.reshape(B, N, shape.d)))
        xp.append(dev_bf16(prev.reshape(B, N, shape.d)))
    logits = dev_bf16(synth.planted_logits(g, B * MC, V)[0])
    keys = dev(np.array([[10, 50], [3, 90]][:B], np.int32))
    s_prev = dev(g.uniform(1e-4, 1e-3, (L, B)).astype(np.float32))
    kc = [t.clone() for t in kc0]
    vc = [t.clone() for t in vc0]
    y = [t.clone() for t in y0]
    ws = torch.empty((layers[0].workspace_bytes(B, N, max_rows),), dtype=torch.uint8, device="cuda")
    budgets = torch.empty((B, L), dtype=torch.int32, device="cuda")
    dist = torch.empty((B, N), dtype=torch.float32, device="cuda")
    s_cur = torch.empty((L, B), dtype=torch.float32, device="cuda")
    sel = torch.empty((L, B, N), dtype=torch.int32, device="cuda")
    cnt = torch.empty((L, B), dtype=torch.int32, device="cuda")
    conf = torch.empty((B * MC,), dtype=torch.float32, device="cuda")
    tok = torch.empty((B * MC,), dtype=torch.int32, device="cuda")
    ncom = torch.empty((B,), dtype=torch.int32, device="cuda")
    order = torch.empty((B, MC), dtype=torch.int32, device="cuda")

    def step():
        stc.dcu_budget(s_prev, B, L, 12, out=budgets)
        for l in range(L):
            stc.dcu_distance(xc[l], xp[l], dist=dist, want_mean=False)
            stc.dcu_select(dist, budgets, l, keys, 8, sel_idx=sel[l], sel_count=cnt[l], mean=s_cur[l])
            stc.dcu_selective_layer(layers[l], xc[l], sel[l], cnt[l], kc[l], vc[l], y[l],
                                    max_rows=max_rows, workspace=ws)
        stc.dllm_confidence(logits, V, conf=conf, token=tok)
        stc.frechet_commit(conf.view(B, MC), 0.1, n_commit=ncom, order=order)

    def reset():
        for l in range(L):
            kc[l].copy_(kc0[l])
            vc[l].copy_(vc0[l])
            y[l].copy_(y0[l])

    def snapshot():
        outs = [budgets, s_cur, sel, cnt, conf, tok, ncom, order] + kc + vc + y
        return [t.clone() for t in outs]

    step()
    torch.cuda.synchronize()
    eager = snapshot()
    assert int(cnt.sum()) > 0
    assert int(cnt.sum(dim=1).max()) <= max_rows

    reset()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        reset()
        junk = torch.randn((256, 256), device="cuda") @ torch.randn((256, 256), device="cuda")
        torch.cuda.synchronize()
        for t in (budgets, s_cur, sel, cnt, conf, tok, ncom, order):
            t.zero_()
        graph.replay()
        torch.cuda.synchronize()
        got = snapshot()
        for a, b in zip(eager, got):
            assert torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.uint8) if b.dtype == torch.bfloat16 else b), rep
        del junk
