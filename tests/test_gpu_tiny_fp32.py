"""The tiny fp32 workload end to end on the GPU: 2 layers, N = 64, d = 64 (2 heads of 32, FFN 128),
25% of the rows drifted per step by N(0, (0.05(1+l))^2), B_layer = B_window = 8, key position 40,
four open-loop steps with budgets from the previous step's means, then confidence over 16 candidate
rows of a 1000-entry vocabulary and the Frechet commit (delta = 0.1).

Distance, means, budgets, selection, confidence and commit run in fp32 on the GPU; the layer runs on
the bf16-rounded inputs. Each step is checked against the oracle: distances within fp32 rounding,
budgets and selections bit for bit (the oracle's integer steps take the GPU's fp32 distances and
means, so both sides decide in the same precision), layer outputs to rel-L2 1e-2, confidence and
commit as in the kernel tests."""
import numpy as np
import pytest
import torch

import selective_token_cache_amd as stc
from oracle import budget as obud
from oracle import confidence as oconf
from oracle import distance as odist
from oracle import frechet as ofre
from oracle import layer as olayer
from oracle import select as osel
from tests.util import dev, dev_bf16, host_bf16, rel_l2
from workloads import synth

pytestmark = pytest.mark.gpu


def test_tiny_fp32_workload_four_steps():
    sh = synth.TINY
    L, B, N, MC, V = 2, 1, 64, 16, 1000
    ws = [synth.layer_weights(synth.rng(1, 1, l), sh) for l in range(L)]
    layers = []
    for w in ws:
        t = {k: dev_bf16(v) for k, v in w.items()}
        layers.append(stc.Layer(sh.d, sh.n_heads, sh.head_dim, sh.ffn, sh.eps, t["w_qkv"], t["w_o"],
                                t["w_gate"], t["w_up"], t["w_down"], t["g_attn"], t["g_ffn"]))
    x_prev = [synth.rng(1, 2, l).standard_normal((B, N, sh.d)).astype(np.float32) for l in range(L)]
    # dense fill of the caches from the cached inputs (bf16-rounded for the layer)
    kc = [torch.zeros((B, N, sh.n_heads, sh.head_dim), dtype=torch.bfloat16, device="cuda")
          for _ in range(L)]
    vc = [torch.zeros_like(kc[0]) for _ in range(L)]
    y = [torch.zeros((B, N, sh.d), dtype=torch.bfloat16, device="cuda") for _ in range(L)]
    for l in range(L):
        stc.dcu_selective_layer(layers[l], dev_bf16(synth.f32_to_bf16(x_prev[l])), None, None,
                                kc[l], vc[l], y[l])
    keys = np.array([[40]], np.int32)
    s_prev = None
    for step in range(4):
        budgets = stc.dcu_budget(s_prev, B, L, 8)
        ref_bud = obud.layer_budget(None if s_prev is None else s_prev.cpu().numpy().T.copy(), B, L, 8)
        assert np.array_equal(budgets.cpu().numpy(), ref_bud)
        s_cur = torch.empty((L, B), dtype=torch.float32, device="cuda")
        for l in range(L):
            cur, _, _ = synth.drift_pair(synth.rng(1, 3, step, l), N, sh.d, 16, 0.05 * (1 + l),
                                         bf16=False, base=x_prev[l][0])
            cur = cur[None].astype(np.float32)
            dist, mean = stc.dcu_distance(dev(cur), dev(x_prev[l]))
            rd, rm = odist.distance_and_mean(cur, x_prev[l])
            dh = dist.cpu().numpy()
            assert np.allclose(dh, rd, rtol=1e-5, atol=1e-7)
            assert np.allclose(mean.cpu().numpy(), rm, rtol=1e-5)
            s_cur[l] = mean
            sel, cnt = stc.dcu_select(dist, budgets, l, dev(keys), 8)
            rs, rc = osel.select(dh, budgets.cpu().numpy(), l, keys, 8)
            assert np.array_equal(sel.cpu().numpy(), rs) and np.array_equal(cnt.cpu().numpy(), rc)
            assert set(range(36, 44)) <= set(rs[0, :rc[0]].tolist())
            xb = synth.f32_to_bf16(cur)
            k0, v0, y0 = host_bf16(kc[l]), host_bf16(vc[l]), host_bf16(y[l])
            stc.dcu_selective_layer(layers[l], dev_bf16(xb), sel, cnt, kc[l], vc[l], y[l])
            _, _, ry = olayer.selective_layer(ws[l], sh.n_heads, sh.head_dim, sh.eps, xb, rs, rc,
                                              k0, v0, y0)
            r = rs[0, :rc[0]]
            gy = synth.bf16_to_f32(host_bf16(y[l]))
            assert rel_l2(gy[0, r], ry[0, r]) <= 1e-2
            keep = np.setdiff1d(np.arange(N), r)
            assert np.array_equal(host_bf16(y[l])[0, keep], y0[0, keep])
            x_prev[l] = cur  # the cache roll
        s_prev = s_cur
        # end of step in fp32
        z, _ = synth.planted_logits(synth.rng(1, 4, step), B * MC, V)
        zf = synth.bf16_to_f32(z)
        conf, tok = stc.dllm_confidence(dev(zf), V)
        rcf, rt = oconf.confidence64(zf, V)
        assert np.array_equal(tok.cpu().numpy(), rt)
        assert np.all(np.abs(conf.cpu().numpy() - rcf) <= 1e-5 * rcf)
        n, order = stc.frechet_commit(conf.view(B, MC), 0.1)
        rn, ro = ofre.frechet_commit(conf.cpu().numpy().reshape(B, MC), None, 0.1)
        assert np.array_equal(n.cpu().numpy(), rn) and np.array_equal(order.cpu().numpy(), ro)
