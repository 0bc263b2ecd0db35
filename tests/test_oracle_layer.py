"""Pins of the oracle's selective layer: pure-Python dense loops on tiny shapes, torch library
routines (scaled_dot_product_attention, rms_norm, silu) and closed forms.

What the layer must satisfy comes from the Dynamic-dLLM notes, Key design 1 (only the selected
tokens are recomputed, the rest reuse cached values); that a full selection reproduces the dense
layer is the method's own consistency requirement. The layer internals follow the reading stated in the
oracle's layer module."""
import math

import numpy as np
import pytest
import torch

from oracle import layer as ol
from workloads import synth

S = synth.LayerShape(d=8, n_heads=2, head_dim=4, ffn=6, eps=1e-5)


def _weights(seed, shape=S, std=0.3):
    return synth.layer_weights(synth.rng(400, seed), shape, std=std, bf16=False, gain_jitter=0.5)


def _loops_dense(w, x, shape):
    """Independent dense layer written with explicit Python loops (tiny shapes only)."""
    N, d = len(x), shape.d
    H, dh, F = shape.n_heads, shape.head_dim, shape.ffn

    def mv(Wm, v, rows, cols):
        return [sum(float(Wm[r][c]) * v[c] for c in range(cols)) for r in range(rows)]

    def rms(v, g):
        ms = sum(t * t for t in v) / len(v)
        return [v[i] / math.sqrt(ms + shape.eps) * float(g[i]) for i in range(len(v))]

    xn = [rms([float(t) for t in x[i]], w["g_attn"]) for i in range(N)]
    qkv = [mv(w["w_qkv"], xn[i], 3 * d, d) for i in range(N)]
    out_k = [[qkv[i][d + j] for j in range(d)] for i in range(N)]
    out_v = [[qkv[i][2 * d + j] for j in range(d)] for i in range(N)]
    ys = []
    for i in range(N):
        o = [0.0] * d
        for h in range(H):
            sc = []
            for j in range(N):
                sc.append(sum(qkv[i][h * dh + c] * out_k[j][h * dh + c] for c in range(dh)) / math.sqrt(dh))
            m = max(sc)
            e = [math.exp(t - m) for t in sc]
            z = sum(e)
            for c in range(dh):
                o[h * dh + c] = sum(e[j] / z * out_v[j][h * dh + c] for j in range(N))
        proj = mv(w["w_o"], o, d, d)
        a = [float(x[i][c]) + proj[c] for c in range(d)]
        an = rms(a, w["g_ffn"])
        gt = mv(w["w_gate"], an, F, d)
        up = mv(w["w_up"], an, F, d)
        hdn = [gt[f] / (1 + math.exp(-gt[f])) * up[f] for f in range(F)]
        dn = mv(w["w_down"], hdn, d, F)
        ys.append([a[c] + dn[c] for c in range(d)])
    return np.array(out_k), np.array(out_v), np.array(ys)


def _run(w, x, rows, kc=None, vc=None, y=None, shape=S):
    N = len(x)
    kc = np.zeros((N, shape.n_heads, shape.head_dim)) if kc is None else kc
    vc = np.zeros_like(kc) if vc is None else vc
    y = np.zeros((N, shape.d)) if y is None else y
    return ol.selective_layer_seq(ol.weights64(w), shape.n_heads, shape.head_dim, shape.eps,
                                  np.asarray(x, np.float64), rows, kc, vc, y)


def test_full_selection_matches_independent_python_loops():
    w = _weights(0)
    x = synth.rng(400, 1).standard_normal((5, S.d))
    k, v, y = _run(w, x, np.arange(5))
    rk, rv, ry = _loops_dense(w, x, S)
    np.testing.assert_allclose(k.reshape(5, -1), rk, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(v.reshape(5, -1), rv, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(y, ry, rtol=1e-12, atol=1e-12)


def test_full_selection_matches_torch_library_routines():
    shape = synth.LayerShape(d=32, n_heads=4, head_dim=8, ffn=48)
    w = _weights(2, shape, std=0.2)
    N = 19
    x = synth.rng(400, 3).standard_normal((N, shape.d))
    k, v, y = _run(w, x, np.arange(N), shape=shape)
    tw = {kk: torch.tensor(vv, dtype=torch.float64) for kk, vv in w.items()}
    tx = torch.tensor(x)
    F = torch.nn.functional
    xn = F.rms_norm(tx, (shape.d,), tw["g_attn"], shape.eps)
    q, kk, vv = (xn @ tw["w_qkv"].T).split(shape.d, dim=1)
    heads = lambda t: t.reshape(N, shape.n_heads, shape.head_dim).transpose(0, 1)
    o = F.scaled_dot_product_attention(heads(q), heads(kk), heads(vv))
    a = tx + o.transpose(0, 1).reshape(N, shape.d) @ tw["w_o"].T
    an = F.rms_norm(a, (shape.d,), tw["g_ffn"], shape.eps)
    ry = a + (F.silu(an @ tw["w_gate"].T) * (an @ tw["w_up"].T)) @ tw["w_down"].T
    np.testing.assert_allclose(y, ry.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(k.reshape(N, -1), kk.numpy(), rtol=1e-12, atol=1e-13)


def test_empty_selection_leaves_everything_untouched():
    w = _weights(4)
    g = synth.rng(400, 5)
    x = g.standard_normal((6, S.d))
    kc = g.standard_normal((6, S.n_heads, S.head_dim))
    vc = g.standard_normal((6, S.n_heads, S.head_dim))
    y = g.standard_normal((6, S.d))
    k2, v2, y2 = _run(w, x, np.zeros(0, np.int64), kc, vc, y)
    assert np.array_equal(k2, kc) and np.array_equal(v2, vc) and np.array_equal(y2, y)


def test_unselected_rows_are_bitwise_untouched():
    w = _weights(6)
    g = synth.rng(400, 7)
    x = g.standard_normal((9, S.d))
    kc = g.standard_normal((9, S.n_heads, S.head_dim))
    vc = g.standard_normal((9, S.n_heads, S.head_dim))
    y = g.standard_normal((9, S.d))
    rows = np.array([1, 4, 8])
    k2, v2, y2 = _run(w, x, rows, kc, vc, y)
    keep = np.setdiff1d(np.arange(9), rows)
    assert np.array_equal(k2[keep], kc[keep]) and np.array_equal(y2[keep], y[keep])
    assert not np.allclose(y2[rows], y[rows])


def test_selected_rows_equal_dense_when_all_changed_rows_are_selected():
    w = _weights(8)
    g = synth.rng(400, 9)
    x_prev = g.standard_normal((10, S.d))
    k0, v0, y0 = _run(w, x_prev, np.arange(10))            # dense fill on the cached inputs
    x_cur = x_prev.copy()
    changed = np.array([2, 7])
    x_cur[changed] += 0.5 * g.standard_normal((2, S.d))
    rows = np.array([0, 2, 5, 7])                           # a superset of the changed rows
    k1, v1, y1 = _run(w, x_cur, rows, k0, v0, y0)
    kd, vd, yd = _run(w, x_cur, np.arange(10))              # dense on the current inputs
    np.testing.assert_allclose(y1[rows], yd[rows], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(k1, kd, rtol=1e-12, atol=1e-12)


def test_all_equal_keys_average_the_values_and_zero_ffn_is_identity():
    shape = S
    w = _weights(10)
    w["w_qkv"][shape.d:2 * shape.d] = 0.0                    # every key is 0: uniform attention
    w["w_down"][:] = 0.0                                     # FFN contributes nothing: y = a
    g = synth.rng(400, 11)
    x = g.standard_normal((7, shape.d))
    k, v, y = _run(w, x, np.arange(7))
    mean_v = v.reshape(7, -1).mean(axis=0)
    a = x + mean_v @ np.asarray(w["w_o"], np.float64).T
    np.testing.assert_allclose(y, a, rtol=1e-12, atol=1e-12)


def test_single_key_attention_returns_its_value():
    w = _weights(12)
    w["w_down"][:] = 0.0
    x = synth.rng(400, 13).standard_normal((1, S.d))
    k, v, y = _run(w, x, np.arange(1))
    a = x + v.reshape(1, -1) @ np.asarray(w["w_o"], np.float64).T
    np.testing.assert_allclose(y, a, rtol=1e-12, atol=1e-12)


def test_batched_form_and_bf16_inputs():
    shape = synth.TINY
    g = synth.rng(400, 14)
    w = synth.layer_weights(g, shape)
    x = synth.normal_bf16(g, (2, 12, shape.d))
    sel = np.full((2, 12), -1, np.int32)
    sel[0, :3] = [0, 5, 11]
    sel[1, :1] = [4]
    cnt = np.array([3, 1], np.int32)
    kc = np.zeros((2, 12, shape.n_heads, shape.head_dim))
    k, v, y = ol.selective_layer(w, shape.n_heads, shape.head_dim, shape.eps, x, sel, cnt, kc,
                                 kc.copy(), np.zeros((2, 12, shape.d)))
    for b in range(2):
        rows = sel[b, :cnt[b]]
        rk, rv, ry = ol.selective_layer_seq(ol.weights64(w), shape.n_heads, shape.head_dim,
                                            shape.eps, ol.as64(x[b]), rows, kc[b], kc[b].copy(),
                                            np.zeros((12, shape.d)))
        assert np.array_equal(y[b], ry)


def test_v_features_closed_form():
    """With the V block of W_qkv the identity, unit gains and eps = 0, the Value vectors are the
    RMS-normalised inputs: unit mean square and proportional to x row by row."""
    g = np.random.default_rng(12)
    d, B, N = 64, 2, 9
    x = g.normal(0, 3, (B, N, d)).astype(np.float32)
    w = {"w_qkv": np.zeros((3 * d, d), np.float32), "w_o": np.zeros((d, d), np.float32),
         "g_attn": np.ones(d, np.float32)}
    w["w_qkv"][2 * d:] = np.eye(d, dtype=np.float32)
    w["w_qkv"][:d] = 5.0                                     # the Q and K rows must not leak in
    v = ol.v_features(w, 0.0, x)
    assert np.allclose(np.mean(v * v, axis=-1), 1.0, rtol=1e-12)
    ratio = v / x
    assert np.allclose(ratio, ratio[..., :1], rtol=1e-12)
