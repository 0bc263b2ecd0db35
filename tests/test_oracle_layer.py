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


def _loops_dense(w, x, shape, theta=0.0):
    """Independent dense layer written with explicit Python loops (tiny shapes only); theta > 0
    turns each head's (i, i + dh/2) pair of q and k at row p by p * theta^(-2i/dh) radians."""
    N, d = len(x), shape.d
    H, dh, F = shape.n_heads, shape.head_dim, shape.ffn

    def mv(Wm, v, rows, cols):
        return [sum(float(Wm[r][c]) * v[c] for c in range(cols)) for r in range(rows)]

    def rms(v, g):
        ms = sum(t * t for t in v) / len(v)
        return [v[i] / math.sqrt(ms + shape.eps) * float(g[i]) for i in range(len(v))]

    xn = [rms([float(t) for t in x[i]], w["g_attn"]) for i in range(N)]
    qkv = [mv(w["w_qkv"], xn[i], 3 * d, d) for i in range(N)]
    if theta > 0:
        for p in range(N):
            for base in [h * dh for h in range(2 * H)]:           # the Q heads, then the K heads
                for i in range(dh // 2):
                    ang = p * theta ** (-2.0 * i / dh)
                    a, b = qkv[p][base + i], qkv[p][base + i + dh // 2]
                    qkv[p][base + i] = a * math.cos(ang) - b * math.sin(ang)
                    qkv[p][base + i + dh // 2] = b * math.cos(ang) + a * math.sin(ang)
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


def _run(w, x, rows, kc=None, vc=None, y=None, shape=S, theta=0.0):
    N = len(x)
    kc = np.zeros((N, shape.n_heads, shape.head_dim)) if kc is None else kc
    vc = np.zeros_like(kc) if vc is None else vc
    y = np.zeros((N, shape.d)) if y is None else y
    return ol.selective_layer_seq(ol.weights64(w), shape.n_heads, shape.head_dim, shape.eps,
                                  np.asarray(x, np.float64), rows, kc, vc, y, theta)


@pytest.mark.parametrize("theta", [0.0, 10.0])
def test_full_selection_matches_independent_python_loops(theta):
    w = _weights(0)
    x = synth.rng(400, 1).standard_normal((5, S.d))
    k, v, y = _run(w, x, np.arange(5), theta=theta)
    rk, rv, ry = _loops_dense(w, x, S, theta)
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


@pytest.mark.parametrize("theta", [0.0, 100.0])
def test_selected_rows_equal_dense_when_all_changed_rows_are_selected(theta):
    """With RoPE this also fixes the position of a selected row: its row index, not its slot."""
    w = _weights(8)
    g = synth.rng(400, 9)
    x_prev = g.standard_normal((10, S.d))
    k0, v0, y0 = _run(w, x_prev, np.arange(10), theta=theta)   # dense fill on the cached inputs
    x_cur = x_prev.copy()
    changed = np.array([2, 7])
    x_cur[changed] += 0.5 * g.standard_normal((2, S.d))
    rows = np.array([0, 2, 5, 7])                           # a superset of the changed rows
    k1, v1, y1 = _run(w, x_cur, rows, k0, v0, y0, theta=theta)
    kd, vd, yd = _run(w, x_cur, np.arange(10), theta=theta)    # dense on the current inputs
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


# --- rotary position embedding (RoFormer's rotation; rotate-half pairing of LLaMA-family models)

def test_rope_position_zero_is_the_identity():
    x = synth.rng(400, 20).standard_normal((3, 16))
    assert np.array_equal(ol.rope(x, np.zeros(3), 10000.0), x)


def test_rope_two_dims_is_a_plane_rotation_by_the_position():
    """dh = 2: the only frequency is theta^0 = 1, so (a, b) turns by pos radians whatever theta:
    the complex product (a + ib) e^{i pos}."""
    g = synth.rng(400, 21)
    x = g.standard_normal((7, 2))
    pos = np.arange(7) * 3.0
    for theta in (10.0, 5e5):
        z = (x[:, 0] + 1j * x[:, 1]) * np.exp(1j * pos)
        np.testing.assert_allclose(ol.rope(x, pos, theta), np.stack([z.real, z.imag], 1),
                                   rtol=1e-13, atol=1e-13)


def test_rope_frequencies_and_pairing_on_unit_vectors():
    """dh = 4, theta = 10000: frequencies 1 and 10000^(-1/2) = 0.01; e_1 at position p lands on
    cos(0.01 p) e_1 + sin(0.01 p) e_3 (dims 1 and 3 are a pair), e_0 on cos p e_0 + sin p e_2."""
    p = 37.0
    e = np.eye(4)
    r = ol.rope(e, np.full(4, p), 10000.0)
    np.testing.assert_allclose(r[0], [math.cos(p), 0, math.sin(p), 0], atol=1e-14)
    np.testing.assert_allclose(r[1], [0, math.cos(0.01 * p), 0, math.sin(0.01 * p)], atol=1e-14)
    np.testing.assert_allclose(r[2], [-math.sin(p), 0, math.cos(p), 0], atol=1e-14)
    np.testing.assert_allclose(r[3], [0, -math.sin(0.01 * p), 0, math.cos(0.01 * p)], atol=1e-14)


def test_rope_keeps_norms_and_scores_depend_on_the_offset_only():
    """A rotation keeps every pair's length, and <R(m) q, R(n) k> is a function of m - n."""
    g = synth.rng(400, 22)
    q, k = g.standard_normal((2, 128))
    theta = 5e5
    rq = ol.rope(q[None], np.array([5.0]), theta)[0]
    np.testing.assert_allclose(np.hypot(rq[:64], rq[64:]), np.hypot(q[:64], q[64:]), rtol=1e-13)
    def score(m, n):
        return ol.rope(q[None], np.array([m]), theta)[0] @ ol.rope(k[None], np.array([n]), theta)[0]
    for m, n, s in [(3.0, 10.0, 1000.0), (900.0, 17.0, 2500.0)]:
        np.testing.assert_allclose(score(m + s, n + s), score(m, n), rtol=1e-9, atol=1e-10)
    assert abs(score(3.0, 10.0) - score(10.0, 3.0)) > 1e-6     # not symmetric: order matters


def test_rope_layer_rotates_cached_keys_by_row_position_and_leaves_values():
    w = _weights(30)
    g = synth.rng(400, 31)
    x = g.standard_normal((9, S.d))
    rows = np.array([1, 6, 8])
    k0, v0, _ = _run(w, x, rows)
    k1, v1, _ = _run(w, x, rows, theta=50.0)
    assert np.array_equal(v1, v0)
    np.testing.assert_allclose(k1[rows], ol.rope(k0[rows], rows[:, None].astype(float), 50.0),
                               rtol=1e-13, atol=1e-14)
    assert not np.allclose(k1[rows[1:]], k0[rows[1:]])


# --- attention context of every row (DyLLM-style feature)

def test_attention_context_matches_torch_attention():
    """Against torch's scaled_dot_product_attention on the same q (RMSNorm + W_q) and caches."""
    shape = synth.LayerShape(d=32, n_heads=4, head_dim=8, ffn=48)
    w = _weights(40, shape, std=0.3)
    g = synth.rng(400, 41)
    B, N = 2, 11
    x = g.standard_normal((B, N, shape.d))
    kc = g.standard_normal((B, N, shape.n_heads, shape.head_dim))
    vc = g.standard_normal((B, N, shape.n_heads, shape.head_dim))
    got = ol.attention_context(w, shape.n_heads, shape.head_dim, shape.eps, x, kc, vc)
    F = torch.nn.functional
    tw = {k: torch.tensor(v, dtype=torch.float64) for k, v in w.items()}
    for b in range(B):
        xn = F.rms_norm(torch.tensor(x[b]), (shape.d,), tw["g_attn"], shape.eps)
        q = (xn @ tw["w_qkv"][:shape.d].T).reshape(N, shape.n_heads, shape.head_dim).transpose(0, 1)
        k = torch.tensor(kc[b]).transpose(0, 1)
        v = torch.tensor(vc[b]).transpose(0, 1)
        ref = F.scaled_dot_product_attention(q, k, v).transpose(0, 1).reshape(N, shape.d)
        np.testing.assert_allclose(got[b], ref.numpy(), rtol=1e-11, atol=1e-12)


def test_attention_context_closed_forms():
    """One cached row: every context is that row's value; zero query weights: uniform attention,
    the mean of the values; rotary embedding at N = 1 changes nothing (position 0)."""
    w = _weights(42)
    g = synth.rng(400, 43)
    x = g.standard_normal((1, 1, S.d))
    kc = g.standard_normal((1, 1, S.n_heads, S.head_dim))
    vc = g.standard_normal((1, 1, S.n_heads, S.head_dim))
    c = ol.attention_context(w, S.n_heads, S.head_dim, S.eps, x, kc, vc)
    np.testing.assert_allclose(c.reshape(-1), vc.reshape(-1), rtol=1e-14)
    c2 = ol.attention_context(w, S.n_heads, S.head_dim, S.eps, x, kc, vc, rope_theta=100.0)
    np.testing.assert_allclose(c2, c, rtol=1e-14)
    w0 = dict(w)
    w0["w_qkv"] = np.array(w["w_qkv"], copy=True)
    w0["w_qkv"][:S.d] = 0.0
    N = 7
    x = g.standard_normal((1, N, S.d))
    kc = g.standard_normal((1, N, S.n_heads, S.head_dim))
    vc = g.standard_normal((1, N, S.n_heads, S.head_dim))
    c = ol.attention_context(w0, S.n_heads, S.head_dim, S.eps, x, kc, vc, rope_theta=100.0)
    np.testing.assert_allclose(c[0], np.broadcast_to(vc[0].mean(axis=0).reshape(-1), (N, S.d)),
                               rtol=1e-12, atol=1e-13)
