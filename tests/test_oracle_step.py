"""Pins of the oracle's multi-layer step: the "stuck in the mud" feedback of the Dynamic-dLLM notes
(Key design 2: a token not recomputed at layer l has distance exactly 0 at layer l+1), full budget
reproducing the dense step, identical inputs selecting only the windows, and determinism."""
import numpy as np
import pytest

from oracle import layer as ol
from oracle import step as ostep
from workloads import synth

SH = synth.LayerShape(d=16, n_heads=2, head_dim=8, ffn=24)


def _setup(seed, L=3, B=2, N=24, theta=0.0):
    g = synth.rng(700, seed)
    ws = [synth.layer_weights(g, SH, std=0.2, bf16=False, gain_jitter=0.3) for _ in range(L)]
    x0 = g.standard_normal((B, N, SH.d))
    # closed loop: layer l's cached input is layer l-1's output of the dense pass
    xs = [x0]
    for l in range(L - 1):
        z = np.zeros((B, N, SH.n_heads, SH.head_dim))
        _, _, y = ol.selective_layer(ws[l], SH.n_heads, SH.head_dim, SH.eps, xs[-1], None, None,
                                     z, z.copy(), np.zeros((B, N, SH.d)), theta)
        xs.append(y)
    st = ostep.dense_fill(ws, SH.n_heads, SH.head_dim, SH.eps, xs, theta)
    return g, ws, x0, st


@pytest.mark.parametrize("theta", [0.0, 1e4])
def test_stuck_in_the_mud_closed_loop(theta):
    g, ws, x0, st = _setup(0, theta=theta)
    B, N = x0.shape[:2]
    x1 = x0.copy()
    x1[:, ::3] += 0.05 * g.standard_normal(x1[:, ::3].shape)
    keys = np.array([[5], [17]], np.int32)
    rec = ostep.dcu_step(st, ws, SH.n_heads, SH.head_dim, SH.eps, b_layer=3, b_window=4,
                         key_pos=keys, x0=x1, rope_theta=theta)
    for l in range(1, len(ws)):
        for b in range(B):
            sel = set(rec[l - 1]["sel_idx"][b, :rec[l - 1]["sel_count"][b]].tolist())
            for i in range(N):
                if i not in sel:
                    assert rec[l]["dist"][b, i] == 0.0


@pytest.mark.parametrize("theta", [0.0, 1e4])
def test_full_budget_reproduces_the_dense_step(theta):
    g, ws, x0, st = _setup(1, theta=theta)
    B, N = x0.shape[:2]
    x1 = x0 + 0.1 * g.standard_normal(x0.shape)        # every row moves
    rec = ostep.dcu_step(st, ws, SH.n_heads, SH.head_dim, SH.eps, b_layer=N, b_window=4,
                         key_pos=np.full((B, 1), 3, np.int32), x0=x1, rope_theta=theta)
    x = x1
    for l in range(len(ws)):
        assert np.all(rec[l]["sel_count"] == N)
        z = np.zeros((B, N, SH.n_heads, SH.head_dim))
        _, _, y = ol.selective_layer(ws[l], SH.n_heads, SH.head_dim, SH.eps, x, None, None, z,
                                     z.copy(), np.zeros((B, N, SH.d)), theta)
        np.testing.assert_allclose(st.y[l], y, rtol=1e-12, atol=1e-12)
        x = y


def test_rotary_step_differs_from_the_plain_step_only_through_positions():
    """With rotary embedding the dense-filled caches hold rotated keys; a full-budget step from the
    same inputs then gives the same outputs as a plain step exactly when every position is 0, i.e.
    the rotation enters the step only through the positions (one-row sequences)."""
    g = synth.rng(700, 9)
    ws = [synth.layer_weights(g, SH, std=0.2, bf16=False) for _ in range(2)]
    x0 = g.standard_normal((3, 1, SH.d))
    x1 = x0 + 0.1 * g.standard_normal(x0.shape)
    outs = []
    for theta in (0.0, 1e4):
        xs = [x0]
        z = np.zeros((3, 1, SH.n_heads, SH.head_dim))
        xs.append(ol.selective_layer(ws[0], SH.n_heads, SH.head_dim, SH.eps, x0, None, None, z,
                                     z.copy(), np.zeros((3, 1, SH.d)), theta)[2])
        st = ostep.dense_fill(ws, SH.n_heads, SH.head_dim, SH.eps, xs, theta)
        ostep.dcu_step(st, ws, SH.n_heads, SH.head_dim, SH.eps, b_layer=1, b_window=0,
                       key_pos=np.full((3, 1), -1, np.int32), x0=x1, rope_theta=theta)
        outs.append(st.y)
    for a, b in zip(*outs):
        np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-13)


def test_end_of_step_on_the_pages_profile():
    """end_of_step = confidence then the Frechet commit: logits built so that the confidences are
    the Fast-dLLM++ background profile (0.99, 0.95, 0.82, 0.78, 0.74) (one logit a over V - 1
    zeros gives c = e^a / (e^a + V - 1)) commit 4 positions at delta = 0.30, the most confident
    first, with the argmax at the planted index."""
    V = 1000
    prof = np.array([0.78, 0.99, 0.74, 0.95, 0.82])          # slots in a shuffled order
    logits = np.zeros((5, V))
    idx = np.array([3, 17, 999, 0, 500])
    logits[np.arange(5), idx] = np.log(prof * (V - 1) / (1 - prof))
    conf, tok, n, order = ostep.end_of_step(logits, V, 1, 5, None, 0.30)
    np.testing.assert_allclose(conf, prof, rtol=1e-6)
    assert tok.tolist() == idx.tolist()
    assert n.tolist() == [4]
    assert order[0, :4].tolist() == [1, 3, 4, 0]


def test_identical_inputs_select_only_windows_and_keep_outputs():
    g, ws, x0, st = _setup(2)
    y_before = [y.copy() for y in st.y]
    keys = np.array([[0], [23]], np.int32)
    rec = ostep.dcu_step(st, ws, SH.n_heads, SH.head_dim, SH.eps, b_layer=5, b_window=4,
                         key_pos=keys, x0=x0.copy())
    for l in range(len(ws)):
        assert np.all(rec[l]["dist"] == 0.0)
        assert rec[l]["sel_idx"][0, :rec[l]["sel_count"][0]].tolist() == [0, 1]
        assert rec[l]["sel_idx"][1, :rec[l]["sel_count"][1]].tolist() == [21, 22, 23]
        # recomputing rows whose inputs did not move reproduces the dense values
        np.testing.assert_allclose(st.y[l], y_before[l], rtol=1e-12, atol=1e-12)
    assert np.all(st.s_prev == 0.0)


def test_budgets_follow_previous_means_and_run_is_deterministic():
    def run():
        g, ws, x0, st = _setup(3)
        B = x0.shape[0]
        keys = np.array([[4], [12]], np.int32)
        recs = []
        x = x0
        for step in range(3):
            x = x + 0.02 * (step + 1) * synth.rng(701, step).standard_normal(x.shape)
            recs.append(ostep.dcu_step(st, ws, SH.n_heads, SH.head_dim, SH.eps, b_layer=4,
                                       b_window=2, key_pos=keys, x0=x))
        return recs, st

    r1, s1 = run()
    r2, s2 = run()
    for a, b in zip(r1, r2):
        for la, lb in zip(a, b):
            for k in la:
                assert np.array_equal(la[k], lb[k])
    for ya, yb in zip(s1.y, s2.y):
        assert np.array_equal(ya, yb)
    # step 0 budgets are uniform; later steps sum to b_layer * L per sequence
    assert np.all(r1[0][0]["budgets"] == 4)
    tot = sum(r1[1][l]["budgets"] for l in range(3))
    assert np.all(tot == 12)


def test_tiny_fp32_config_end_to_end():
    """The tiny fp32 workload: 2 layers, N=64, d=64, 2 heads of 32, FFN 128, 25% of rows drifted
    by N(0, (0.05(1+l))^2), B_layer = B_window = 8, key position 40, 4 steps (open loop)."""
    sh = synth.TINY
    L, B, N = 2, 1, 64
    g = synth.rng(1, 0)
    ws = [synth.layer_weights(synth.rng(1, 1, l), sh, bf16=False) for l in range(L)]
    x_prev = [synth.rng(1, 2, l).standard_normal((B, N, sh.d)).astype(np.float32) for l in range(L)]
    st = ostep.dense_fill(ws, sh.n_heads, sh.head_dim, sh.eps, x_prev)
    keys = np.array([[40]], np.int32)
    for step in range(4):
        x_cur = []
        for l in range(L):
            cur, _, _ = synth.drift_pair(synth.rng(1, 3, step, l), N, sh.d, 16, 0.05 * (1 + l),
                                         bf16=False, base=np.asarray(st.x_prev[l][0], np.float32))
            x_cur.append(cur[None])
        rec = ostep.dcu_step(st, ws, sh.n_heads, sh.head_dim, sh.eps, 8, 8, keys, x_cur=x_cur)
        for l in range(L):
            sel = rec[l]["sel_idx"][0, :rec[l]["sel_count"][0]].tolist()
            assert set(range(36, 44)) <= set(sel)
            assert len(sel) == 8 + min(int(rec[l]["budgets"][0]), int(np.sum(rec[l]["dist"][0] > 0)) -
                                        int(np.sum(rec[l]["dist"][0, 36:44] > 0)))
        if step == 0:
            assert np.all(rec[0]["budgets"] == 8)
        else:
            assert sum(int(rec[l]["budgets"][0]) for l in range(L)) == 16
