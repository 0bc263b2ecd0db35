"""Pins of the oracle's selection: top-B by distance outside the forced windows, united with the
windows (Dynamic-dLLM notes, Key designs 1 and 2)."""
import numpy as np

from oracle import select as osel
from workloads import synth


def _brute(dist, budget, keys, bw):
    """Independent brute force: explicit window loops, rank by pairwise comparison."""
    N = len(dist)
    W = set()
    for p in keys:
        if 0 <= p < N and bw > 0:
            start = p - bw // 2
            for i in range(start, start + bw):
                if 0 <= i < N:
                    W.add(i)
    C = [i for i in range(N) if i not in W and dist[i] > 0]
    A = []
    for i in C:
        rank = sum(1 for j in C if dist[j] > dist[i] or (dist[j] == dist[i] and j < i))
        if rank < budget:
            A.append(i)
    return sorted(W | set(A)), W, C


def test_against_brute_force_on_tiny_inputs():
    g = synth.rng(300, 0)
    for trial in range(300):
        N = int(g.integers(1, 40))
        d = g.uniform(0, 1, N).astype(np.float32)
        # plant zeros and ties
        d[g.random(N) < 0.3] = 0.0
        d[g.random(N) < 0.2] = np.float32(0.5)
        keys = g.integers(-3, N + 3, size=int(g.integers(0, 4)))
        bw = int(g.integers(0, 9))
        b = int(g.integers(0, N + 3))
        u = osel.select_row(d, b, keys, bw)
        ref, W, C = _brute(d, b, keys.tolist(), bw)
        assert u.tolist() == ref
        assert W <= set(u.tolist())
        assert len(u) == len(W) + min(b, len(C))


def test_identical_inputs_select_only_the_window():
    d = np.zeros(100, np.float32)
    u = osel.select_row(d, 32, [40], 8)
    assert u.tolist() == list(range(36, 44))


def test_window_holds_exactly_b_window_positions_and_clips():
    N = 64
    d = np.zeros(N, np.float32)
    assert osel.select_row(d, 0, [40], 8).tolist() == list(range(36, 44))
    assert osel.select_row(d, 0, [40], 7).tolist() == list(range(37, 44))
    assert osel.select_row(d, 0, [1], 8).tolist() == list(range(0, 5))
    assert osel.select_row(d, 0, [62], 8).tolist() == list(range(58, 64))
    assert osel.select_row(d, 0, [-1, 64, 99], 8).tolist() == []
    # the page's literal inclusive bracket [p - B/2, p + B/2] holds B + 1 positions
    assert len(osel.select_row(d, 0, [40], 8)) == 8
    assert osel.window_mask([40], N, 8, literal_window=True).sum() == 9


def test_ties_go_to_lower_position_and_zero_distance_never_selected():
    d = np.array([0.0, 0.2, 0.5, 0.5, 0.1, 0.5, 0.0], np.float32)
    assert osel.select_row(d, 2, [], 0).tolist() == [2, 3]
    assert osel.select_row(d, 3, [], 0).tolist() == [2, 3, 5]
    assert osel.select_row(d, 100, [], 0).tolist() == [1, 2, 3, 4, 5]


def test_budget_is_spent_outside_the_window():
    d = np.zeros(50, np.float32)
    d[20:30] = np.linspace(1, 2, 10, dtype=np.float32)   # the largest distances sit in the window
    d[0] = 0.01
    d[49] = 0.02
    u = osel.select_row(d, 2, [25], 10)                   # window [20, 29]
    assert u.tolist() == [0] + list(range(20, 30)) + [49]


def test_batched_form():
    g = synth.rng(300, 1)
    B, N, L = 3, 30, 4
    d = g.uniform(0, 1, (B, N)).astype(np.float32)
    budgets = g.integers(0, 10, (B, L)).astype(np.int32)
    keys = np.array([[5, -1], [29, 0], [-1, -1]], np.int32)
    sel, cnt = osel.select(d, budgets, 2, keys, 4)
    for b in range(B):
        ref = osel.select_row(d[b], budgets[b, 2], keys[b], 4)
        assert sel[b, :cnt[b]].tolist() == ref.tolist()
        assert np.all(sel[b, cnt[b]:] == -1)
