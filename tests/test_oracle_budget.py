"""Pins of the oracle's per-layer budget (Dynamic-dLLM notes, Key design 1, budget equation:
T = B_layer * LayerNum split in proportion to the previous step's layer means), integerised by
floor plus largest remainder with ties to the lower layer."""
from fractions import Fraction

import numpy as np

from oracle import budget as ob
from workloads import synth


def _hamilton_exact(s, T):
    """Independent exact-rational largest-remainder apportionment (ties to the lower index)."""
    fs = [Fraction(float(np.float32(v))) for v in s]
    S = sum(fs)
    q = [T * v / S for v in fs]
    f = [x.numerator // x.denominator for x in q]
    r = [q[i] - f[i] for i in range(len(s))]
    R = T - sum(f)
    ranked = sorted(range(len(s)), key=lambda i: (-r[i], i))
    b = list(f)
    for i in ranked[:R]:
        b[i] += 1
    return b, r


def test_sum_is_exact_on_random_means():
    g = synth.rng(200, 0)
    for trial in range(300):
        L = int(g.integers(1, 64))
        b_layer = int(g.integers(0, 200))
        s = g.uniform(0, 1e-3, size=L).astype(np.float32)
        b = ob.layer_budget_row(s, L, b_layer)
        assert b.sum() == b_layer * L
        assert np.all(b >= 0)


def test_first_step_and_all_zero_means_are_uniform():
    assert np.array_equal(ob.layer_budget(None, 3, 5, 32), np.full((3, 5), 32))
    z = np.zeros((2, 4), np.float32)
    assert np.array_equal(ob.layer_budget(z, 2, 4, 7), np.full((2, 4), 7))


def test_uniform_one_hot_and_exact_proportions():
    L = 32
    assert np.array_equal(ob.layer_budget_row(np.full(L, 3e-4, np.float32), L, 32), np.full(L, 32))
    oh = np.zeros(L, np.float32)
    oh[7] = 1e-4
    b = ob.layer_budget_row(oh, L, 32)
    assert b[7] == 1024 and b.sum() == 1024
    # means proportional to 1:2:3:2 with T = 8*4 = 32 -> shares 4, 8, 12, 8 exactly
    b = ob.layer_budget_row(np.array([1, 2, 3, 2], np.float32) * np.float32(0.25), 4, 8)
    assert b.tolist() == [4, 8, 12, 8]


def test_tie_goes_to_lower_layer():
    # means (1, 1, 1, 2), T = 2*4 = 8: shares 1.6, 1.6, 1.6, 3.2 -> floors 1, 1, 1, 3 with two units
    # left over and three equal remainders 0.6: layers 0 and 1 get them
    b = ob.layer_budget_row(np.array([1, 1, 1, 2], np.float32), 4, 2)
    assert b.tolist() == [2, 2, 1, 3]
    # means (1, 1, 2), T = 6: shares 1.5, 1.5, 3 -> the single leftover unit goes to layer 0
    b = ob.layer_budget_row(np.array([1, 1, 2], np.float32), 3, 2)
    assert b.tolist() == [2, 1, 3]
    # equal means give exact equal shares
    assert ob.layer_budget_row(np.ones(4, np.float32), 4, 3).tolist() == [3, 3, 3, 3]


def test_agrees_with_exact_rational_apportionment():
    g = synth.rng(200, 1)
    checked = 0
    for trial in range(400):
        L = int(g.integers(2, 40))
        b_layer = int(g.integers(1, 80))
        s = g.uniform(0, 1e-3, size=L).astype(np.float32)
        if trial % 5 == 0:
            s[g.integers(0, L, size=L // 3)] = 0.0
        if s.sum() == 0:
            continue
        ref, r = _hamilton_exact(s, b_layer * L)
        rs = sorted(r, reverse=True)
        # skip only where two exact remainders lie within fp64 resolution of each other
        near_tie = any(abs(float(rs[i] - rs[i + 1])) < 1e-9 for i in range(len(rs) - 1))
        if near_tie:
            continue
        assert ob.layer_budget_row(s, L, b_layer).tolist() == ref
        checked += 1
    assert checked > 300


def test_depth_increasing_means_give_depth_increasing_budgets():
    L = 32
    s = np.array([(1 + l / 8) ** 2 for l in range(L)], np.float32) * np.float32(1e-5)
    b = ob.layer_budget_row(s, L, 32)
    assert b.sum() == 1024
    assert np.all(np.diff(b) >= 0)
    ref, _ = _hamilton_exact(s, 1024)
    assert b.tolist() == ref


def test_batched_rows_are_independent():
    g = synth.rng(200, 2)
    s = g.uniform(0, 1, size=(5, 9)).astype(np.float32)
    b = ob.layer_budget(s, 5, 9, 11)
    for i in range(5):
        assert b[i].tolist() == ob.layer_budget_row(s[i], 9, 11).tolist()


def test_floors_never_overshoot_on_adversarial_means():
    """The floors of q_l = (T s_l) / S never sum past T (the module docstring's bound), so the
    largest-remainder step only ever adds: means spread over the whole fp32 exponent range, long
    runs of equal means, T close to 2^31 and L up to 1024 keep sum(b) == T with every b_l >= 0."""
    g = synth.rng(200, 3)
    for trial in range(200):
        L = int(g.integers(1, 1025)) if trial % 4 else 1024
        b_layer = int(g.integers(1, (2 ** 31 - 1) // L + 1)) if trial % 3 == 0 else int(g.integers(0, 300))
        kind = trial % 5
        if kind == 0:
            s = (2.0 ** g.uniform(-126, 100, size=L)).astype(np.float32)
        elif kind == 1:
            s = np.full(L, np.float32(g.uniform(1e-6, 1.0)))
        elif kind == 2:
            s = g.uniform(0, 2, size=L).astype(np.float32)
            s[g.integers(0, L, size=max(1, L // 2))] = np.float32(1e-45)   # smallest subnormal
        elif kind == 3:
            s = np.nextafter(np.float32(1.0), np.float32(2.0), dtype=np.float32) * np.ones(L, np.float32)
            s[::3] = np.float32(1.0)
        else:
            s = g.uniform(0, 1e-3, size=L).astype(np.float32)
        b = ob.layer_budget_row(s, L, b_layer)
        assert int(b.astype(np.int64).sum()) == b_layer * L
        assert np.all(b >= 0)


def test_negative_means_read_as_zero():
    """Means are averages of distances in [0, 2]; a negative entry counts as 0 (a layer that gets
    no share), and an all-negative row is the all-zero row (uniform budgets)."""
    s = np.array([0.5, -0.25, 1.5, -3.0], np.float32)
    assert ob.layer_budget_row(s, 4, 8).tolist() == ob.layer_budget_row(np.maximum(s, 0), 4, 8).tolist()
    assert ob.layer_budget_row(s, 4, 8).tolist() == [8, 0, 24, 0]
    assert ob.layer_budget_row(-np.ones(3, np.float32), 3, 5).tolist() == [5, 5, 5]
