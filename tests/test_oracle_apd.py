"""Pins of the oracle's adaptive-parallel-decoding signals and threshold rule (Dynamic-dLLM notes,
Key design 3): closed forms worked by hand, softmax invariances, and the unmask rule by brute force."""
import math

import numpy as np
import pytest

from oracle import apd


def test_two_token_worked_example():
    # z = (0, ln 3): p = (1/4, 3/4), u = 1, c = 1 - 1/4; previous z = (ln 3, 0): q = (3/4, 1/4),
    # cos = (3/16 + 3/16) / (10/16) = 3/5, H = 2/5; tau = 0.9 - 0.1 * 0.75 + 0.2 * 0.4 = 0.905
    z = np.array([[0.0, math.log(3.0)]], np.float32)
    zp = np.array([[math.log(3.0), 0.0]], np.float32)
    pmax, tok, c, H = apd.signals(z, zp)
    assert tok[0] == 1
    assert pmax[0] == pytest.approx(0.75, rel=1e-6)
    assert c[0] == pytest.approx(0.75, rel=1e-6)
    assert H[0] == pytest.approx(0.4, rel=1e-6)
    tau = apd.update_threshold(np.array([0.9]), c, H, 0.1, 0.2)
    assert tau[0] == pytest.approx(0.905, rel=1e-6)


def test_single_entry_uniform_and_top_ties():
    pmax, tok, c, H = apd.signals(np.array([[2.5]], np.float32), None)
    assert pmax[0] == 1.0 and c[0] == 1.0 and H[0] == 0.0 and tok[0] == 0
    z = np.zeros((1, 4), np.float32)
    pmax, tok, c, H = apd.signals(z, z)
    assert tok[0] == 0 and pmax[0] == pytest.approx(0.25) and c[0] == pytest.approx(0.75)
    assert abs(H[0]) < 1e-15
    # a tie at the top: the runner-up probability equals the top one
    z = np.array([[1.0, 3.0, 3.0, 0.0]], np.float32)
    pmax, tok, c, _ = apd.signals(z, None)
    assert tok[0] == 1 and c[0] == pytest.approx(1.0 - pmax[0], rel=1e-12)


def test_instability_invariances():
    g = np.random.default_rng(3)
    z = g.normal(0, 2, (5, 300)).astype(np.float32)
    zp = g.normal(0, 2, (5, 300)).astype(np.float32)
    _, _, _, H = apd.signals(z, zp)
    _, _, _, Hs = apd.signals(z + np.float32(7.0), zp - np.float32(3.0))   # softmax shift
    _, _, _, Hr = apd.signals(zp, z)                                        # symmetry
    _, _, _, H0 = apd.signals(z, z)
    assert np.allclose(H, Hs, atol=1e-6) and np.allclose(H, Hr, atol=1e-12)
    assert np.all(np.abs(H0) < 1e-12)
    assert np.all((H > 0) & (H < 1))
    # two sharp peaks on different tokens are nearly orthogonal distributions
    a = np.full((1, 50), -30.0, np.float32)
    b = a.copy()
    a[0, 3] = 30.0
    b[0, 40] = 30.0
    _, _, _, Hd = apd.signals(a, b)
    assert Hd[0] > 1 - 1e-12
    # c = 1 - second-largest probability, by brute force on the explicit distribution
    p = apd.softmax64(z)
    _, _, c, _ = apd.signals(z, None)
    assert np.allclose(c, 1 - np.sort(p, axis=1)[:, -2], rtol=0, atol=1e-15)


def test_threshold_update_is_the_linear_rule():
    g = np.random.default_rng(4)
    tau, c, H = g.uniform(0.5, 1, 9), g.uniform(0, 1, 9), g.uniform(0, 1, 9)
    for a, b in [(0.0, 0.0), (0.1, 0.05), (0.3, 1.0)]:
        assert np.allclose(apd.update_threshold(tau, c, H, a, b), tau - a * c + b * H, rtol=0,
                           atol=1e-15)


def test_unmask_rule_brute_force():
    g = np.random.default_rng(6)
    for trial in range(100):
        B, m = 3, int(g.integers(1, 20))
        conf = g.uniform(0, 1, (B, m)).astype(np.float32)
        if trial % 4 == 0:
            conf[:, ::2] = conf[0, 0]                                   # ties
        tau = g.uniform(0.3, 1.0, (B, m)).astype(np.float32)
        mv = g.integers(0, m + 1, B).astype(np.int32)
        n, order = apd.unmask(conf, tau, mv)
        for b in range(B):
            k = int(mv[b])
            if k == 0:
                assert n[b] == 0 and np.all(order[b] == -1)
                continue
            passed = [i for i in range(k) if float(conf[b, i]) >= float(tau[b, i])]
            if passed:
                assert n[b] == len(passed) and sorted(order[b, :n[b]].tolist()) == passed
            else:
                best = max(range(k), key=lambda i: (float(conf[b, i]), -i))
                assert n[b] == 1 and order[b, 0] == best
            # each group in (conf desc, slot asc) order, and the order is a permutation
            assert sorted(order[b, :k].tolist()) == list(range(k)) and np.all(order[b, k:] == -1)
            for grp in (order[b, :len(passed)], order[b, len(passed):k]):
                keys = [(-float(conf[b, i]), int(i)) for i in grp]
                assert keys == sorted(keys)
