"""Pins of the oracle's Frechet commit rule (Fast-dLLM++ notes, Key designs 1-3): the pages' worked
profile, exact-rational identities of Proposition 4.3 / Corollary 4.4, and Theorem 4.1 by brute
force over tiny joint distributions."""
import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import frechet as of
from workloads import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "frechet_profile_example.json")


def _exact_scores(c):
    """Exact rationals of the fp32 profile, sorted descending: (L, U, G, F, B) lists."""
    cs = sorted((Fraction(float(np.float32(v))) for v in c), reverse=True)
    out = []
    S = Fraction(0)
    for i, cn in enumerate(cs):
        n = i + 1
        S += cn
        L = max(Fraction(0), S - (n - 1))
        U = 1 - cn
        F = (n + 1) * cn - n
        B = sum((cj - cn for cj in cs[:i]), Fraction(0))
        out.append((L, U, L - U, F, B))
    return out


def test_page_worked_example():
    ex = json.load(open(GOLDEN))
    c = np.array(ex["profile"], np.float32)
    # Figure 1's claim: Frechet accepts 4 where the matched factor rule accepts 2. With this profile
    # that holds for delta in [0.28, 0.32); at the default delta = 0.25 the factor rule accepts 3.
    n, order = of.commit_count(c, 0.30)
    assert n == ex["figure1_frechet_n"]
    assert of.factor_count(c, 0.30) == ex["figure1_matched_factor_n"]
    assert order.tolist() == [0, 1, 2, 3, 4]
    n, _ = of.commit_count(c, ex["default_delta"])
    assert n == 4
    assert of.factor_count(c, ex["default_delta"]) == 3
    # the factor surrogate flattens the top-3 profile to c_(3)
    assert [float(np.float32(c[2]))] * 3 == pytest.approx(ex["flattened_factor_proxy_for_n3"], rel=1e-7)


def test_margin_is_frechet_minus_competitor_bound():
    c = np.array([0.99, 0.95, 0.82, 0.78, 0.74], np.float32)
    order, cs = of.sort_profile(c)
    L, U, G = of.margins(cs)
    ex = _exact_scores(c)
    for i in range(5):
        assert Fraction(L[i]) == ex[i][0]
        assert Fraction(U[i]) == ex[i][1]
        assert Fraction(G[i]) == ex[i][2]


def test_decomposition_identity_exact():
    g = synth.rng(600, 0)
    for trial in range(200):
        m = int(g.integers(1, 30))
        c = g.uniform(0.5, 1.0, m).astype(np.float32)
        for (L, U, G, F, B) in _exact_scores(c):
            if L > 0:
                assert G - F == B             # Proposition 4.3, exactly
            assert B >= 0


def test_invariants_on_random_profiles():
    g = synth.rng(600, 1)
    for trial in range(500):
        m = int(g.integers(1, 40))
        c = g.uniform(float(g.uniform(0, 0.9)), 1.0, m).astype(np.float32)
        delta = float(g.choice([0.0, 0.05, 0.1, 0.25, 0.4]))
        n, order = of.commit_count(c, delta)
        nf = of.factor_count(c, delta)
        _, cs = of.sort_profile(c)
        _, _, G = of.margins(cs)
        assert np.all(np.diff(G) <= 0)                 # G_n is non-increasing
        assert n >= nf                                  # never fewer than the matched factor rule
        assert 1 <= n <= m
        ex = _exact_scores(c)
        # Corollary 4.4: strictly more at n exactly when F_n <= delta < F_n + B_n (with L_n > 0)
        if n > nf:
            L, U, Gx, F, B = ex[n - 1]
            assert F <= Fraction(delta) < F + B
        # the exact rational rule gives the same count
        okx = [i + 1 for i, e in enumerate(ex) if e[2] > Fraction(delta)]
        assert n == (okx[-1] if okx else 1)
        assert sorted(order.tolist()) == list(range(m))


def test_homogeneous_profile_reduces_to_factor_rule():
    for cval in [0.6, 0.8, 0.9, 0.97, 0.999]:
        for m in [1, 3, 10]:
            c = np.full(m, cval, np.float32)
            for delta in [0.0, 0.1, 0.25]:
                assert of.commit_count(c, delta)[0] == of.factor_count(c, delta)


def test_fallback_empty_and_negative_delta():
    c = np.array([0.55, 0.3, 0.1], np.float32)     # G_1 = 2*0.55 - 1 = 0.1 <= 0.25
    assert of.commit_count(c, 0.25)[0] == 1
    assert of.commit_count(np.zeros(0, np.float32), 0.25)[0] == 0
    with pytest.raises(ValueError):
        of.commit_count(c, -0.1)


def test_ties_order_by_slot():
    c = np.array([0.5, 0.9, 0.5, 0.9, 0.7], np.float32)
    order, _ = of.sort_profile(c)
    assert order.tolist() == [1, 3, 4, 0, 2]


def test_sequential_fp64_prefix_sums_are_exact_under_the_precondition():
    g = synth.rng(600, 2)
    c = g.uniform(2.0 ** -17, 1.0, 8192).astype(np.float32)
    c[::7] = np.float32(2.0 ** -17)
    _, cs = of.sort_profile(c)
    S = np.cumsum(cs)
    exact = Fraction(0)
    for i in range(0, 8192):
        exact += Fraction(float(cs[i]))
        if i % 97 == 0 or i == 8191:
            assert Fraction(float(S[i])) == exact


def test_batched_form_with_valid_counts():
    g = synth.rng(600, 3)
    c = g.uniform(0.3, 1, (3, 10)).astype(np.float32)
    n, order = of.frechet_commit(c, np.array([10, 4, 0]), 0.1)
    assert n[2] == 0 and np.all(order[2] == -1)
    assert n[1] == of.commit_count(c[1, :4], 0.1)[0]
    assert np.all(order[1, 4:] == -1)


def test_theorem_4_1_brute_force_on_tiny_joint_distributions():
    """Wherever G_n > 0 for the top-n positions, their marginal-argmax tuple is the unique mode of
    the joint distribution of those positions."""
    g = synth.rng(600, 4)
    certified = 0
    for trial in range(3000):
        npos = int(g.integers(2, 4))
        nsym = int(g.integers(2, 4))
        shape = (nsym,) * npos
        # concentrated random joint: a dominant tuple plus Dirichlet noise
        P = g.dirichlet(np.full(np.prod(shape), 0.3)).reshape(shape)
        top = tuple(int(t) for t in g.integers(0, nsym, npos))
        P = (1 - float(g.uniform(0, 0.9))) * P
        P[top] += 1 - P.sum()
        marg = [P.sum(axis=tuple(a for a in range(npos) if a != i)) for i in range(npos)]
        xstar = [int(np.argmax(mg)) for mg in marg]
        conf = np.array([mg.max() for mg in marg])
        order = np.argsort(-conf, kind="stable")
        for n in range(1, npos + 1):
            S = [int(i) for i in order[:n]]
            cs = conf[S]
            L = max(0.0, cs.sum() - (n - 1))
            U = 1 - cs.min()
            if L - U > 1e-12:
                certified += 1
                other = tuple(a for a in range(npos) if a not in S)
                PS = P.sum(axis=other) if other else P
                # PS axes follow ascending position order
                key = tuple(xstar[i] for i in sorted(S))
                best = PS[key]
                for t in itertools.product(range(nsym), repeat=n):
                    if t != key:
                        assert PS[t] < best
                assert best >= L - 1e-12
    assert certified > 500


# --- the comparison rules (Fast-dLLM threshold and factor rules; the page's motivation section) ----
def test_threshold_and_factor_rules_on_the_page_profile():
    c = np.array([0.99, 0.95, 0.82, 0.78, 0.74], np.float32)
    # threshold: every candidate with c >= tau (inclusive), at least one
    assert of.threshold_commit_count(c, 0.9) == 2
    assert of.threshold_commit_count(c, float(np.float32(0.82))) == 3
    assert of.threshold_commit_count(c, 0.999) == 1
    assert of.threshold_commit_count(c, 0.0) == 5
    # factor f = 0.75 (the matched factor of delta = 0.25): 2*0.01, 3*0.05, 4*0.18 < 0.75 <= 5*0.22,
    # the three candidates the page says the factor rule flattens to c_(3)
    assert of.factor_commit_count(c, 0.75) == 3
    assert of.factor_commit_count(c, 0.0) == 1
    assert of.factor_commit_count(np.zeros(0, np.float32), 0.75) == 0
    assert of.threshold_commit_count(np.zeros(0, np.float32), 0.9) == 0


def test_factor_and_threshold_rules_exact_on_random_profiles():
    g = np.random.default_rng(11)
    for trial in range(200):
        m = int(g.integers(1, 40))
        c = g.uniform(0, 1, m).astype(np.float32)
        if trial % 3 == 0:
            c[g.integers(0, m, m // 2)] = c[0]            # ties
        f = float(Fraction(int(g.integers(0, 2 ** 20)), 2 ** 19))   # dyadic: exact in fp64
        tau = float(np.float32(g.uniform(0, 1)))
        cs = sorted((Fraction(float(v)) for v in c), reverse=True)
        want_f = max([n for n in range(1, m + 1) if (n + 1) * (1 - cs[n - 1]) < Fraction(f)],
                     default=1)
        assert of.factor_commit_count(c, f) == want_f
        k = sum(1 for v in cs if v >= Fraction(tau))
        assert of.threshold_commit_count(c, tau) == max(k, 1)
        # the threshold set is a prefix of the sorted order
        order, srt = of.sort_profile(c)
        assert all(srt[:k] >= tau) and all(srt[k:] < tau)


def test_batched_commit_rules():
    g = np.random.default_rng(5)
    conf = g.uniform(0.3, 1.0, (4, 16)).astype(np.float32)
    mv = np.array([16, 3, 0, 9], np.int32)
    for rule, p in [("frechet", 0.1), ("factor", 0.9), ("threshold", 0.8)]:
        n, order = of.commit(conf, mv, rule, p)
        assert n[2] == 0 and np.all(order[2] == -1)
        assert np.all(order[1, 3:] == -1) and sorted(order[1, :3].tolist()) == [0, 1, 2]
        for b in (0, 1, 3):
            ref = {"frechet": lambda c: of.commit_count(c, p)[0],
                   "factor": lambda c: of.factor_commit_count(c, p),
                   "threshold": lambda c: of.threshold_commit_count(c, p)}[rule](conf[b, :mv[b]])
            assert n[b] == ref
    with pytest.raises(ValueError):
        of.commit(conf, mv, "greedy", 0.1)
