"""Frechet-profile commit rule (oracle; test infrastructure only).

Follows "Fast-dLLM++: Frechet Profile Decoding" reading notes, Key designs:
* design 1 (Theorem 4.1): for the top-n candidates sorted by confidence c_(1) >= ... >= c_(m), the
  Frechet lower bound L_n = max{0, sum_{j<=n} c_(j) - (n-1)} and the competitor upper bound
  U_n = 1 - c_(n);
* design 2 (selection rule): G_n = L_n - U_n, commit n* = max{n : G_n > delta}, else n* = 1;
* design 3 (Proposition 4.3 / Corollary 4.4): F_n = (n+1) c_(n) - n (the factor kernel, i.e. the
  factor rule (n+1)(1 - c_(n)) < f with f = 1 - delta), B_n = sum_{j<n} (c_(j) - c_(n)), and
  G_n = F_n + B_n whenever L_n > 0.

The two rules the page compares against (its motivation section, Fast-dLLM's confidence-aware
parallel decoding): the threshold rule commits every candidate with c_i >= tau independently, and
the factor rule accepts the top n candidates when (n+1)(1 - c_(n)) < f. Readings: both commit at
least one candidate when there is one (the progress guarantee the page states for n*), the factor
rule takes the largest such n (its left side never decreases with n, so that is the accepted
prefix), and c_i >= tau is inclusive.

Readings: ties in c are ordered by candidate slot ascending; m = 0 commits 0;
delta must be >= 0; sums are fp64 in sorted order (exact whenever every c is an fp32 value >= 2^-17
and m <= 8192, because every term is then a multiple of 2^-40 and every partial sum is below 2^13).
"""
from __future__ import annotations

import numpy as np


def sort_profile(c: np.ndarray):
    """c [m] fp32 -> (order int32 [m] by (c desc, slot asc), sorted fp64 values)."""
    c = np.asarray(c, np.float32)
    m = c.shape[0]
    order = np.lexsort((np.arange(m), -c.astype(np.float64))).astype(np.int32)
    return order, c[order].astype(np.float64)


def margins(c_sorted: np.ndarray):
    """fp64 sorted profile -> (L, U, G) for n = 1..m, prefix sums taken sequentially."""
    m = len(c_sorted)
    L = np.empty(m)
    U = np.empty(m)
    S = 0.0
    for i in range(m):
        S += float(c_sorted[i])
        n = i + 1
        L[i] = max(0.0, S - (n - 1))
        U[i] = 1.0 - float(c_sorted[i])
    return L, U, L - U


def commit_count(c: np.ndarray, delta: float) -> tuple[int, np.ndarray]:
    """Frechet rule for one sequence: c [m] -> (n*, order)."""
    if delta < 0:
        raise ValueError("delta must be >= 0")
    order, cs = sort_profile(c)
    if len(cs) == 0:
        return 0, order
    _, _, G = margins(cs)
    ok = np.nonzero(G > delta)[0]
    n_star = int(ok[-1]) + 1 if ok.size else 1
    return n_star, order


def frechet_commit(conf: np.ndarray, m_valid: np.ndarray | None, delta: float):
    """Batched form matching the library call: conf [B, m] -> (n_commit [B], order [B, m]).
    Only the first m_valid[b] slots are candidates; order entries past m_valid[b] are -1."""
    conf = np.asarray(conf, np.float32)
    B, m = conf.shape
    n = np.zeros(B, np.int32)
    order = np.full((B, m), -1, np.int32)
    for b in range(B):
        mv = m if m_valid is None else int(m_valid[b])
        nb, ob = commit_count(conf[b, :mv], delta)
        n[b] = nb
        order[b, :mv] = ob
    return n, order


# --- the comparator of Proposition 4.3 / Corollary 4.4 (used by the tests) ---------------------
def factor_kernel(c_sorted: np.ndarray) -> np.ndarray:
    n = np.arange(1, len(c_sorted) + 1, dtype=np.float64)
    return (n + 1) * c_sorted - n


def heterogeneity_bonus(c_sorted: np.ndarray) -> np.ndarray:
    out = np.empty(len(c_sorted))
    for i in range(len(c_sorted)):
        out[i] = float(np.sum(c_sorted[:i] - c_sorted[i]))
    return out


def factor_commit_count(c: np.ndarray, f: float) -> int:
    """Factor rule: largest n with (n+1)(1 - c_(n)) < f (fp64), else 1 (0 if m = 0)."""
    _, cs = sort_profile(c)
    if len(cs) == 0:
        return 0
    n_star = 1
    for i in range(len(cs)):
        n = i + 1
        if (n + 1.0) * (1.0 - float(cs[i])) < f:
            n_star = n
    return n_star


def factor_count(c: np.ndarray, delta: float) -> int:
    """Matched factor rule of Corollary 4.4: the factor rule with f = 1 - delta."""
    return factor_commit_count(c, 1.0 - delta)


def threshold_commit_count(c: np.ndarray, tau: float) -> int:
    """Threshold rule: the number of candidates with c_i >= tau (fp64 compare), at least 1
    (0 if m = 0). They are the first entries of the (c desc, slot asc) order."""
    c = np.asarray(c, np.float32)
    if c.shape[0] == 0:
        return 0
    k = sum(1 for v in c if float(v) >= tau)
    return max(k, 1)


RULES = ("frechet", "factor", "threshold")


def commit(conf: np.ndarray, m_valid: np.ndarray | None, rule: str, param: float):
    """Batched commit under one rule: conf [B, m] -> (n_commit [B], order [B, m]); param is delta
    (frechet), f (factor) or tau (threshold). The order is the same for every rule."""
    if rule not in RULES:
        raise ValueError(rule)
    if rule == "frechet":
        return frechet_commit(conf, m_valid, param)
    conf = np.asarray(conf, np.float32)
    B, m = conf.shape
    n = np.zeros(B, np.int32)
    order = np.full((B, m), -1, np.int32)
    for b in range(B):
        mv = m if m_valid is None else int(m_valid[b])
        ob, _ = sort_profile(conf[b, :mv])
        order[b, :mv] = ob
        n[b] = (factor_commit_count(conf[b, :mv], param) if rule == "factor"
                else threshold_commit_count(conf[b, :mv], param))
    return n, order
