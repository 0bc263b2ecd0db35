"""Per-layer recompute budget (oracle; test infrastructure only).

Follows "Dynamic-dLLM" reading notes, Key design 1 (DCU), the budget equation
B^{t,l} = (B_layer * LayerNum) * s^{t+1,l} / sum_k s^{t+1,k}: the total budget T = B_layer * L is
split across layers in proportion to the previous step's layer means (the page's step t+1 is the
previous step because its step index counts down).

The page gives a real-valued share. Readings:
* integer budgets by floor plus largest remainder, ties to the lower layer, in IEEE fp64 with the
  fixed operation order below, so that sum_l b_l == T exactly;
* with no previous step, or when every previous mean is 0, each layer gets B_layer;
* a layer mean is an average of distances in [0, 2], so it is never negative; a negative entry is
  read as 0.

The floors never overshoot T, so only the "add one to the largest remainders" step exists: with
every s_l >= 0 and finite, the sequential fp64 sum S is at least (1 - (L-1) u) times the exact sum
(u = 2^-53), and each q_l = fl(fl(T s_l) / S) is at most T s_l (1 + u)^2 / S. Summed over the
layers this bounds sum_l q_l by T (1 + (L + 2) u) up to higher-order terms, which is below T + 1
for every T < 2^31 and L <= 1024. The floors are integers summing to at most sum_l q_l, hence to at
most T: the remainder count R = T - sum_l floor(q_l) is never negative.
"""
from __future__ import annotations

import numpy as np


def layer_budget_row(s_prev: np.ndarray | None, L: int, b_layer: int) -> np.ndarray:
    T = b_layer * L
    if s_prev is None:
        return np.full(L, b_layer, np.int32)
    s = [max(float(np.float32(v)), 0.0) for v in np.asarray(s_prev, np.float32).reshape(L)]
    S = 0.0
    for v in s:  # ascending layer order
        S += v
    if S == 0.0:
        return np.full(L, b_layer, np.int32)
    q = [(float(T) * v) / S for v in s]
    f = [float(np.floor(x)) for x in q]
    r = [q[i] - f[i] for i in range(L)]
    b = [int(x) for x in f]
    R = T - sum(b)
    assert R >= 0, "the floors cannot overshoot T (see the module docstring)"
    # the R largest remainders get +1; ties to the lower layer
    order = sorted(range(L), key=lambda i: (-r[i], i))
    for i in order[:R]:
        b[i] += 1
    return np.asarray(b, np.int32)


def layer_budget(s_prev: np.ndarray | None, B: int, L: int, b_layer: int) -> np.ndarray:
    """[B, L] fp32 previous-step means (or None) -> [B, L] int32 budgets, each row summing to b_layer*L."""
    if s_prev is None:
        return np.full((B, L), b_layer, np.int32)
    s_prev = np.asarray(s_prev, np.float32).reshape(B, L)
    return np.stack([layer_budget_row(s_prev[b], L, b_layer) for b in range(B)])
