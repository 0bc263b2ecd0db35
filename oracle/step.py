"""One DCU denoising step over all layers, plus the end of step (oracle; test infrastructure only).

Order of operations per step (see the per-module docstrings for the passages each part follows):

1. budgets from the previous step's layer means (budget.layer_budget);
2. for each layer l in order: distance and mean against the cached input of the previous step,
   top-B plus window selection, the selective layer on the selected rows, then the cached input of
   layer l becomes this step's input (all rows);
3. this step's means become the next step's previous means;
4. end of step: confidence and argmax per candidate position, then the Frechet commit.

``open loop``: every layer's current input is given (the synthetic drift workloads).
``closed loop``: layer l+1's input is layer l's output buffer Y[l] after its scatter, which is what
makes the "stuck in the mud" effect of Key design 2 in the Dynamic-dLLM notes observable.

The initial cache fill is one dense pass (every row selected) over each layer's cached input; the
pages do not describe the initial fill, so this is a reading.

``rope_theta`` > 0 runs every layer with rotary position embedding of that base (see
layer.selective_layer_seq), as the models the pages' diffusion LLMs are built on do.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from . import budget as _budget
from . import confidence as _conf
from . import distance as _dist
from . import frechet as _frechet
from . import layer as _layer
from . import select as _select


@dataclasses.dataclass
class State:
    x_prev: list          # per layer [B, N, d] (bf16 bits or fp32/fp64 values)
    k_cache: list         # per layer [B, N, H, dh] fp64
    v_cache: list
    y: list               # per layer [B, N, d] fp64
    s_prev: np.ndarray | None = None   # [B, L] fp32


def dense_fill(weights: list, n_heads: int, head_dim: int, eps: float, x_prev: list,
               rope_theta: float = 0.0) -> State:
    L = len(weights)
    B, N, d = np.asarray(x_prev[0]).shape
    kc, vc, ys = [], [], []
    for l in range(L):
        z = np.zeros((B, N, n_heads, head_dim))
        k, v, y = _layer.selective_layer(weights[l], n_heads, head_dim, eps, x_prev[l], None, None,
                                         z, z.copy(), np.zeros((B, N, d)), rope_theta)
        kc.append(k)
        vc.append(v)
        ys.append(y)
    return State(x_prev=list(x_prev), k_cache=kc, v_cache=vc, y=ys, s_prev=None)


def dcu_step(state: State, weights: list, n_heads: int, head_dim: int, eps: float, b_layer: int,
             b_window: int, key_pos: np.ndarray, x_cur: list | None = None, x0=None,
             rope_theta: float = 0.0):
    """Runs one step in place on ``state``. Open loop if ``x_cur`` (a per-layer list) is given,
    closed loop from the first-layer input ``x0`` otherwise. Returns a per-layer record."""
    L = len(weights)
    B, N = np.asarray(state.x_prev[0]).shape[:2]
    budgets = _budget.layer_budget(state.s_prev, B, L, b_layer)
    s = np.zeros((B, L), np.float32)
    rec = []
    X = x0
    for l in range(L):
        if x_cur is not None:
            X = x_cur[l]
        d, mean = _dist.distance_and_mean(X, state.x_prev[l])
        s[:, l] = mean
        sel, cnt = _select.select(d, budgets, l, key_pos, b_window)
        k, v, y = _layer.selective_layer(weights[l], n_heads, head_dim, eps, X, sel, cnt,
                                         state.k_cache[l], state.v_cache[l], state.y[l], rope_theta)
        state.k_cache[l], state.v_cache[l], state.y[l] = k, v, y
        state.x_prev[l] = X
        rec.append(dict(dist=d, mean=mean, sel_idx=sel, sel_count=cnt, budgets=budgets[:, l]))
        X = y
    state.s_prev = s
    return rec


def end_of_step(logits: np.ndarray, V: int, B: int, m: int, m_valid, delta: float):
    """logits [B*m, >=V] for B sequences of m candidate slots -> conf, token, n_commit, order."""
    conf, tok = _conf.confidence(logits, V)
    n, order = _frechet.frechet_commit(conf.reshape(B, m), m_valid, delta)
    return conf, tok, n, order
