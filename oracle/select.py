"""Top-B selection united with forced update windows (oracle; test infrastructure only).

Follows "Dynamic-dLLM" reading notes:
* Key design 1 (DCU): each layer recomputes the top-B tokens by distance d_i; every other token
  reuses its cached values;
* Key design 2 (forced update window): around each key token p unmasked at the previous step, a
  window of fixed size B_window is always recomputed (the U^{t,l} union equation), and the remaining
  budget is spent outside the window.

Readings:
* the window holds exactly B_window positions, [p - floor(B_window/2), p - floor(B_window/2) +
  B_window - 1], clipped to [0, N) (the page's inclusive bracket [p - B/2, p + B/2] would hold
  B + 1; ``literal_window=True`` switches to that form for sensitivity checks only);
* several key tokens: the union of their windows; positions outside [0, N) are ignored;
* candidates are the positions outside the window with d_i > 0, ranked by (d_i descending,
  position ascending) on the exact fp32 values; the top min(b, |C|) are taken;
* the result is the ascending list of W union A.
"""
from __future__ import annotations

import numpy as np


def window_mask(key_pos, N: int, b_window: int, literal_window: bool = False) -> np.ndarray:
    w = np.zeros(N, bool)
    for p in np.asarray(key_pos).reshape(-1).tolist():
        if p < 0 or p >= N or b_window <= 0:
            continue
        if literal_window:
            lo, hi = p - b_window // 2, p + b_window // 2
        else:
            lo = p - b_window // 2
            hi = lo + b_window - 1
        lo = max(lo, 0)
        hi = min(hi, N - 1)
        if lo <= hi:
            w[lo:hi + 1] = True
    return w


def select_row(dist: np.ndarray, budget: int, key_pos, b_window: int,
               literal_window: bool = False) -> np.ndarray:
    """dist [N] fp32, budget b >= 0 -> ascending int32 positions U."""
    dist = np.asarray(dist, np.float32)
    N = dist.shape[0]
    w = window_mask(key_pos, N, b_window, literal_window)
    cand = np.nonzero((~w) & (dist > 0))[0]
    # rank by distance descending, then position ascending
    order = np.lexsort((cand, -dist[cand].astype(np.float64)))
    chosen = cand[order[:max(0, min(int(budget), len(cand)))]]
    u = np.zeros(N, bool)
    u[w] = True
    u[chosen] = True
    return np.nonzero(u)[0].astype(np.int32)


def select(dist: np.ndarray, budgets: np.ndarray, layer: int, key_pos: np.ndarray, b_window: int):
    """Batched form matching the library call: dist [B, N], budgets [B, L] (column ``layer`` is
    used), key_pos [B, P] (-1 = unused) -> (sel_idx [B, N] int32 padded with -1, sel_count [B])."""
    dist = np.asarray(dist, np.float32)
    B, N = dist.shape
    sel = np.full((B, N), -1, np.int32)
    cnt = np.zeros(B, np.int32)
    for b in range(B):
        u = select_row(dist[b], int(budgets[b, layer]), key_pos[b], b_window)
        sel[b, :len(u)] = u
        cnt[b] = len(u)
    return sel, cnt
