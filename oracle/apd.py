"""Adaptive parallel decoding (APD) thresholds (oracle; test infrastructure only).

Follows "Dynamic-dLLM" reading notes, Key design 3 (adaptive parallel decoding):
* the distribution of position i at step t is z_i^t (a probability vector over the vocabulary),
  u = argmax_v z_v;
* confidence concentration  c_i^t = 1 - max_{v != u} (z_i^t)_v  (one minus the second-largest
  probability);
* temporal instability  H_i^t = 1 - <z_i^t, z_i^{t+1}> / (|z_i^t| |z_i^{t+1}|), the cosine distance
  between this step's distribution and the previous step's (step t+1 is the previous one: the
  page counts steps down);
* threshold update  tau_i^t = tau_i^{t+1} - alpha c_i^t + beta H_i^t, with alpha, beta >= 0 and
  tau initialised near 0.9;
* a position unmasks when its confidence reaches its own threshold (the static-threshold rule of
  Fast-dLLM with the per-token tau in place of the fixed one).

Readings: z is the temperature-1 softmax of the logits, taken in fp64; u is the lowest index among
equal maxima, and a tie at the top makes the second-largest probability equal to the largest; with
one vocabulary entry c = 1; at the first step (no previous distribution) H = 0; the unmask test is
p_max >= tau (inclusive), with p_max the confidence of dllm_confidence; a sequence with candidates
unmasks at least its most confident one (lowest slot on ties), the progress guarantee the
Frechet-decoding page states for its rule; alpha and beta are not given by the page and are inputs.
"""
from __future__ import annotations

import numpy as np

from oracle.confidence import _values


def softmax64(logits: np.ndarray, V: int | None = None) -> np.ndarray:
    """logits [R, >=V] (fp32, or bf16 bit patterns as uint16) -> probabilities fp64 [R, V]."""
    z = _values(logits)
    if V is not None:
        z = z[:, :V]
    e = np.exp(z - z.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


def signals(logits: np.ndarray, logits_prev: np.ndarray | None, V: int | None = None):
    """-> (p_max, token, c, H) per row, fp64 (token int32)."""
    p = softmax64(logits, V)
    R, Vv = p.shape
    tok = np.argmax(p, axis=1).astype(np.int32)
    pmax = p[np.arange(R), tok]
    c = np.empty(R)
    for r in range(R):
        if Vv == 1:
            c[r] = 1.0
        else:
            others = np.delete(p[r], tok[r])
            c[r] = 1.0 - others.max()
    if logits_prev is None:
        H = np.zeros(R)
    else:
        q = softmax64(logits_prev, V)
        H = np.empty(R)
        for r in range(R):
            H[r] = 1.0 - float(p[r] @ q[r]) / (np.linalg.norm(p[r]) * np.linalg.norm(q[r]))
    return pmax, tok, c, H


def update_threshold(tau_prev: np.ndarray, c: np.ndarray, H: np.ndarray, alpha: float,
                     beta: float) -> np.ndarray:
    return np.asarray(tau_prev, np.float64) - alpha * np.asarray(c) + beta * np.asarray(H)


def unmask(conf: np.ndarray, tau: np.ndarray, m_valid: np.ndarray | None = None):
    """Per sequence: conf, tau [B, m] -> (n_commit [B], order [B, m]): the candidates with
    conf >= tau first (conf desc, slot asc), then the others (conf desc, slot asc); n_commit is how
    many pass, at least 1 when the row has candidates (then the first of the order)."""
    conf = np.asarray(conf, np.float32)
    tau = np.asarray(tau, np.float32)
    B, m = conf.shape
    n = np.zeros(B, np.int32)
    order = np.full((B, m), -1, np.int32)
    for b in range(B):
        mv = m if m_valid is None else int(m_valid[b])
        mv = max(0, min(m, mv))
        if mv == 0:
            continue
        c, t = conf[b, :mv].astype(np.float64), tau[b, :mv].astype(np.float64)
        passed = c >= t
        slots = np.arange(mv)
        ordr = np.lexsort((slots, -c, ~passed))
        order[b, :mv] = ordr
        n[b] = max(int(passed.sum()), 1)
    return n, order
