"""Token cosine distance and layer dynamics (oracle; test infrastructure only).

Follows "Dynamic-dLLM" reading notes, Key design 1 (DCU):

* token distance between the layer input now and the cached input of the previous denoising step,
  d_i = 1 - <x_i^t, x_i^{t+1}> / (||x_i^t|| ||x_i^{t+1}||)   (the d_i^{t,l} equation);
* layer dynamics s = (1/N) sum_i d_i over all N positions (the s^{t,l} definition).

Readings where the page is silent:
* bitwise-identical rows give exactly 0; if exactly one row has zero norm the distance is 1; two
  zero-norm rows give 0;
* the exact value is clamped to [0, 2] and rounded once to fp32 (RNE);
* the mean is taken over the fp32-rounded distances, summed in fp64 in ascending position order,
  divided by N, rounded once to fp32.
"""
from __future__ import annotations

import numpy as np


def _bits(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x.view(np.uint32)
    if x.dtype == np.float64:
        return x.view(np.uint64)
    if x.dtype == np.uint16:  # bf16 bit patterns
        return x
    raise TypeError(f"unsupported dtype {x.dtype}")


def _values(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) or fp32/fp64 values -> exact fp64 values."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def cosine_distance64(x_cur: np.ndarray, x_prev: np.ndarray) -> np.ndarray:
    """Per-row cosine distance in fp64, before the final rounding. Inputs [..., d]."""
    same = np.all(_bits(x_cur) == _bits(x_prev), axis=-1)
    a = _values(x_cur)
    b = _values(x_prev)
    dot = np.sum(a * b, axis=-1)
    na = np.sum(a * a, axis=-1)
    nb = np.sum(b * b, axis=-1)
    with np.errstate(divide="ignore", invalid="ignore"):
        d = 1.0 - dot / np.sqrt(na * nb)
    d = np.clip(d, 0.0, 2.0)
    za = na == 0.0
    zb = nb == 0.0
    d = np.where(za & zb, 0.0, d)
    d = np.where(za ^ zb, 1.0, d)
    d = np.where(same, 0.0, d)
    return d


def cosine_distance(x_cur: np.ndarray, x_prev: np.ndarray) -> np.ndarray:
    """fp32 distance per row: [G, N, d] -> [G, N]."""
    return cosine_distance64(x_cur, x_prev).astype(np.float32)


def layer_mean(dist32: np.ndarray) -> np.ndarray:
    """s[g] = (sum_i dist[g, i]) / N with an fp64 ascending-order sum; fp32 result. [G, N] -> [G]."""
    dist32 = np.asarray(dist32, dtype=np.float32)
    G, N = dist32.shape
    out = np.empty(G, np.float32)
    for g in range(G):
        acc = 0.0
        for v in dist32[g].astype(np.float64).tolist():
            acc += v
        out[g] = np.float32(acc / N)
    return out


def distance_and_mean(x_cur: np.ndarray, x_prev: np.ndarray):
    d = cosine_distance(x_cur, x_prev)
    return d, layer_mean(d)
