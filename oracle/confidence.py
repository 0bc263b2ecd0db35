"""Per-position confidence over the vocabulary (oracle; test infrastructure only).

Follows "Fast-dLLM++" reading notes, Key designs / overall framework: after the forward pass each
masked position takes the argmax of its marginal prediction and that argmax's probability as its
confidence c_i.

Readings: temperature-1 softmax over the full vocabulary; no sampling noise;
the argmax is the lowest index among equal maxima; c = 1 / sum_v exp(z_v - max z) in fp64.
"""
from __future__ import annotations

import numpy as np


def _values(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z)
    if z.dtype == np.uint16:
        return (z.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return z.astype(np.float64)


def confidence64(logits: np.ndarray, V: int | None = None):
    """logits [R, >=V] -> (conf fp64 [R], token int32 [R])."""
    z = _values(logits)
    if V is not None:
        z = z[:, :V]
    tok = np.argmax(z, axis=1).astype(np.int32)        # first occurrence = lowest index
    m = z[np.arange(z.shape[0]), tok]
    c = 1.0 / np.sum(np.exp(z - m[:, None]), axis=1)
    return c, tok


def confidence(logits: np.ndarray, V: int | None = None):
    c, tok = confidence64(logits, V)
    return c.astype(np.float32), tok
