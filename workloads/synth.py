"""Seeded synthetic inputs shared by the CPU oracle tests, the GPU parity tests and the benchmark.

This module only draws random numbers and encodes them (fp32 -> bf16 bit patterns). It holds none
of the method's arithmetic: no distance, budget, selection, layer, softmax or commit logic lives here.

Every array comes from ``numpy.random.default_rng([seed, cfg, *keys])`` so that each purpose
(step, layer, tensor) has its own independent stream and any single tensor can be regenerated
without generating the others.

bf16 tensors are returned as ``uint16`` bit patterns (round-to-nearest-even from fp32); use
``bf16_to_f32`` to widen them exactly.
"""
from __future__ import annotations

import dataclasses

import numpy as np

SEED = 0


def rng(cfg: int, *keys: int, seed: int = SEED) -> np.random.Generator:
    return np.random.default_rng([seed, cfg, *keys])


# ----------------------------------------------------------------------------- bf16 encoding
def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (r >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(g: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    return f32_to_bf16(g.standard_normal(shape, dtype=np.float32) * np.float32(std))


# ----------------------------------------------------------------------------- drift inputs
def drift_pair(g: np.random.Generator, n_rows: int, d: int, n_drift: int, sigma: float,
               bf16: bool = True, base: np.ndarray | None = None):
    """(x_cur, x_prev, drifted_rows): x_prev ~ N(0,1); ``n_drift`` distinct random rows of x_cur get
    +N(0, sigma^2) noise, every other row is a bitwise copy of x_prev.

    Returned as bf16 bit patterns (bf16=True) or fp32 arrays.
    """
    if base is None:
        prev32 = g.standard_normal((n_rows, d), dtype=np.float32)
        prev = f32_to_bf16(prev32) if bf16 else prev32
    else:
        prev = base
    rows = np.sort(g.choice(n_rows, size=n_drift, replace=False)) if n_drift else np.zeros(0, np.int64)
    cur = prev.copy()
    noise = g.standard_normal((len(rows), d), dtype=np.float32) * np.float32(sigma)
    if bf16:
        cur[rows] = f32_to_bf16(bf16_to_f32(prev[rows]) + noise)
    else:
        cur[rows] = prev[rows] + noise
    return cur, prev, rows


def key_positions(g: np.random.Generator, batch: int, n_keys: int, lo: int, hi: int) -> np.ndarray:
    """[batch, n_keys] int32 distinct positions uniform in [lo, hi)."""
    out = np.empty((batch, n_keys), np.int32)
    for b in range(batch):
        out[b] = np.sort(g.choice(np.arange(lo, hi), size=n_keys, replace=False))
    return out


# ----------------------------------------------------------------------------- layer weights
@dataclasses.dataclass
class LayerShape:
    d: int
    n_heads: int
    head_dim: int
    ffn: int
    eps: float = 1e-5


LLADA8B = LayerShape(d=4096, n_heads=32, head_dim=128, ffn=12288)
TINY = LayerShape(d=64, n_heads=2, head_dim=32, ffn=128)


def layer_weights(g: np.random.Generator, s: LayerShape, std: float = 0.02, bf16: bool = True,
                  gain_jitter: float = 0.0) -> dict:
    """Random-init weights of one layer. Matrices are [out, in] row-major.

    gains are ones unless ``gain_jitter`` > 0 (then 1 + U(-j, j), used by tests to make sure the
    gain vectors are applied).
    """
    def mat(rows, cols):
        x = g.standard_normal((rows, cols), dtype=np.float32) * np.float32(std)
        return f32_to_bf16(x) if bf16 else x

    def gain():
        x = np.ones(s.d, np.float32)
        if gain_jitter:
            x = x + g.uniform(-gain_jitter, gain_jitter, s.d).astype(np.float32)
        return f32_to_bf16(x) if bf16 else x

    return dict(w_qkv=mat(3 * s.d, s.d), w_o=mat(s.d, s.d), w_gate=mat(s.ffn, s.d),
                w_up=mat(s.ffn, s.d), w_down=mat(s.d, s.ffn), g_attn=gain(), g_ffn=gain())


# ----------------------------------------------------------------------------- logits
def planted_logits(g: np.random.Generator, rows: int, vocab: int, lo: float = 2.0, hi: float = 12.0,
                   bf16: bool = True):
    """logits ~ N(0,1) with U(lo, hi) added at one uniform-random vocab index per row."""
    z = g.standard_normal((rows, vocab), dtype=np.float32)
    idx = g.integers(0, vocab, size=rows)
    z[np.arange(rows), idx] += g.uniform(lo, hi, size=rows).astype(np.float32)
    return (f32_to_bf16(z) if bf16 else z), idx


def confidence_profile(g: np.random.Generator, batch: int, m: int, lo: float = 0.0, hi: float = 1.0):
    """[batch, m] fp32 confidences uniform in [lo, hi] (inputs for the commit rule on its own)."""
    return g.uniform(lo, hi, size=(batch, m)).astype(np.float32)
