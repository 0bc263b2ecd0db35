"""Selective transformer layer on the recomputed rows (oracle; test infrastructure only).

What is recomputed follows "Dynamic-dLLM" reading notes, Key design 1 (DCU): only the selected
tokens are recomputed, all others reuse their cached values. The layer is a bidirectional
(unmasked) attention block, as the notes' background section states for diffusion LLMs, with a QKV
projection, attention of the selected queries over every cached key/value, an output projection and
a SwiGLU feed-forward block.

The pages do not fix the layer internals. Reading used here ("parity unpinned"
by the pages, pinned by the tests as an implementation of this reading):
* pre-norm residual block with RMSNorm (gain vectors, eps given), no attention mask, softmax scale
  1/sqrt(head_dim);
* rotary position embedding optional (rope_theta > 0; 0 = none, the default): the RoFormer rotation
  in the rotate-half pairing used by LLaMA-family models such as LLaDA, applied to every head's q
  and k (not v) with the token's position in its sequence (its row index, 0 .. N-1). Head dim i and
  i + dh/2 (i < dh/2) form a pair rotated by the angle pos * theta^(-2i/dh). The pages say nothing
  about positions; this is the standard form of the model family they evaluate;
* weights stored [out, in]; w_qkv rows are Wq | Wk | Wv; heads are contiguous head_dim slices;
* cached K/V rows of the selected tokens are overwritten before attention, so the selected queries
  see each other's new keys and values;
* rows outside the selection keep their K, V and output bit for bit.

Everything is computed in fp64 from the exact input values (bf16 bit patterns are widened exactly).
"""
from __future__ import annotations

import numpy as np


def as64(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def weights64(w: dict) -> dict:
    return {k: as64(v) for k, v in w.items()}


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * g


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def softmax_rows(s: np.ndarray) -> np.ndarray:
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotary embedding of head vectors x [..., dh] at positions pos (broadcast against x[..., 0]):
    with h = dh/2 and angle a_i = pos * theta^(-2i/dh), the pair (x_i, x_{i+h}) becomes
    (x_i cos a_i - x_{i+h} sin a_i, x_{i+h} cos a_i + x_i sin a_i). fp64."""
    dh = x.shape[-1]
    h = dh // 2
    inv_freq = float(theta) ** (-(2.0 * np.arange(h)) / dh)
    ang = np.asarray(pos, np.float64)[..., None] * inv_freq
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def selective_layer_seq(w64: dict, n_heads: int, head_dim: int, eps: float, x: np.ndarray,
                        rows: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, y: np.ndarray,
                        rope_theta: float = 0.0):
    """One sequence. x [N, d] fp64 layer input; rows: ascending selected positions;
    k_cache, v_cache [N, H, dh] fp64; y [N, d] fp64. Returns new (k_cache, v_cache, y) copies.
    rope_theta > 0 rotates q and k of each selected row by its position (its row index)."""
    N, d = x.shape
    H, dh = n_heads, head_dim
    kc = k_cache.copy()
    vc = v_cache.copy()
    yo = y.copy()
    rows = np.asarray(rows, np.int64)
    if rows.size == 0:
        return kc, vc, yo
    xs = x[rows]                                      # gather
    xn = rmsnorm(xs, w64["g_attn"], eps)
    qkv = xn @ w64["w_qkv"].T                         # [M, 3d]
    q = qkv[:, :d].reshape(-1, H, dh)
    k = qkv[:, d:2 * d].reshape(-1, H, dh)
    if rope_theta > 0:
        q = rope(q, rows[:, None], rope_theta)
        k = rope(k, rows[:, None], rope_theta)
    kc[rows] = k                                      # K/V scatter into the cache
    vc[rows] = qkv[:, 2 * d:].reshape(-1, H, dh)
    o = np.empty((len(rows), H, dh))
    scale = 1.0 / np.sqrt(dh)
    for h in range(H):
        p = softmax_rows((q[:, h, :] @ kc[:, h, :].T) * scale)   # over all N cached keys
        o[:, h, :] = p @ vc[:, h, :]
    a = xs + o.reshape(-1, d) @ w64["w_o"].T          # output projection + residual
    an = rmsnorm(a, w64["g_ffn"], eps)
    z = (silu(an @ w64["w_gate"].T) * (an @ w64["w_up"].T)) @ w64["w_down"].T
    yo[rows] = a + z                                  # scatter back
    return kc, vc, yo


def selective_layer(w: dict, n_heads: int, head_dim: int, eps: float, x_in: np.ndarray,
                    sel_idx: np.ndarray | None, sel_count: np.ndarray | None,
                    k_cache: np.ndarray, v_cache: np.ndarray, y: np.ndarray,
                    rope_theta: float = 0.0):
    """Batched form matching the library call. x_in [B, N, d]; sel_idx [B, N] (first sel_count[b]
    valid) or None for every row (dense mode); caches [B, N, H, dh]; y [B, N, d].
    Returns fp64 (k_cache, v_cache, y)."""
    w64 = weights64(w)
    x = as64(x_in)
    kc = as64(k_cache)
    vc = as64(v_cache)
    yo = as64(y)
    B, N, _ = x.shape
    for b in range(B):
        rows = np.arange(N) if sel_idx is None else np.asarray(sel_idx[b, :int(sel_count[b])])
        kc[b], vc[b], yo[b] = selective_layer_seq(w64, n_heads, head_dim, eps, x[b], rows,
                                                  kc[b], vc[b], yo[b], rope_theta)
    return kc, vc, yo


def v_features(w: dict, eps: float, x: np.ndarray) -> np.ndarray:
    """Value vectors of every row (the V-feature distance's input, dLLM-Cache style): [B, N, d]
    fp64 = RMSNorm(x; g_attn) W_v^T, W_v the last d rows of W_qkv."""
    w64 = weights64(w)
    d = w64["w_o"].shape[0]
    x64 = as64(x)
    xn = rmsnorm(x64, w64["g_attn"], eps)
    return xn @ w64["w_qkv"][2 * d:3 * d].T


def attention_context(w: dict, n_heads: int, head_dim: int, eps: float, x: np.ndarray,
                      k_cache: np.ndarray, v_cache: np.ndarray, rope_theta: float = 0.0) -> np.ndarray:
    """Attention context of every row (the DyLLM-style saliency feature: its cosine similarity
    between adjacent steps marks the salient tokens), [B, N, d] fp64: per sequence and head,
    softmax(q K^T / sqrt(head_dim)) V over the N cached rows as given, with q = RMSNorm(x; g_attn)
    W_q^T (W_q the first d rows of W_qkv), rotated by each row's position when rope_theta > 0.
    Reading: the caches are the previous step's (the feature decides what to recompute, so it is
    taken before any recomputation)."""
    w64 = weights64(w)
    x64 = as64(x)
    kc, vc = as64(k_cache), as64(v_cache)
    B, N, d = x64.shape
    H, dh = n_heads, head_dim
    out = np.empty((B, N, d))
    scale = 1.0 / np.sqrt(dh)
    for b in range(B):
        q = (rmsnorm(x64[b], w64["g_attn"], eps) @ w64["w_qkv"][:d].T).reshape(N, H, dh)
        if rope_theta > 0:
            q = rope(q, np.arange(N)[:, None], rope_theta)
        for h in range(H):
            p = softmax_rows((q[:, h, :] @ kc[b, :, h, :].T) * scale)
            out[b, :, h * dh:(h + 1) * dh] = p @ vc[b, :, h, :]
    return out
