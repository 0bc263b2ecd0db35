"""Seeded synthetic inputs generated directly in GPU memory (for workloads too large to draw on the
host: 32 layers of LLaDA-8B-shaped weights are 14 GB). Inputs only; none of the method's arithmetic.

Each tensor has its own torch.Generator seeded from (seed, cfg, *keys), so any tensor can be
regenerated alone. Normals are drawn in fp32 and rounded to bf16 (round to nearest even).
"""
from __future__ import annotations

import hashlib

import torch


def _seed(cfg: int, *keys: int, seed: int = 0) -> int:
    h = hashlib.sha256(repr((seed, cfg) + tuple(keys)).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def gen(cfg: int, *keys: int, device="cuda") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(cfg, *keys))
    return g


def normal_bf16(shape, std: float, cfg: int, *keys: int, device="cuda") -> torch.Tensor:
    x = torch.randn(shape, generator=gen(cfg, *keys, device=device), device=device,
                    dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(torch.bfloat16)


def layer_weights(d: int, ffn: int, std: float, cfg: int, layer: int, device="cuda") -> dict:
    w = {
        "w_qkv": normal_bf16((3 * d, d), std, cfg, layer, 0, device=device),
        "w_o": normal_bf16((d, d), std, cfg, layer, 1, device=device),
        "w_gate": normal_bf16((ffn, d), std, cfg, layer, 2, device=device),
        "w_up": normal_bf16((ffn, d), std, cfg, layer, 3, device=device),
        "w_down": normal_bf16((d, ffn), std, cfg, layer, 4, device=device),
        "g_attn": torch.ones(d, dtype=torch.bfloat16, device=device),
        "g_ffn": torch.ones(d, dtype=torch.bfloat16, device=device),
    }
    return w


def drift_inputs(B: int, N: int, d: int, frac: float, sigma: float, cfg: int, layer: int,
                 device="cuda"):
    """(x_cur, x_prev): x_prev ~ N(0,1) bf16 [B, N, d]; in each sequence round(frac*N) distinct
    random rows of x_cur get +N(0, sigma^2) (then bf16 rounding); all other rows are bitwise copies."""
    x_prev = normal_bf16((B, N, d), 1.0, cfg, layer, 10, device=device)
    x_cur = x_prev.clone()
    n = int(round(frac * N))
    g = gen(cfg, layer, 11, device=device)
    for b in range(B):
        rows = torch.randperm(N, generator=g, device=device)[:n]
        noise = torch.randn((n, d), generator=g, device=device, dtype=torch.float32) * sigma
        x_cur[b, rows] = (x_prev[b, rows].float() + noise).to(torch.bfloat16)
    return x_cur, x_prev


def planted_logits(R: int, V: int, cfg: int, lo: float = 2.0, hi: float = 12.0, device="cuda"):
    """bf16 [R, V] logits ~ N(0,1) with U(lo, hi) added at one uniform-random index per row."""
    g = gen(cfg, 20, device=device)
    z = torch.randn((R, V), generator=g, device=device, dtype=torch.float32)
    idx = torch.randint(0, V, (R,), generator=g, device=device)
    bump = torch.rand((R,), generator=g, device=device) * (hi - lo) + lo
    z[torch.arange(R, device=device), idx] += bump
    return z.to(torch.bfloat16)


def drifted_logits(z: torch.Tensor, sigma: float, cfg: int) -> torch.Tensor:
    """The same positions' logits one step earlier: z + N(0, sigma^2) per entry, bf16."""
    g = gen(cfg, 21, device=z.device)
    n = torch.randn(z.shape, generator=g, device=z.device, dtype=torch.float32)
    return (z.float() + sigma * n).to(torch.bfloat16)


def key_positions(B: int, P: int, lo: int, hi: int, cfg: int, device="cuda") -> torch.Tensor:
    g = gen(cfg, 30, device="cpu")
    out = torch.stack([torch.randperm(hi - lo, generator=g)[:P] + lo for _ in range(B)])
    return out.sort(dim=1).values.to(torch.int32).to(device)
