"""Seeded synthetic token streams for the int8-state GDN / KDA decode path.

This module only draws random numbers and shapes them into the documented
distributions; it computes nothing of the method itself, so both the CPU
oracle and the HIP path can consume the very same arrays.

Distributions (the workload presets in ``configs.py`` choose among them):

* q, k  ~ N(0, 1) per element, every (t, b, h) vector L2-normalised
  (guard 1e-12), optionally with fixed per-head key channels scaled by a
  factor *before* normalisation (outlier stress preset);
* v     ~ N(0, 1), optionally with fixed per-head value columns scaled;
* alpha = exp(-softplus(x)) = sigmoid(-x), x ~ N(-3, 0.5): one decay per
  (t, b, h) for Gated DeltaNet, one per (t, b, h, key channel) for
  Kimi-Delta-style diagonal gating;
* beta  ~ U(lo, hi).

Host streams use numpy ``Generator(Philox(seed))`` and draw in the fixed order
(x_alpha, beta, q, k, v).  ``device_tokens`` draws the same distributions on a
torch device with torch's own Philox generator; it is for timing runs only,
where values matter only through their distribution.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Outliers:
    """Fixed outlier channels per head: ``key_ch[h]`` (n_key channels) are
    multiplied by ``key_scale`` before L2 normalisation, ``val_col[h]`` by
    ``val_scale``."""
    key_ch: np.ndarray      # [H, n_key] int
    val_col: np.ndarray     # [H, n_val] int
    key_scale: float
    val_scale: float


def make_outliers(seed: int, H: int, dk: int, dv: int, n_key: int = 4, n_val: int = 2,
                  key_scale: float = 30.0, val_scale: float = 20.0) -> Outliers:
    """Per head, draw ``n_key`` distinct key channels and ``n_val`` distinct
    value columns; they stay fixed over batch and time."""
    rng = np.random.Generator(np.random.Philox(seed + 0x5EED))
    kc = np.stack([rng.choice(dk, size=n_key, replace=False) for _ in range(H)])
    vc = np.stack([rng.choice(dv, size=n_val, replace=False) for _ in range(H)])
    return Outliers(kc.astype(np.int64), vc.astype(np.int64), key_scale, val_scale)


def _l2n(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(n, 1e-12)


def host_tokens(seed: int, T: int, B: int, H: int, dk: int, dv: int, *, per_key: bool,
                beta_lo: float, beta_hi: float, outliers: Outliers | None = None) -> dict:
    """T tokens for every (b, h), as contiguous float32 arrays:
    q, k [T,B,H,dk]; v [T,B,H,dv]; alpha [T,B,H] or [T,B,H,dk]; beta [T,B,H]."""
    rng = np.random.Generator(np.random.Philox(seed))
    ashape = (T, B, H, dk) if per_key else (T, B, H)
    xa = rng.normal(-3.0, 0.5, size=ashape)
    beta = rng.uniform(beta_lo, beta_hi, size=(T, B, H))
    q = rng.standard_normal((T, B, H, dk))
    k = rng.standard_normal((T, B, H, dk))
    v = rng.standard_normal((T, B, H, dv))
    if outliers is not None:
        for h in range(H):
            k[:, :, h, outliers.key_ch[h]] *= outliers.key_scale
            v[:, :, h, outliers.val_col[h]] *= outliers.val_scale
    alpha = 1.0 / (1.0 + np.exp(xa))          # exp(-softplus(x))
    f32 = lambda a: np.ascontiguousarray(a, dtype=np.float32)
    return dict(q=f32(_l2n(q)), k=f32(_l2n(k)), v=f32(v), alpha=f32(alpha), beta=f32(beta))


def device_tokens(seed: int, T: int, B: int, H: int, dk: int, dv: int, *, per_key: bool,
                  beta_lo: float, beta_hi: float, device, outliers: Outliers | None = None) -> dict:
    """Same distributions as ``host_tokens``, drawn on ``device`` with torch's
    generator (different numbers).  Used to fill large timing rings."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    f = dict(device=device, dtype=torch.float32, generator=g)
    ashape = (T, B, H, dk) if per_key else (T, B, H)
    xa = torch.randn(ashape, **f) * 0.5 - 3.0
    beta = torch.rand((T, B, H), **f) * (beta_hi - beta_lo) + beta_lo
    q = torch.randn((T, B, H, dk), **f)
    k = torch.randn((T, B, H, dk), **f)
    v = torch.randn((T, B, H, dv), **f)
    if outliers is not None:
        for h in range(H):
            kc = torch.as_tensor(outliers.key_ch[h], device=device)
            vc = torch.as_tensor(outliers.val_col[h], device=device)
            k[:, :, h, kc] *= outliers.key_scale
            v[:, :, h, vc] *= outliers.val_scale
    q = q / q.norm(dim=-1, keepdim=True).clamp_min(1e-12)
    k = k / k.norm(dim=-1, keepdim=True).clamp_min(1e-12)
    alpha = torch.sigmoid(-xa)
    return dict(q=q.contiguous(), k=k.contiguous(), v=v.contiguous(),
                alpha=alpha.contiguous(), beta=beta.contiguous())
