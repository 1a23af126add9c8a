"""Seeded random draws for the KIVI workload (torch; any device).

Keys are N(0,1) with a few fixed outlier channels per head scaled up across
every token, values are N(0,1); both fp16.  This mirrors the KIVI page's
observation that key caches have a handful of persistent large-magnitude
channels while value caches do not (distribution-evidence section, Fig. 2).
"""

from __future__ import annotations

import math
from typing import Tuple

import numpy as np
import torch

from .configs import KiviConfig


def _gen(cfg: KiviConfig, device, part: int) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(cfg.seed * 1_000_003 + 7919 * part + 1)
    return g


def outlier_channels(cfg: KiviConfig) -> np.ndarray:
    """[H][n_outlier] channel ids, seeded, distinct within a head."""
    rng = np.random.default_rng(cfg.seed * 31 + 5)
    return np.stack([rng.choice(cfg.D, size=cfg.n_outlier, replace=False) for _ in range(cfg.H)])


def raw_kv(cfg: KiviConfig, device="cpu", L: int = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """(k, v) fp16 [B][H][L][D] (L defaults to cfg.L)."""
    L = cfg.L if L is None else L
    k = torch.randn((cfg.B, cfg.H, L, cfg.D), generator=_gen(cfg, device, 1), device=device)
    v = torch.randn((cfg.B, cfg.H, L, cfg.D), generator=_gen(cfg, device, 2), device=device)
    ch = torch.as_tensor(outlier_channels(cfg), device=device)
    scale = torch.ones((cfg.H, cfg.D), device=device)
    scale.scatter_(1, ch, cfg.outlier_scale)
    k = k * scale[None, :, None, :]
    return k.to(torch.float16), v.to(torch.float16)


def new_tokens(cfg: KiviConfig, n: int, device="cpu") -> Tuple[torch.Tensor, torch.Tensor]:
    """n further decode tokens per (request, head): (k, v) fp16 [n][B][H][D], same statistics."""
    k = torch.randn((n, cfg.B, cfg.H, cfg.D), generator=_gen(cfg, device, 3), device=device)
    v = torch.randn((n, cfg.B, cfg.H, cfg.D), generator=_gen(cfg, device, 4), device=device)
    ch = torch.as_tensor(outlier_channels(cfg), device=device)
    scale = torch.ones((cfg.H, cfg.D), device=device)
    scale.scatter_(1, ch, cfg.outlier_scale)
    return (k * scale[None, None]).to(torch.float16), v.to(torch.float16)


def queries(cfg: KiviConfig, device="cpu", n: int = 1) -> torch.Tensor:
    """Queries [n][B][Hq][D] fp16, N(0,1) (Hq = H unless the workload groups query heads)."""
    q = torch.randn((n, cfg.B, cfg.Hq or cfg.H, cfg.D), generator=_gen(cfg, device, 5), device=device)
    return q.to(torch.float16)


def softmax_scale(cfg: KiviConfig) -> float:
    return 1.0 / math.sqrt(cfg.D)
