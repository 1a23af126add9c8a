"""Seeded random draws for the LoopVQ workloads (torch; any device).

Only random numbers are produced here.  The layout of the cache (which
tokens are sinks, pages or recent) and every step of the method are left to
the consumers.

Streams are deterministic for a given (config seed, device type); the CPU
and the GPU generators give different streams, so a test that compares two
implementations draws once and hands the same tensors to both.
"""

from __future__ import annotations

import math
from typing import Iterator, List, Tuple

import numpy as np
import torch

from .configs import LoopVQConfig

_KIND = {"k": 1, "v": 2, "q": 3, "cb": 4, "base": 5}


def _seed(cfg: LoopVQConfig, *parts: int) -> int:
    s = cfg.seed * 1_000_003
    for p in parts:
        s = (s * 7919 + int(p) + 1) % (2**62)
    return s


def _gen(cfg: LoopVQConfig, device, *parts: int) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(_seed(cfg, *parts))
    return g


def lengths(cfg: LoopVQConfig) -> List[int]:
    """Per-request context lengths: all cfg.L, or floor(exp(U(ln lo, ln hi))) when ragged."""
    if cfg.ragged is None:
        return [cfg.L] * cfg.B
    lo, hi = cfg.ragged
    rng = np.random.default_rng(_seed(cfg, 11))
    u = rng.uniform(math.log(lo), math.log(hi), size=cfg.B)
    return [int(min(hi, max(lo, math.floor(math.exp(x))))) for x in u]


def page_permutation(cfg: LoopVQConfig, n_phys: int) -> np.ndarray:
    """A seeded permutation of physical page ids (identity unless cfg.random_pages)."""
    if not cfg.random_pages:
        return np.arange(n_phys, dtype=np.int64)
    rng = np.random.default_rng(_seed(cfg, 12))
    return rng.permutation(n_phys).astype(np.int64)


def _rho(cfg: LoopVQConfig, t: int) -> float:
    """Correlation between loop steps t and t+1 for the AR(1) model: linear from first to last pair."""
    _, r0, r1 = cfg.corr
    if cfg.T <= 2:
        return r0
    return r0 + (r1 - r0) * t / (cfg.T - 2)


def raw_blocks(cfg: LoopVQConfig, kind: str, device="cpu",
               batch: slice = slice(None)) -> Iterator[Tuple[int, torch.Tensor]]:
    """Yield (beta, x) for beta = 0 .. T/Tc-1 with x: bf16 [B][H][L][Tc][D].

    x[b, h, p, m] is the pre-RoPE key (kind "k") or value ("v") of token p of
    request b, head h at loop step beta*Tc + m.  Two data models:

    * ("equi", rho): per-token base z ~ N(0,1)^D shared by all loop steps and
      x_t = sqrt(rho) z + sqrt(1-rho) eps_t, so any two steps correlate at rho.
    * ("ar1", r0, r1): x_0 ~ N(0,1), x_{t+1} = rho_t x_t + sqrt(1-rho_t^2) eps,
      rho_t linear from r0 (first pair) to r1 (last pair).

    Draws are made per block for the whole batch and then sliced by `batch`,
    so a slice sees exactly the rows the full draw would have.
    """
    assert kind in ("k", "v")
    kid = _KIND[kind]
    B, H, L, D, T, Tc = cfg.B, cfg.H, cfg.L, cfg.D, cfg.T, cfg.Tc
    shape = (B, H, L, D)
    nb = T // Tc
    if cfg.corr[0] == "equi":
        rho = float(cfg.corr[1])
        base = torch.randn(shape, generator=_gen(cfg, device, kid, _KIND["base"]),
                           device=device, dtype=torch.float32)[batch]
        a, b_ = math.sqrt(rho), math.sqrt(1.0 - rho)
        for beta in range(nb):
            g = _gen(cfg, device, kid, 100 + beta)
            steps = []
            for m in range(Tc):
                eps = torch.randn(shape, generator=g, device=device, dtype=torch.float32)[batch]
                steps.append((a * base + b_ * eps).to(torch.bfloat16))
                del eps
            yield beta, torch.stack(steps, dim=3)
            del steps
    elif cfg.corr[0] == "ar1":
        prev = None
        for beta in range(nb):
            g = _gen(cfg, device, kid, 100 + beta)
            steps = []
            for m in range(Tc):
                t = beta * Tc + m
                eps = torch.randn(shape, generator=g, device=device, dtype=torch.float32)[batch]
                if prev is None:
                    cur = eps
                else:
                    r = _rho(cfg, t - 1)
                    cur = r * prev + math.sqrt(1.0 - r * r) * eps
                    del eps
                steps.append(cur.to(torch.bfloat16))
                prev = cur
            yield beta, torch.stack(steps, dim=3)
            del steps
    else:
        raise ValueError(cfg.corr)


def raw_kv(cfg: LoopVQConfig, device="cpu", batch: slice = slice(None)) -> Tuple[torch.Tensor, torch.Tensor]:
    """All loop steps at once: (k, v) bf16 [B][H][L][T][D].  Only for small workloads."""
    out = []
    for kind in ("k", "v"):
        blocks = [x for _, x in raw_blocks(cfg, kind, device, batch)]
        out.append(torch.cat(blocks, dim=3))
    return out[0], out[1]


def codebooks(cfg: LoopVQConfig, device="cpu") -> torch.Tensor:
    """Codebooks [T/Tc][H][2 (K,V)][D*Tc/G][K][G], entries N(0,1), in cfg.cb_dtype."""
    nb, ng = cfg.T // cfg.Tc, cfg.D * cfg.Tc // cfg.G
    x = torch.randn((nb, cfg.H, 2, ng, cfg.K, cfg.G), generator=_gen(cfg, device, _KIND["cb"]),
                    device=device, dtype=torch.float32)
    return x.to(torch.bfloat16) if cfg.cb_dtype == "bf16" else x


def queries(cfg: LoopVQConfig, device="cpu") -> torch.Tensor:
    """Post-RoPE queries [T][B][H][D] bf16: N(0,1), or N(0,1)/sqrt(D) when cfg.q_prescaled."""
    x = torch.randn((cfg.T, cfg.B, cfg.H, cfg.D), generator=_gen(cfg, device, _KIND["q"]),
                    device=device, dtype=torch.float32)
    if cfg.q_prescaled:
        x = x / math.sqrt(cfg.D)
    return x.to(torch.bfloat16)


def softmax_scale(cfg: LoopVQConfig) -> float:
    return 1.0 if cfg.q_prescaled else 1.0 / math.sqrt(cfg.D)
