"""Workload descriptions (plain parameters, no derived arithmetic).

Every workload is named by what it is.  The LoopVQ ones use the layout
parameters of the LoopVQ page (method step 4: 8 sink tokens, a recent window
of 64 tokens, 256 at long context, 8-token index pages; K=256 codewords so
indices are 8-bit); the KIVI one uses the KIVI page's group size 32 and
residual length 128 (core-design section).
"""

from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional, Tuple


@dataclass(frozen=True)
class LoopVQConfig:
    name: str
    B: int                      # requests
    H: int                      # KV heads (multi-head attention: q heads == KV heads)
    T: int                      # loop steps
    Tc: int                     # loop steps sharing one index row
    G: int                      # codeword dimension
    L: int                      # context length (max over requests when ragged)
    D: int = 128
    K: int = 256                # codewords per codebook
    sink: int = 8
    window: int = 64
    page: int = 8
    cb_dtype: str = "bf16"      # "bf16" | "fp32"
    rope_base: float = 10000.0
    q_prescaled: bool = False   # q ~ N(0,1)/sqrt(D) with softmax scale 1 (else N(0,1), scale 1/sqrt(D))
    corr: Tuple = ("equi", 0.85)        # ("equi", rho) or ("ar1", rho_first, rho_last)
    ragged: Optional[Tuple[int, int]] = None   # (lo, hi) for log-uniform lengths
    random_pages: bool = False  # physical page ids in seeded random order
    seed: int = 0


@dataclass(frozen=True)
class KiviConfig:
    name: str
    B: int
    H: int
    L: int
    D: int = 128
    bits: int = 2               # key code width
    v_bits: int = 0             # value code width (0: as the keys)
    Hq: int = 0                 # query heads (0: one per KV head; a multiple of H for grouped-query attention)
    group: int = 32             # tokens per key group (per-channel) and channels per value group (per-token)
    R: int = 128                # residual length kept in fp16
    n_outlier: int = 4          # fixed outlier key channels per head
    outlier_scale: float = 20.0
    seed: int = 0


# The five workloads.  `loopvq-b64-6k` is the serving-scale headline.
LOOPVQ_CONFIGS = {
    # 0.5 bit per element, batch 1, one head, fp32 codebooks, 1K context.
    "loopvq-b1-1k-fp32cb": LoopVQConfig(
        name="loopvq-b1-1k-fp32cb", B=1, H=1, T=4, Tc=2, G=16, L=1024,
        cb_dtype="fp32", q_prescaled=True, seed=1001),
    # 0.5 bit per element, batch 64, 16 heads, 6K context (two requests per workgroup).
    "loopvq-b64-6k": LoopVQConfig(
        name="loopvq-b64-6k", B=64, H=16, T=4, Tc=2, G=16, L=6144, seed=1003),
    # 0.25 bit per element, batch 8, 32K context, 256-token recent window.
    "loopvq-b8-32k": LoopVQConfig(
        name="loopvq-b8-32k", B=8, H=16, T=4, Tc=4, G=32, L=32768, window=256, seed=1004),
    # 32 loop steps, ragged lengths log-uniform in [1024, 16384], random page order.
    "loopvq-deep-ragged": LoopVQConfig(
        name="loopvq-deep-ragged", B=128, H=8, T=32, Tc=4, G=16, L=16384,
        corr=("ar1", 0.69, 0.94), ragged=(1024, 16384), random_pages=True, seed=1005),
}

KIVI_CONFIGS = {
    "kivi-b16-4k": KiviConfig(name="kivi-b16-4k", B=16, H=32, L=4096, seed=1002),
    # the page's variants: 4-bit codes (KIVI-4), and grouped-query attention (32 query heads over 8 KV heads)
    "kivi4-b16-4k": KiviConfig(name="kivi4-b16-4k", B=16, H=32, L=4096, bits=4, seed=1004),
    "kivi-gqa-b16-4k": KiviConfig(name="kivi-gqa-b16-4k", B=16, H=8, Hq=32, L=4096, seed=1005),
}


def loopvq_config(name: str, **overrides) -> LoopVQConfig:
    """A named workload, optionally with fields overridden (reduced test sizes)."""
    return replace(LOOPVQ_CONFIGS[name], **overrides) if overrides else LOOPVQ_CONFIGS[name]


def kivi_config(name: str, **overrides) -> KiviConfig:
    return replace(KIVI_CONFIGS[name], **overrides) if overrides else KIVI_CONFIGS[name]
