"""Seeded synthetic inputs for quantized-KV decode attention.

This package draws random numbers and nothing else: token bases plus
per-loop-step noise, N(0,1) codebooks, queries, ragged request lengths and
page permutations.  It holds no arithmetic of the quantisation or attention
methods, so both the fp64 oracle and the HIP path can take their inputs from
it without sharing any of the computation under test.

Shapes and statistics follow the workloads of the two pages this project is
built from:

* LoopVQ (Cheong & Yoo, "LoopVQ: Sub 1-bit KV Cache Quantization for Looped
  Transformers"): looped models run T loop steps per layer and the same
  token's key/value at adjacent loop steps are strongly correlated (the
  "research motivation" section gives 0.69 rising to 0.94 across the loop,
  and about 0.85 for one channel at adjacent steps).  Serving is measured at
  batch 64 with 6K context (method step 5) and at 32K context.
* KIVI ("KIVI 完全拆解" walkthrough): keys carry a few fixed outlier channels
  across all tokens, values have no such structure (the "distribution
  evidence" section).
"""

from .configs import (  # noqa: F401
    LoopVQConfig,
    KiviConfig,
    LOOPVQ_CONFIGS,
    KIVI_CONFIGS,
    loopvq_config,
    kivi_config,
)
