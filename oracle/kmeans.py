"""Fisher-weighted k-means codebook initialisation, restated plainly in float64 (oracle; test
infrastructure only).

Source: the LoopVQ page ("LoopVQ: Sub 1-bit KV Cache Quantization for Looped Transformers"):

* background, "Fisher-weighted k-means": plain k-means treats every sub-vector alike; the weighted
  form multiplies the error of sub-vector n by a scalar weight w_n (the squared norm of the loss
  gradient with respect to it, the diagonal of the empirical Fisher information), so errors on
  sensitive sub-vectors cost more;
* "method steps", step 2: the codebooks B_{beta, layer, head, group} are initialised by this weighted
  k-means (Eq. 3), the weight of a coupled vector summing the squared gradients of the T_c loop steps
  it covers.

Objective: J(E) = sum_n w_n ||z_n - e_{a(n)}||^2 with a(n) the nearest codeword.  A scalar weight
scales all of sample n's distances alike, so the assignment is the plain nearest codeword; for fixed
assignments J is minimised by the weighted mean of each cluster, e_r = sum_{a(n)=r} w_n z_n /
sum_{a(n)=r} w_n (Lloyd's two steps, each of which cannot raise J).  Readings where the page is silent:
a codeword whose cluster has zero total weight keeps its value; the weights are supplied (the page
derives them from gradients of a trained model, which is not available here).
"""

from __future__ import annotations

from typing import Tuple

import numpy as np

from .loopvq import nearest_codeword


def weighted_update(z: np.ndarray, w: np.ndarray, a: np.ndarray, E: np.ndarray) -> np.ndarray:
    """One update step: e_r = sum_{a(n)=r} w_n z_n / sum_{a(n)=r} w_n, kept when that sum is zero.

    z [N][G], w [N] >= 0, a [N] codeword of each sample, E [K][G] the current codebook."""
    K, G = E.shape
    num = np.zeros((K, G), dtype=np.float64)
    den = np.zeros(K, dtype=np.float64)
    for n in range(z.shape[0]):
        num[a[n]] += w[n] * z[n]
        den[a[n]] += w[n]
    out = E.astype(np.float64).copy()
    nz = den > 0
    out[nz] = num[nz] / den[nz, None]
    return out


def objective(z: np.ndarray, w: np.ndarray, E: np.ndarray) -> float:
    """J(E) = sum_n w_n min_r ||z_n - e_r||^2."""
    a, d = nearest_codeword(z, E)
    return float(np.sum(w * d[np.arange(z.shape[0]), a]))


def lloyd_step(z: np.ndarray, w: np.ndarray, E: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Assignment (nearest codeword, lowest index on ties) then the weighted update.
    Returns (new codebook, assignments)."""
    a, _ = nearest_codeword(z, E)
    return weighted_update(z, w, a, E), a


def weighted_kmeans(z: np.ndarray, w: np.ndarray, E0: np.ndarray, iters: int) -> np.ndarray:
    """`iters` Lloyd steps from E0."""
    E = E0.astype(np.float64)
    for _ in range(iters):
        E, _ = lloyd_step(z, w, E)
    return E
