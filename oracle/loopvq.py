"""LoopVQ decode attention, restated plainly in float64 (oracle; test infrastructure only).

Source: the LoopVQ page ("LoopVQ: Sub 1-bit KV Cache Quantization for Looped
Transformers").  Sections cited below:

* background, "vector quantization and codebooks": a D-dim cache vector is cut
  into sub-vectors, each class of sub-vector has a K = 2^b entry codebook,
  the cache stores the 8-bit index of the nearest entry
  a(z) = argmin_r ||z - e_r||^2, costing b/G bits per element;
* background, "RoPE": keys are quantized before RoPE and the attention kernel
  rotates every reconstructed key by its own position;
* background, "SGLang and Flash-Decoding": the KV sequence is cut into splits
  whose partial softmax results are merged exactly through logsumexp;
* "method steps", step 1: loop steps are cut into consecutive blocks of T_c
  (T_c divides T and G); coordinate i*T_c + m of the coupled vector of group g
  comes from loop step beta*T_c + m (the page counts steps from 1) and
  channel g*c + i, with c = G/T_c, i < c, m < T_c;
* "method steps", step 4 and Figure 5: the first 8 tokens (sinks) and the
  most recent 64 (256 at long context) stay bf16 at every loop step, every
  other token is stored as indices in 8-token pages, and the oldest recent
  page is encoded once every 8 generated tokens;
* "method steps", step 5, Figure 3 and Figure 5: loop step t reads the shared
  indices through its own slice B_t of each codeword, rebuilds the key,
  applies RoPE and scores it; index pages and bf16 pages are attended
  separately and merged through logsumexp.

Readings of points the page leaves open (each also listed in the design notes):
the channel subscript printed as "g_{c+i}" is read as g*c + i; loop steps
are counted from 0 here; RoPE is the rotate-half form pairing channel i with
i + D/2, theta_i = base^(-2i/D), angles at the absolute token position
counted from 0; the query is supplied already rotated; the attention output
is rounded to fp32 only by the caller of the oracle.

Key scale stream (TaSQ+LoopVQ, the page's limitations note: the keys carry an
extra fp16 scale of about 0.008 bit per element): read as one fp16 scale per
paged key token and loop step, shared by the heads (16 bits over H*D = 2048
elements at 16 heads of 128 channels), multiplying the reconstructed key; the
transform that produces the scales is not on the page, so they are inputs.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Sequence, Tuple

import numpy as np


# ---------------------------------------------------------------------------
# Geometry and bit accounting
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class Geometry:
    D: int
    T: int
    Tc: int
    G: int
    K: int = 256
    sink: int = 8
    window: int = 64
    page: int = 8

    def __post_init__(self):
        # "method steps", step 1: T_c must divide both T and G.
        if self.T % self.Tc or self.G % self.Tc:
            raise ValueError("T_c must divide T and G")
        if self.D % self.c:
            raise ValueError("c = G/T_c must divide D")

    @property
    def c(self) -> int:
        """Channels one codeword covers at one loop step."""
        return self.G // self.Tc

    @property
    def NG(self) -> int:
        """Index groups per token, per loop step: D / c."""
        return self.D // self.c

    @property
    def NB(self) -> int:
        """Loop blocks: T / T_c."""
        return self.T // self.Tc


def bits_per_element(G: int, index_bits: int = 8) -> float:
    """b/G bits per cached element (background, vector quantization).

    One b-bit index covers G elements: c channels at each of T_c loop steps
    ("core method": the coupled codeword keeps the same b/G cost)."""
    return index_bits / G


def block_of_step(t: int, Tc: int) -> Tuple[int, int]:
    """Loop step t (from 0) -> (block beta, position m inside the block)."""
    return t // Tc, t % Tc


# ---------------------------------------------------------------------------
# Loop-axis grouping, encode, dequant ("method steps", steps 1 and 4-5)
# ---------------------------------------------------------------------------

def couple(x_block: np.ndarray, G: int) -> np.ndarray:
    """Coupled sub-vectors of one loop block.

    x_block: [Tc][N][D], the values of the block's T_c loop steps.
    Returns z: [N][NG][G] with z[j, g, i*Tc + m] = x_block[m, j, g*c + i].
    """
    Tc, N, D = x_block.shape
    c = G // Tc
    NG = D // c
    z = np.empty((N, NG, G), dtype=np.float64)
    for g in range(NG):
        for i in range(c):
            for m in range(Tc):
                z[:, g, i * Tc + m] = x_block[m, :, g * c + i]
    return z


def nearest_codeword(z: np.ndarray, E: np.ndarray, chunk: int = 4096) -> Tuple[np.ndarray, np.ndarray]:
    """a(z) = argmin_r sum_k (z_k - E[r, k])^2 (background, vector quantization).

    z: [N][G], E: [K][G].  Distances are direct differences in float64 on the
    values as given; the scan keeps the first minimum, so the lowest index wins
    exact ties (numpy's argmin returns the first occurrence).
    Returns (indices [N] int64, distances [N][K]).
    """
    N, G = z.shape
    K = E.shape[0]
    d = np.zeros((N, K), dtype=np.float64)
    for lo in range(0, N, chunk):
        hi = min(N, lo + chunk)
        acc = d[lo:hi]
        for k in range(G):
            diff = z[lo:hi, k:k + 1] - E[None, :, k]
            acc += diff * diff
    return np.argmin(d, axis=1), d


def encode_block(x_block: np.ndarray, E_block: np.ndarray, G: int) -> np.ndarray:
    """Indices of one loop block: x_block [Tc][N][D], E_block [NG][K][G] -> [N][NG] uint8."""
    z = couple(np.asarray(x_block, dtype=np.float64), G)
    N, NG, _ = z.shape
    out = np.empty((N, NG), dtype=np.uint8)
    for g in range(NG):
        a, _ = nearest_codeword(z[:, g, :], np.asarray(E_block[g], dtype=np.float64))
        out[:, g] = a
    return out


def dequant_step(idx: np.ndarray, E_block: np.ndarray, m: int, Tc: int, G: int) -> np.ndarray:
    """Rebuild step m of a block from its indices through the step's slice B_t.

    idx: [N][NG]; E_block: [NG][K][G].  Channel g*c + i of token j is
    E_block[g, idx[j, g], i*Tc + m] (the inverse of `couple` at step m).
    """
    N, NG = idx.shape
    c = G // Tc
    out = np.empty((N, NG * c), dtype=np.float64)
    for g in range(NG):
        rows = np.asarray(E_block[g], dtype=np.float64)[idx[:, g].astype(np.int64)]  # [N][G]
        for i in range(c):
            out[:, g * c + i] = rows[:, i * Tc + m]
    return out


def step_slice(E_block: np.ndarray, m: int, Tc: int, G: int) -> np.ndarray:
    """B_t for t = beta*Tc + m: [NG][K][c] with B_t[g, r, i] = E_block[g, r, i*Tc + m]."""
    c = G // Tc
    NG, K, _ = E_block.shape
    out = np.empty((NG, K, c), dtype=np.asarray(E_block).dtype)
    for i in range(c):
        out[:, :, i] = E_block[:, :, i * Tc + m]
    return out


# ---------------------------------------------------------------------------
# Cache regions ("method steps", step 4; Figure 5)
# ---------------------------------------------------------------------------

def cache_regions(L: int, geo: Geometry) -> Tuple[int, int, int]:
    """Where the tokens of a request of length L live.

    Returns (n_pages, q_lo, q_hi): positions [0, min(L, sink)) are sinks,
    [q_lo, q_hi) = [sink, sink + page*n_pages) are index pages, [q_hi, L)
    are recent bf16 tokens.  A page is encoded once the recent part would
    hold window + page tokens, so the recent part keeps between window and
    window + page - 1 tokens once the context is long enough.
    """
    n_pages = max(0, (L - geo.sink - geo.window) // geo.page)
    q_lo = geo.sink
    q_hi = geo.sink + geo.page * n_pages
    return n_pages, q_lo, q_hi


def encode_request(raw: np.ndarray, E: np.ndarray, geo: Geometry, L: int) -> np.ndarray:
    """Indices of the paged tokens of one (request, head).

    raw: [L][T][D] pre-RoPE bf16 values (as floats); E: [NB][NG][K][G].
    Returns [NB][n_tok][NG] uint8 for the tokens [q_lo, q_hi)."""
    _, q_lo, q_hi = cache_regions(L, geo)
    out = np.zeros((geo.NB, q_hi - q_lo, geo.NG), dtype=np.uint8)
    if q_hi == q_lo:
        return out
    for beta in range(geo.NB):
        x_block = np.transpose(np.asarray(raw[q_lo:q_hi, beta * geo.Tc:(beta + 1) * geo.Tc, :], np.float64),
                               (1, 0, 2))
        out[beta] = encode_block(x_block, E[beta], geo.G)
    return out


def assemble_step(t: int, raw: np.ndarray, idx: np.ndarray, E: np.ndarray, geo: Geometry, L: int,
                  scales: np.ndarray = None) -> np.ndarray:
    """Pre-RoPE keys (or values) that loop step t attends over: [L][D] float64.

    Sinks and recent tokens come from the bf16 values of step t; paged tokens
    from their indices through B_t, each multiplied by its scale when `scales`
    ([n_tok] for step t, the key scale stream) is given."""
    _, q_lo, q_hi = cache_regions(L, geo)
    beta, m = block_of_step(t, geo.Tc)
    out = np.asarray(raw[:L, t, :], dtype=np.float64).copy()
    if q_hi > q_lo:
        out[q_lo:q_hi] = dequant_step(idx[beta], E[beta], m, geo.Tc, geo.G)
        if scales is not None:
            out[q_lo:q_hi] *= np.asarray(scales[:q_hi - q_lo], dtype=np.float64)[:, None]
    return out


# ---------------------------------------------------------------------------
# RoPE (background, "RoPE")
# ---------------------------------------------------------------------------

def rope_angles(positions: np.ndarray, D: int, base: float = 10000.0) -> np.ndarray:
    """phi[p, i] = p * base^(-2i/D) for i < D/2, float64."""
    i = np.arange(D // 2, dtype=np.float64)
    theta = np.power(float(base), -2.0 * i / D)
    return np.outer(np.asarray(positions, dtype=np.float64), theta)


def apply_rope(x: np.ndarray, positions: np.ndarray, base: float = 10000.0) -> np.ndarray:
    """Rotate-half RoPE of rows x [N][D] at the given positions:
    x'_i = x_i cos phi_i - x_{i+D/2} sin phi_i, x'_{i+D/2} = x_{i+D/2} cos phi_i + x_i sin phi_i."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[1]
    phi = rope_angles(positions, D, base)
    c, s = np.cos(phi), np.sin(phi)
    x1, x2 = x[:, :D // 2], x[:, D // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=1)


# ---------------------------------------------------------------------------
# Attention and the logsumexp merge (background, Flash-Decoding)
# ---------------------------------------------------------------------------

def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, sm_scale: float) -> Tuple[np.ndarray, float]:
    """Single-query softmax attention in float64.

    s_p = sm_scale * q . k_p;  o = sum_p e^{s_p - m} v_p / sum_p e^{s_p - m};
    lse = m + ln sum_p e^{s_p - m}, m = max_p s_p.  With no tokens: o = 0, lse = -inf."""
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if k.shape[0] == 0:
        return np.zeros(v.shape[1]), -np.inf
    s = sm_scale * (k @ np.asarray(q, dtype=np.float64))
    m = s.max()
    w = np.exp(s - m)
    l = w.sum()
    return (w @ v) / l, float(m + np.log(l))


def merge(parts: Sequence[Tuple[np.ndarray, float]]) -> Tuple[np.ndarray, float]:
    """Exact merge of split partials (o_s, lse_s): lse = M + ln sum_s e^{lse_s - M},
    o = sum_s e^{lse_s - lse} o_s, M = max_s lse_s.  Splits with lse = -inf add nothing."""
    lses = np.array([p[1] for p in parts], dtype=np.float64)
    M = lses.max()
    if M == -np.inf:
        return np.zeros_like(np.asarray(parts[0][0], dtype=np.float64)), -np.inf
    w = np.exp(lses - M)
    lse = M + np.log(w.sum())
    o = sum(np.exp(l - lse) * np.asarray(o_s, dtype=np.float64) for (o_s, l) in parts if l != -np.inf)
    return o, float(lse)


# ---------------------------------------------------------------------------
# One loop step of decode attention for one (request, head)
# ---------------------------------------------------------------------------

def decode_step(q: np.ndarray, t: int, raw_k: np.ndarray, raw_v: np.ndarray,
                idx_k: np.ndarray, idx_v: np.ndarray, E_k: np.ndarray, E_v: np.ndarray,
                geo: Geometry, L: int, sm_scale: float, base: float = 10000.0,
                k_scales: np.ndarray = None) -> Tuple[np.ndarray, float]:
    """Decode attention of the post-RoPE query q at loop step t over the whole cache.

    raw_k/raw_v: [>=L][T][D] bf16 values (sinks and recent tokens are read from
    them); idx_k/idx_v: [NB][n_tok][NG] indices of the paged tokens; E_k/E_v:
    [NB][NG][K][G] codebooks; k_scales: optional [n_tok][T] key scale stream of
    the paged tokens.  Keys are rotated at positions 0..L-1."""
    k = assemble_step(t, raw_k, idx_k, E_k, geo, L, None if k_scales is None else np.asarray(k_scales)[:, t])
    v = assemble_step(t, raw_v, idx_v, E_v, geo, L)
    k = apply_rope(k, np.arange(L), base)
    return attention(q, k, v, sm_scale)


def decode_step_permuted(q: np.ndarray, t: int, raw_k: np.ndarray, raw_v: np.ndarray,
                         idx_k: np.ndarray, idx_v: np.ndarray, E_k: np.ndarray, E_v: np.ndarray,
                         geo: Geometry, L: int, sm_scale: float, base: float, perm: np.ndarray
                         ) -> Tuple[np.ndarray, float]:
    """decode_step for a cache kept in a permuted channel order (LoopVQ page, technical novelty: with TaSQ, a
    channel permutation P is optimised together with the grouping).  perm[j] is the original channel stored
    at channel j; raw_k/raw_v, idx_k/idx_v and E_k/E_v describe the stored channels, q and the returned output
    are in the original channel order.  The keys and values are rebuilt in the stored order, put back in the
    original order, and then rotated and attended exactly as in decode_step."""
    perm = np.asarray(perm)
    k_st = assemble_step(t, raw_k, idx_k, E_k, geo, L)
    v_st = assemble_step(t, raw_v, idx_v, E_v, geo, L)
    k = np.empty_like(k_st)
    v = np.empty_like(v_st)
    k[:, perm] = k_st                                   # original channel perm[j] <- stored channel j
    v[:, perm] = v_st
    k = apply_rope(k, np.arange(L), base)
    return attention(q, k, v, sm_scale)


def decode_step_two_part(q, t, raw_k, raw_v, idx_k, idx_v, E_k, E_v, geo, L, sm_scale, base=10000.0):
    """The same result computed the way Figure 5 splits it: one partial over
    the index pages, one over the bf16 sinks and recent tokens, then `merge`."""
    k = apply_rope(assemble_step(t, raw_k, idx_k, E_k, geo, L), np.arange(L), base)
    v = assemble_step(t, raw_v, idx_v, E_v, geo, L)
    _, q_lo, q_hi = cache_regions(L, geo)
    quant = np.arange(q_lo, q_hi)
    bf16 = np.concatenate([np.arange(0, min(L, q_lo)), np.arange(q_hi, L)])
    return merge([attention(q, k[quant], v[quant], sm_scale),
                  attention(q, k[bf16], v[bf16], sm_scale)])

