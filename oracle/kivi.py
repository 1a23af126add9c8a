"""KIVI-style 2-bit asymmetric KV quantization and decode attention (oracle; test infrastructure only).

Source: the KIVI page ("KIVI 完全拆解：非对称 2-bit KV Cache 量化，为什么 Key
按通道、Value 按 token").  Sections cited below:

* background ("decoding is a bandwidth game"): the KV memory formula
  M = 2 * N_layer * H_kv * d_head * S * bytes, with the Llama-2-7B example of
  524,288 bytes per token;
* "definitions: per-token and per-channel": q = clamp(round(X/s + z), 0, 2^b - 1),
  X_hat = s * (q - z), the range [min, max] divided evenly by s; per-token
  groups share (s, z) along a row, per-channel groups along a column;
* "core design: grouped quantization + FP16 residual window": keys are
  quantized per channel in groups of G tokens, values per token; the newest
  tokens stay fp16 in a residual of at most R rows (G = 32, R = 128); the
  simplified pseudo-code gives prefill (tail R rows fp16) and decode (append to
  the residual; keys flush the residual once it reaches R rows, values
  quantize whatever overflows R); attention concatenates the logits of the
  quantized and the fp16 segments and takes ONE softmax over the
  concatenation; group parameters are fp16 (2 bytes each), 0.375 bytes per
  element at group 32;
* "engineering": splitting the softmax per segment is a pitfall; the
  normaliser must be shared.

Precision.  The pages fix fp16 storage for s and z and fp16 caches; they do
not say in which precision s, z and the code are computed.  A code is an
integer decided by floating point, so the oracle takes that decision in the
same precision as the device kernel: IEEE binary32 with round-to-nearest-even
for each +, -, *, / (numpy float32 arithmetic), no fused multiply-add,
rounding half to even for round().  Attention itself is float64.

Readings (also listed in the design notes):
* s = fp16(fl32(fl32(max - min) / 3)); if that is 0, s = 1 (constant group);
  z = fp16(fl32(-min / s)) using the stored fp16 s;
* prefill quantizes the first G*floor((L-R)/G) keys (so the tail of at least R
  keys stays fp16 and the quantized part is whole groups) and the first L-R
  values;
* decode, keys: after appending, once the residual holds R or more rows its
  oldest R rows (R/G whole groups) are quantized and dropped; in the steady
  state that is the page's "quantize the whole residual when it reaches R";
* decode, values: after appending, rows beyond the newest R are quantized.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Tuple

import numpy as np

F32 = np.float32
F16 = np.float16


# ---------------------------------------------------------------------------
# Accounting (background; core design)
# ---------------------------------------------------------------------------

def kv_cache_bytes(n_layer: int, h_kv: int, d_head: int, seq: int, bytes_per_elem: float) -> float:
    """M_KV = 2 * N_layer * H_kv * d_head * S * b (keys and values)."""
    return 2 * n_layer * h_kv * d_head * seq * bytes_per_elem


def bytes_per_element(bits: int = 2, group: int = 32, param_bytes: int = 2) -> float:
    """Code bits plus one fp16 scale and one fp16 zero-point shared by `group` elements."""
    return bits / 8 + 2 * param_bytes / group


# ---------------------------------------------------------------------------
# The quantizer ("definitions: per-token and per-channel")
# ---------------------------------------------------------------------------

def group_params(x: np.ndarray, bits: int = 2) -> Tuple[np.float16, np.float16]:
    """(s, z) of one group of fp16 values: s splits [min, max] into 2^b - 1 steps, z = -min/s."""
    xf = np.asarray(x, dtype=F16).astype(F32)
    mn, mx = xf.min(), xf.max()
    levels = F32(2 ** bits - 1)
    s = F16(F32(mx - mn) / levels)
    if s == F16(0):
        s = F16(1)
    z = F16(F32(-mn) / F32(s))
    return s, z


def quantize(x: np.ndarray, s, z, bits: int = 2) -> np.ndarray:
    """q = clamp(rint_even(fl32(fl32(x / s) + z)), 0, 2^b - 1) elementwise."""
    xf = np.asarray(x, dtype=F16).astype(F32)
    sf, zf = np.asarray(s, dtype=F16).astype(F32), np.asarray(z, dtype=F16).astype(F32)
    u = (xf / sf).astype(F32)
    u = (u + zf).astype(F32)
    return np.clip(np.rint(u), 0, 2 ** bits - 1).astype(np.uint8)


def dequantize(q: np.ndarray, s, z) -> np.ndarray:
    """X_hat = fl32(s * fl32(q - z)) as float32."""
    qf = np.asarray(q, dtype=F32)
    sf, zf = np.asarray(s, dtype=F16).astype(F32), np.asarray(z, dtype=F16).astype(F32)
    return (sf * (qf - zf).astype(F32)).astype(F32)


def quantize_keys(k: np.ndarray, group: int = 32, bits: int = 2):
    """Per-channel key quantization over whole groups of `group` tokens.

    k: [n][D] fp16 with n a multiple of `group`.  Returns codes [n][D] uint8,
    s [n/group][D] fp16, z [n/group][D] fp16."""
    n, D = k.shape
    assert n % group == 0
    codes = np.empty((n, D), dtype=np.uint8)
    s = np.empty((n // group, D), dtype=F16)
    z = np.empty((n // group, D), dtype=F16)
    for gi in range(n // group):
        rows = slice(gi * group, (gi + 1) * group)
        for d in range(D):
            s[gi, d], z[gi, d] = group_params(k[rows, d], bits)
            codes[rows, d] = quantize(k[rows, d], s[gi, d], z[gi, d], bits)
    return codes, s, z


def quantize_values(v: np.ndarray, group: int = 32, bits: int = 2):
    """Per-token value quantization over groups of `group` channels.

    v: [n][D] fp16.  Returns codes [n][D] uint8, s [n][D/group], z [n][D/group] fp16."""
    n, D = v.shape
    codes = np.empty((n, D), dtype=np.uint8)
    s = np.empty((n, D // group), dtype=F16)
    z = np.empty((n, D // group), dtype=F16)
    for j in range(n):
        for gi in range(D // group):
            cols = slice(gi * group, (gi + 1) * group)
            s[j, gi], z[j, gi] = group_params(v[j, cols], bits)
            codes[j, cols] = quantize(v[j, cols], s[j, gi], z[j, gi], bits)
    return codes, s, z


def dequantize_keys(codes, s, z, group: int = 32) -> np.ndarray:
    return dequantize(codes, np.repeat(s, group, axis=0), np.repeat(z, group, axis=0))


def dequantize_values(codes, s, z, group: int = 32) -> np.ndarray:
    return dequantize(codes, np.repeat(s, group, axis=1), np.repeat(z, group, axis=1))


# ---------------------------------------------------------------------------
# Cache state of one (request, head) ("core design", pseudo-code)
# ---------------------------------------------------------------------------

@dataclass
class KiviState:
    D: int = 128
    group: int = 32
    R: int = 128
    bits: int = 2                 # key code width
    v_bits: int = 0               # value code width (0: the same as the keys')
    k_codes: List[np.ndarray] = field(default_factory=list)   # blocks of [group][D]
    k_s: List[np.ndarray] = field(default_factory=list)       # blocks of [D]
    k_z: List[np.ndarray] = field(default_factory=list)
    k_res: List[np.ndarray] = field(default_factory=list)     # fp16 rows [D]
    v_codes: List[np.ndarray] = field(default_factory=list)   # rows [D]
    v_s: List[np.ndarray] = field(default_factory=list)       # rows [D/group]
    v_z: List[np.ndarray] = field(default_factory=list)
    v_res: List[np.ndarray] = field(default_factory=list)

    @property
    def n_kq(self) -> int:
        return self.group * len(self.k_codes)

    @property
    def n_vq(self) -> int:
        return len(self.v_codes)

    @property
    def length(self) -> int:
        return self.n_kq + len(self.k_res)

    def _flush_keys(self, n_rows: int):
        block = np.stack(self.k_res[:n_rows]).astype(F16)
        codes, s, z = quantize_keys(block, self.group, self.bits)
        for gi in range(n_rows // self.group):
            self.k_codes.append(codes[gi * self.group:(gi + 1) * self.group])
            self.k_s.append(s[gi])
            self.k_z.append(z[gi])
        del self.k_res[:n_rows]

    def _flush_values(self, n_rows: int):
        block = np.stack(self.v_res[:n_rows]).astype(F16)
        codes, s, z = quantize_values(block, self.group, self.v_bits or self.bits)
        for j in range(n_rows):
            self.v_codes.append(codes[j])
            self.v_s.append(s[j])
            self.v_z.append(z[j])
        del self.v_res[:n_rows]

    def prefill(self, k: np.ndarray, v: np.ndarray):
        """Prefill of an empty cache with L tokens: k, v [L][D] fp16."""
        assert self.length == 0
        L = k.shape[0]
        n_kq = self.group * max(0, (L - self.R) // self.group)
        n_vq = max(0, L - self.R)
        self.k_res = [np.asarray(r, dtype=F16) for r in k]
        self.v_res = [np.asarray(r, dtype=F16) for r in v]
        if n_kq:
            self._flush_keys(n_kq)
        if n_vq:
            self._flush_values(n_vq)

    def append(self, k: np.ndarray, v: np.ndarray):
        """One decode token: k, v [D] fp16."""
        self.k_res.append(np.asarray(k, dtype=F16))
        if len(self.k_res) >= self.R:
            self._flush_keys(self.R)
        self.v_res.append(np.asarray(v, dtype=F16))
        if len(self.v_res) > self.R:
            self._flush_values(len(self.v_res) - self.R)

    def keys(self) -> np.ndarray:
        """All keys as attention sees them: dequantized segment then fp16 residual, [L][D] float64."""
        parts = []
        if self.k_codes:
            parts.append(dequantize_keys(np.concatenate(self.k_codes), np.stack(self.k_s),
                                         np.stack(self.k_z), self.group).astype(np.float64))
        if self.k_res:
            parts.append(np.stack(self.k_res).astype(np.float64))
        return np.concatenate(parts) if parts else np.zeros((0, self.D))

    def values(self) -> np.ndarray:
        parts = []
        if self.v_codes:
            parts.append(dequantize_values(np.stack(self.v_codes), np.stack(self.v_s),
                                           np.stack(self.v_z), self.group).astype(np.float64))
        if self.v_res:
            parts.append(np.stack(self.v_res).astype(np.float64))
        return np.concatenate(parts) if parts else np.zeros((0, self.D))


def attention(q: np.ndarray, state: KiviState, sm_scale: float) -> Tuple[np.ndarray, float]:
    """Decode attention over both segments with one softmax over the concatenated logits.

    Returns (o [D] float64, lse)."""
    k, v = state.keys(), state.values()
    s = sm_scale * (k @ np.asarray(q, dtype=np.float64))
    m = s.max()
    w = np.exp(s - m)
    l = w.sum()
    return (w @ v) / l, float(m + np.log(l))


def attention_per_segment_softmax(q: np.ndarray, state: KiviState, sm_scale: float) -> np.ndarray:
    """The pitfall the page warns about (each segment normalised on its own,
    outputs added).  Kept only as a negative control for the tests."""
    k, v = state.keys(), state.values()
    n_q = state.n_kq
    out = np.zeros(state.D)
    for sl in (slice(0, n_q), slice(n_q, k.shape[0])):
        if sl.stop > sl.start:
            s = sm_scale * (k[sl] @ np.asarray(q, np.float64))
            w = np.exp(s - s.max())
            out += (w / w.sum()) @ v[sl]
    return out
