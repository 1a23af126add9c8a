"""Streaming decode over a LoopVQ cache (the LoopVQ page, "method steps" step 4 and Figure 5).

Each generated token adds, at every loop step, its pre-RoPE bf16 K and V to the recent window
(lvq_window_append) and is attended with that step's query (lvq_decode_attn); after every 8 tokens the
window's oldest page is encoded into the index pool (lvq_encode reading the window ring through its
strides) and leaves the window.  This class keeps the per-request lengths on the host, decides which
requests complete a page, and issues the library calls on one stream; every step of the path runs in
the library's kernels.
"""

from __future__ import annotations

from typing import Optional, Sequence

import numpy as np
import torch

from . import lvq_decode_attn, lvq_decode_attn_workspace, lvq_encode, lvq_request_order, lvq_window_append
from .layout import LoopVQCache, n_index_pages


class LoopVQStream:
    """Decode state of a batch: `cache` is allocated for the final lengths (page table and pool hold
    every page the stream will write), and holds the first `lengths[b]` tokens of each request (index
    pages encoded, window filled)."""

    def __init__(self, cache: LoopVQCache, codebooks: torch.Tensor, slices: torch.Tensor,
                 rope_cos: torch.Tensor, rope_sin: torch.Tensor, rope16: Optional[torch.Tensor],
                 sm_scale: float, lengths: Sequence[int], stream=None):
        g = cache.g
        self.g, self.cache = g, cache
        self.codebooks, self.slices = codebooks, slices
        self.rope_cos, self.rope_sin, self.rope16 = rope_cos, rope_sin, rope16
        self.sm_scale = float(sm_scale)
        self.stream = stream
        self.B = cache.B
        self.len = np.asarray(lengths, dtype=np.int64).copy()
        if self.len.shape != (self.B,) or (self.len < 0).any():
            raise ValueError("one non-negative length per request")
        cap = np.asarray([n_index_pages(L, g) for L in cache.lengths])
        self.cap_pages = cap
        self.dev = cache.seq_len.device
        self._set_lengths()
        self.order: Optional[torch.Tensor] = None
        self.ws: Optional[torch.Tensor] = None
        # encode arguments: one page per request that completes one
        self._first = torch.zeros(self.B, dtype=torch.int32, device=self.dev)
        self._npg = torch.zeros(self.B, dtype=torch.int32, device=self.dev)
        self._tok0 = torch.zeros(self.B, dtype=torch.int64, device=self.dev)

    @property
    def max_len(self) -> int:
        return int(self.len.max()) if self.B else 0

    def _set_lengths(self):
        self.cache.seq_len.copy_(torch.from_numpy(self.len.astype(np.int32)), non_blocking=False)

    def begin_token(self, reorder: bool = False):
        """Count one new token for every request; encode the index page that it completes (the window's
        oldest, every block, K and V).  Call once per generated token, before its loop steps."""
        g = self.g
        new = self.len + 1
        n_old = np.maximum(0, (self.len - g.sink - g.window) // g.page)
        n_new = np.maximum(0, (new - g.sink - g.window) // g.page)
        if (n_new > self.cap_pages).any():
            raise ValueError("a request outgrows the page table it was allocated with")
        grow = n_new > n_old
        self.len = new
        self._set_lengths()
        if grow.any():
            lp = np.where(grow, n_new - 1, 0)
            p0 = g.sink + g.page * lp                                  # first position of the page
            slot0 = g.sink + (p0 - g.sink) % (g.window + g.page)       # its first window slot (8 in a row)
            self._first.copy_(torch.from_numpy(lp.astype(np.int32)))
            self._npg.copy_(torch.from_numpy(grow.astype(np.int32)))
            self._tok0.copy_(torch.from_numpy(np.where(grow, slot0, 0).astype(np.int64)))
            c = self.cache
            for beta in range(g.T // g.Tc):
                xk = c.win_k[:, beta * g.Tc:(beta + 1) * g.Tc].permute(0, 2, 3, 1, 4)   # [B][H][slot][Tc][D]
                xv = c.win_v[:, beta * g.Tc:(beta + 1) * g.Tc].permute(0, 2, 3, 1, 4)
                lvq_encode(g, beta, xk, xv, self.codebooks, c.pool, c.page_table, self._first, self._npg, 1,
                           x_tok0=self._tok0, stream=self.stream)
        if reorder:
            self.order = lvq_request_order(self.cache.seq_len, self.max_len, out=self.order, stream=self.stream)
        return grow

    def append(self, t: int, k: Optional[torch.Tensor], v: Optional[torch.Tensor]):
        """The current token's pre-RoPE K and V ([B][H][D] bf16) of loop step t into the window."""
        lvq_window_append(self.g, t, k, v, self.cache, self.max_len, stream=self.stream)

    def attend(self, t: int, q: torch.Tensor, out: Optional[torch.Tensor] = None,
               lse_out: Optional[torch.Tensor] = None, num_splits: int = 0):
        """Attention of loop step t for the current token (q post-RoPE, [B][H][D] bf16)."""
        c = self.cache
        need = lvq_decode_attn_workspace(self.g, self.B, self.max_len, num_splits)
        if self.ws is None or self.ws.numel() < need:
            self.ws = torch.empty(max(need, 256), dtype=torch.uint8, device=self.dev)
        return lvq_decode_attn(self.g, t, q, c.pool, c.page_table, c.seq_len, self.max_len, c.win_k, c.win_v,
                               self.slices, self.rope_cos, self.rope_sin, self.sm_scale, out=out, lse_out=lse_out,
                               ws=self.ws, num_splits=num_splits, stream=self.stream, rope_f16=self.rope16,
                               order=self.order)
