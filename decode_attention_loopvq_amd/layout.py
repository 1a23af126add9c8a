"""LoopVQ cache layout: sizes, slot mapping and allocation (torch plumbing).

The layout is the one include/lvq.h documents.  Tokens of a request of
length L: sinks [0, sink), index pages [sink, sink + 8*n_pages) with
n_pages = max(0, (L - sink - W) // 8), recent bf16 tokens after that (the
LoopVQ page, "method steps" step 4 and Figure 5: 8 sinks, a recent window of
64 or 256 tokens, 8-token index pages, one page encoded per 8 generated
tokens).
"""

from __future__ import annotations

from typing import Optional, Sequence

import numpy as np
import torch

from ._lib import LVQ_BF16, lvq_geom


def n_index_pages(L: int, g: lvq_geom) -> int:
    return max(0, (L - g.sink - g.window) // g.page)


def window_capacity(g: lvq_geom) -> int:
    return g.sink + g.window + g.page


def window_slot(p, g: lvq_geom):
    """Window slot of absolute position p (scalar or numpy array)."""
    p = np.asarray(p)
    return np.where(p < g.sink, p, g.sink + (p - g.sink) % (g.window + g.page))


def window_positions(L: int, g: lvq_geom) -> np.ndarray:
    """Positions held in the bf16 window for a request of length L: sinks then recent tokens."""
    hi = g.sink + g.page * n_index_pages(L, g)
    return np.concatenate([np.arange(min(L, g.sink)), np.arange(hi, L)]).astype(np.int64)


def index_groups(g: lvq_geom) -> int:
    return g.D // (g.G // g.Tc)


def page_bytes(g: lvq_geom) -> int:
    return (g.T // g.Tc) * g.H * 2 * g.page * index_groups(g)


class LoopVQCache:
    """Device buffers of a LoopVQ cache for B requests.

    pool        uint8 [P][NB][H][2][page][NG]
    page_table  int32 [B][max_pages]
    win_k/win_v bf16  [B][T][H][sink+W+page][D]
    seq_len     int32 [B]
    """

    def __init__(self, g: lvq_geom, lengths: Sequence[int], device="cuda",
                 phys_perm: Optional[np.ndarray] = None):
        self.g = g
        self.lengths = [int(x) for x in lengths]
        self.B = len(self.lengths)
        self.max_len = max(self.lengths)
        self.n_pages = [n_index_pages(L, g) for L in self.lengths]
        self.max_pages = max(self.n_pages) if self.n_pages else 0
        total = sum(self.n_pages)
        self.n_phys = max(1, total)
        perm = np.arange(self.n_phys) if phys_perm is None else np.asarray(phys_perm)
        assert len(perm) >= total
        pt = np.zeros((self.B, max(1, self.max_pages)), dtype=np.int32)
        off = 0
        for b, n in enumerate(self.n_pages):
            pt[b, :n] = perm[off:off + n]
            off += n
        NG, NB = index_groups(g), g.T // g.Tc
        self.pool = torch.zeros((self.n_phys, NB, g.H, 2, g.page, NG), dtype=torch.uint8, device=device)
        self.page_table = torch.from_numpy(pt).to(device)
        self.page_table_host = pt
        wshape = (self.B, g.T, g.H, window_capacity(g), g.D)
        self.win_k = torch.zeros(wshape, dtype=torch.bfloat16, device=device)
        self.win_v = torch.zeros(wshape, dtype=torch.bfloat16, device=device)
        self.seq_len = torch.tensor(self.lengths, dtype=torch.int32, device=device)
        self.first_page = torch.zeros((self.B,), dtype=torch.int32, device=device)
        self.n_pages_dev = torch.tensor(self.n_pages, dtype=torch.int32, device=device)
        self.tok0 = torch.full((self.B,), g.sink, dtype=torch.int64, device=device)


def cb_torch_dtype(g: lvq_geom):
    return torch.bfloat16 if g.cb_dtype == LVQ_BF16 else torch.float32
