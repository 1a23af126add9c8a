"""Builds LoopVQ / KIVI problems on the GPU from the seeded generators.

Used by the GPU tests and by bench.py.  It drives only the HIP library (and
torch for allocation and copies); it never imports the oracle.  Rows picked
for checking are copied back to the host as raw bf16 values so that the
oracle can recompute them independently.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Sequence, Tuple

import numpy as np
import torch

import decode_attention_loopvq_amd as lvq
from decode_attention_loopvq_amd.layout import LoopVQCache, n_index_pages
from synth import loopvq as syn
from synth import kivi as synk
from synth.configs import KiviConfig, LoopVQConfig


@dataclass
class LoopVQProblem:
    cfg: LoopVQConfig
    g: object
    lengths: List[int]
    cache: LoopVQCache
    codebooks: torch.Tensor
    slices: torch.Tensor
    rope_cos: torch.Tensor
    rope_sin: torch.Tensor
    rope16: torch.Tensor                  # packed fp16 table for the index-page pass
    q: torch.Tensor                       # [T][B][H][D] bf16
    sm_scale: float
    raw: Dict[Tuple[str, int, int], np.ndarray] = field(default_factory=dict)   # (kind, b, h) -> [L][T][D] f64


def geom_of(cfg: LoopVQConfig):
    return lvq.make_geom(D=cfg.D, T=cfg.T, Tc=cfg.Tc, G=cfg.G, K=cfg.K, page=cfg.page, sink=cfg.sink,
                         window=cfg.window, H=cfg.H, cb_dtype=cfg.cb_dtype)


def build_loopvq(cfg: LoopVQConfig, device="cuda", keep: Sequence[Tuple[int, int]] = (),
                 batch_chunk: int = 0) -> LoopVQProblem:
    """Draw the workload, encode every index page with lvq_encode and fill the
    bf16 window.  `keep` lists (b, h) rows whose raw values are copied to the host."""
    g = geom_of(cfg)
    lengths = syn.lengths(cfg)
    total_pages = sum(n_index_pages(L, g) for L in lengths)
    perm = syn.page_permutation(cfg, max(1, total_pages))
    cache = LoopVQCache(g, lengths, device=device, phys_perm=perm)
    codebooks = syn.codebooks(cfg, device)
    slices = lvq.lvq_slice_codebooks(g, codebooks)
    rope_cos, rope_sin = lvq.lvq_rope_table(cache.max_len, cfg.D, cfg.rope_base, device=device)
    rope16 = lvq.lvq_rope_table_f16(cache.max_len, cfg.D, cfg.rope_base, device=device)
    raw = {}
    keep = list(keep)
    for kind in ("k", "v"):
        host_steps = {key: [] for key in keep}
        for beta, x in syn.raw_blocks(cfg, kind, device):
            x_k = x if kind == "k" else None
            x_v = x if kind == "v" else None
            lvq.lvq_encode(g, beta, x_k, x_v, codebooks, cache.pool, cache.page_table, cache.first_page,
                           cache.n_pages_dev, cache.max_pages, x_tok0=cache.tok0)
            _fill_window(cache, beta, x, kind)
            for (b, h) in keep:
                host_steps[(b, h)].append(x[b, h, :lengths[b]].float().cpu().numpy())
            del x, x_k, x_v
        for (b, h) in keep:
            raw[(kind, b, h)] = np.concatenate(host_steps[(b, h)], axis=1).astype(np.float64)
    q = syn.queries(cfg, device)
    torch.cuda.synchronize()
    return LoopVQProblem(cfg, g, lengths, cache, codebooks, slices, rope_cos, rope_sin, rope16, q,
                         syn.softmax_scale(cfg), raw)


def _fill_window(cache: LoopVQCache, beta: int, x: torch.Tensor, kind: str, lengths=None):
    g = cache.g
    win = cache.win_k if kind == "k" else cache.win_v
    from decode_attention_loopvq_amd.layout import window_positions, window_slot
    groups: Dict[int, List[int]] = {}
    for b, L in enumerate(cache.lengths if lengths is None else lengths):
        groups.setdefault(L, []).append(b)
    for L, bs in groups.items():
        pos = window_positions(L, g)
        slots = torch.from_numpy(window_slot(pos, g)).to(x.device)
        posd = torch.from_numpy(pos).to(x.device)
        bidx = torch.tensor(bs, device=x.device)
        for m in range(g.Tc):
            t = beta * g.Tc + m
            sub = x[:, :, posd, m].index_select(0, bidx)          # [nb][H][npos][D]
            tmp = win[:, t].index_select(0, bidx)                # [nb][H][Wcap][D]
            tmp[:, :, slots] = sub
            win[:, t].index_copy_(0, bidx, tmp)


def gpu_indices(p: LoopVQProblem, b: int, h: int, kind: str) -> np.ndarray:
    """Indices the GPU wrote for (b, h): [NB][n_tok][NG] uint8."""
    g = p.g
    n = p.cache.n_pages[b]
    pages = p.cache.page_table_host[b, :n]
    kv = 0 if kind == "k" else 1
    sel = p.cache.pool[torch.as_tensor(pages, dtype=torch.long, device=p.cache.pool.device)]  # [n][NB][H][2][8][NG]
    sel = sel[:, :, h, kv]                                                                   # [n][NB][8][NG]
    NB, NG = sel.shape[1], sel.shape[3]
    rows = sel.permute(1, 0, 2, 3).reshape(NB, n * g.page, NG).cpu().numpy()
    tau = np.arange(n * g.page)[:, None]
    grp = np.arange(NG)[None, :]
    return rows[:, tau, index_byte(kind, NG, grp, tau)]


def index_byte(kind: str, NG: int, grp, tau):
    """Byte position of group `grp` in the index row of index-token `tau` (the pool layout of lvq.h): value
    rows are XOR-rotated, byte grp ^ (tau & 15); key rows of 16 groups hold group P(j) ^ (tau & 15) in byte j,
    P the bit permutation (j3 j2 j1 j0) -> (j1 j3 j2 j0); key rows of 32 groups are in group order."""
    grp = np.asarray(grp)
    tau = np.asarray(tau)
    if kind == "v":
        return grp ^ (tau & 15)
    if NG != 16:
        return grp + 0 * tau
    b = grp ^ (tau & 15)
    return (b & 1) | (((b >> 3) & 1) << 1) | (((b >> 1) & 1) << 2) | (((b >> 2) & 1) << 3)


def host_codebooks(p: LoopVQProblem, h: int, kind: str) -> np.ndarray:
    """[NB][NG][K][G] float64 codebooks of head h."""
    kv = 0 if kind == "k" else 1
    return p.codebooks[:, h, kv].float().cpu().numpy().astype(np.float64)


def run_step(p: LoopVQProblem, t: int, num_splits: int = 0, out=None, lse=None, ws=None, order=None,
             k_scales=None):
    return lvq.lvq_decode_attn(p.g, t, p.q[t].contiguous(), p.cache.pool, p.cache.page_table, p.cache.seq_len,
                               p.cache.max_len, p.cache.win_k, p.cache.win_v, p.slices, p.rope_cos, p.rope_sin,
                               p.sm_scale, out=out, lse_out=lse, ws=ws, num_splits=num_splits, rope_f16=p.rope16,
                               order=order, k_scales=k_scales)


# ---------------------------------------------------------------------------
# KIVI
# ---------------------------------------------------------------------------

@dataclass
class KiviProblem:
    cfg: KiviConfig
    g: object
    cache: "lvq.KiviCache"
    k: torch.Tensor          # [B][H][L][D] fp16 prefill data
    v: torch.Tensor
    q: torch.Tensor          # [B][Hq][D] fp16
    sm_scale: float


def build_kivi(cfg: KiviConfig, device="cuda", cap: int = 0) -> KiviProblem:
    cap = cap or ((cfg.L + 256 + cfg.group - 1) // cfg.group) * cfg.group
    g = lvq.make_kivi_geom(D=cfg.D, H=cfg.H, bits=cfg.bits, group=cfg.group, R=cfg.R, cap=cap, v_bits=cfg.v_bits,
                           Hq=cfg.Hq)
    cache = lvq.KiviCache(g, cfg.B, device=device)
    k, v = synk.raw_kv(cfg, device)
    lvq.kivi_append(g, k, v, cache, prefill=True)
    q = synk.queries(cfg, device)[0].contiguous()
    torch.cuda.synchronize()
    return KiviProblem(cfg, g, cache, k, v, q, synk.softmax_scale(cfg))
