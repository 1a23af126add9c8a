"""Quantized-KV decode attention for AMD MI355X (gfx950).

A thin binding over liblvq.so: each function here has the name of a C entry
point in include/lvq.h, takes torch tensors that already live on the GPU,
checks dtypes and shapes, and passes raw pointers and the current HIP stream
through.  Every step of the computation runs in the library's HIP kernels;
torch only provides device memory and streams.  Importing this package fails
if liblvq.so has not been built.
"""

from __future__ import annotations

import ctypes as C
from typing import Optional, Tuple

import numpy as np
import torch

from ._lib import LVQ_BF16, LVQ_FP32, LvqError, check, kivi_cache, kivi_geom, lib, lvq_geom  # noqa: F401
from . import layout  # noqa: F401

__all__ = [
    "LvqError", "lvq_geom", "kivi_geom", "make_geom", "make_kivi_geom",
    "lvq_slice_codebooks", "lvq_rope_table", "lvq_rope_table_f16", "lvq_channel_perm_check", "lvq_rope_table_perm",
    "lvq_encode", "lvq_decode_attn_workspace", "lvq_decode_attn", "lvq_decode_attn_noalloc", "lvq_request_order", "lvq_check_pages", "lvq_window_append",
    "lvq_codebook_update",
    "lvq_decode_attn_splits", "lvq_quant_partial", "lvq_quant_partial_workspace", "lvq_window_partial", "splitk_lse_merge", "kivi_append",
    "kivi_decode_attn_workspace", "kivi_decode_attn", "KiviCache", "kivi_widths", "layout",
]


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _need(t: torch.Tensor, name: str, dtype=None, contiguous=True):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def make_geom(D=128, T=4, Tc=2, G=16, K=256, page=8, sink=8, window=64, H=1, cb_dtype="bf16") -> lvq_geom:
    cb = {"bf16": LVQ_BF16, "fp32": LVQ_FP32}[cb_dtype]
    return lvq_geom(D, T, Tc, G, K, page, sink, window, H, cb)


def make_kivi_geom(D=128, H=1, bits=2, group=32, R=128, cap=4096, v_bits=0, Hq=0) -> kivi_geom:
    """bits: key code width (2 or 4); v_bits: value code width (0 = as keys); Hq: query heads (0 = H)."""
    return kivi_geom(D, H, bits, group, R, cap, v_bits, Hq)


def kivi_widths(g: kivi_geom):
    """(key bits, value bits, query heads) of a geometry."""
    return g.bits, (g.v_bits or g.bits), (g.Hq or g.H)


def _cb_torch_dtype(g: lvq_geom):
    return torch.bfloat16 if g.cb_dtype == LVQ_BF16 else torch.float32


# ---------------------------------------------------------------------------
# LoopVQ
# ---------------------------------------------------------------------------

def lvq_slice_codebooks(g: lvq_geom, codebooks: torch.Tensor, slices: Optional[torch.Tensor] = None,
                        stream=None) -> torch.Tensor:
    """codebooks [T/Tc][H][2][NG][K][G] -> slices [T][H][2][NG][K][c]."""
    _need(codebooks, "codebooks", _cb_torch_dtype(g))
    c = g.G // g.Tc
    shape = (g.T, g.H, 2, g.D // c, g.K, c)
    if slices is None:
        slices = torch.empty(shape, dtype=codebooks.dtype, device=codebooks.device)
    _need(slices, "slices", codebooks.dtype)
    if tuple(codebooks.shape) != (g.T // g.Tc, g.H, 2, g.D // c, g.K, g.G) or tuple(slices.shape) != shape:
        raise ValueError("codebook / slice shape does not match the geometry")
    check(lib.lvq_slice_codebooks(C.byref(g), codebooks.data_ptr(), slices.data_ptr(), _stream(stream)),
          "lvq_slice_codebooks")
    return slices


def lvq_rope_table(length: int, D: int = 128, base: float = 10000.0, device="cuda",
                   stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """(cos, sin) fp32 [length][D/2], evaluated in fp64 on the device."""
    cos = torch.empty((length, D // 2), dtype=torch.float32, device=device)
    sin = torch.empty_like(cos)
    check(lib.lvq_rope_table(int(length), int(D), float(base), cos.data_ptr(), sin.data_ptr(), _stream(stream)),
          "lvq_rope_table")
    return cos, sin


def lvq_rope_table_f16(length: int, D: int = 128, base: float = 10000.0, device="cuda",
                       stream=None) -> torch.Tensor:
    """Packed fp16 cos/sin for the index-page pass, 384 halves per position (layout in include/lvq.h)."""
    out = torch.empty((length * 384,), dtype=torch.float16, device=device)
    check(lib.lvq_rope_table_f16(int(length), int(D), float(base), out.data_ptr(), _stream(stream)),
          "lvq_rope_table_f16")
    return out


def _perm_array(perm) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(perm, dtype=np.int32))


def lvq_channel_perm_check(g: lvq_geom, perm) -> int:
    """Status of a channel permutation (stored channel j holds original channel perm[j]): LVQ_OK when it maps
    RoPE pairs to RoPE pairs, else LVQ_ERR_UNSUPPORTED / LVQ_ERR_INVALID_ARG (include/lvq.h)."""
    p = _perm_array(perm)
    return int(lib.lvq_channel_perm_check(C.byref(g), p.ctypes.data))


def lvq_rope_table_perm(g: lvq_geom, perm, length: int, base: float = 10000.0, device="cuda", packed=True,
                        stream=None):
    """(cos, sin, packed fp16 or None) for a channel permutation accepted by lvq_channel_perm_check:
    frequency column j holds frequency perm[j]."""
    p = _perm_array(perm)
    cos = torch.empty((length, g.D // 2), dtype=torch.float32, device=device)
    sin = torch.empty_like(cos)
    f16 = torch.empty((length * 384,), dtype=torch.float16, device=device) if packed else None
    check(lib.lvq_rope_table_perm(C.byref(g), p.ctypes.data, int(length), float(base), cos.data_ptr(),
                                  sin.data_ptr(), f16.data_ptr() if packed else None, _stream(stream)),
          "lvq_rope_table_perm")
    return cos, sin, f16


def _rope_f16_ptr(rope_f16: Optional[torch.Tensor], rope_cos: torch.Tensor):
    if rope_f16 is None:
        return None
    _need(rope_f16, "rope_f16", torch.float16)
    if rope_f16.numel() != rope_cos.shape[0] * 384:
        raise ValueError("rope_f16 must hold 384 halves per position of rope_cos (lvq_rope_table_f16)")
    return rope_f16.data_ptr()


def lvq_encode(g: lvq_geom, block: int, x_k: Optional[torch.Tensor], x_v: Optional[torch.Tensor],
               codebooks: torch.Tensor, pool: torch.Tensor, page_table: torch.Tensor, first_page: torch.Tensor,
               n_pages: torch.Tensor, max_pages: int, x_tok0: Optional[torch.Tensor] = None, stream=None):
    """Encode index pages of loop block `block`.

    x_k / x_v: bf16 views of shape [B][H][N][Tc][D] (any strides, unit stride
    on D); token j of request b is row x_tok0[b] + j (see include/lvq.h)."""
    xs = [x for x in (x_k, x_v) if x is not None]
    if not xs:
        raise ValueError("x_k and x_v are both None")
    for name, x in (("x_k", x_k), ("x_v", x_v)):
        if x is not None:
            _need(x, name, torch.bfloat16, contiguous=False)
            if x.dim() != 5 or x.shape[-1] != g.D or x.stride(-1) != 1:
                raise ValueError(f"{name} must be [B][H][N][Tc][D] with unit stride on D")
    if x_k is not None and x_v is not None and x_k.stride() != x_v.stride():
        raise ValueError("x_k and x_v must share strides")
    strides = (C.c_int64 * 4)(*xs[0].stride()[:4])
    _need(codebooks, "codebooks", _cb_torch_dtype(g))
    _need(pool, "pool", torch.uint8)
    _need(page_table, "page_table", torch.int32)
    _need(first_page, "first_page", torch.int32)
    _need(n_pages, "n_pages", torch.int32)
    if x_tok0 is not None:
        _need(x_tok0, "x_tok0", torch.int64)
    B = first_page.numel()
    check(lib.lvq_encode(C.byref(g), int(block), x_k.data_ptr() if x_k is not None else None,
                         x_v.data_ptr() if x_v is not None else None, strides,
                         x_tok0.data_ptr() if x_tok0 is not None else None, codebooks.data_ptr(),
                         pool.data_ptr(), page_table.data_ptr(), int(page_table.shape[-1]),
                         first_page.data_ptr(), n_pages.data_ptr(), int(B), int(max_pages), _stream(stream)),
          "lvq_encode")


def lvq_codebook_update(g: lvq_geom, block: int, x_k: Optional[torch.Tensor], x_v: Optional[torch.Tensor],
                        w_k: Optional[torch.Tensor], w_v: Optional[torch.Tensor], codebooks: torch.Tensor,
                        pool: torch.Tensor, page_table: torch.Tensor, first_page: torch.Tensor,
                        n_pages: torch.Tensor, max_pages: int, x_tok0: Optional[torch.Tensor] = None,
                        stream=None):
    """One weighted k-means step for loop block `block` (after lvq_encode of the same pages).

    x_k / x_v: bf16 [B][H][N][Tc][D] views as for lvq_encode; w_k / w_v: fp32 [B][H][N][NG] views
    (unit stride on the group) holding the weight of each coupled vector; codebooks updated in place."""
    xs = [x for x in (x_k, x_v) if x is not None]
    if not xs:
        raise ValueError("x_k and x_v are both None")
    ws_list = []
    for name, x, wname, w in (("x_k", x_k, "w_k", w_k), ("x_v", x_v, "w_v", w_v)):
        if x is None:
            continue
        _need(x, name, torch.bfloat16, contiguous=False)
        if x.dim() != 5 or x.shape[-1] != g.D or x.stride(-1) != 1:
            raise ValueError(f"{name} must be [B][H][N][Tc][D] with unit stride on D")
        if w is None:
            raise ValueError(f"{wname} is required with {name}")
        _need(w, wname, torch.float32, contiguous=False)
        if w.dim() != 4 or tuple(w.shape[:3]) != tuple(x.shape[:3]) or w.stride(-1) != 1:
            raise ValueError(f"{wname} must be [B][H][N][NG] matching {name}, unit stride on the group")
        ws_list.append(w)
    if x_k is not None and x_v is not None and (x_k.stride() != x_v.stride() or w_k.stride() != w_v.stride()):
        raise ValueError("K and V inputs must share strides")
    xstr = (C.c_int64 * 4)(*xs[0].stride()[:4])
    wstr = (C.c_int64 * 3)(*ws_list[0].stride()[:3])
    _need(codebooks, "codebooks", _cb_torch_dtype(g))
    B = first_page.numel()
    check(lib.lvq_codebook_update(C.byref(g), int(block), x_k.data_ptr() if x_k is not None else None,
                                  x_v.data_ptr() if x_v is not None else None, xstr,
                                  x_tok0.data_ptr() if x_tok0 is not None else None,
                                  w_k.data_ptr() if w_k is not None else None,
                                  w_v.data_ptr() if w_v is not None else None, wstr, codebooks.data_ptr(),
                                  pool.data_ptr(), page_table.data_ptr(), int(page_table.shape[-1]),
                                  first_page.data_ptr(), n_pages.data_ptr(), int(B), int(max_pages),
                                  _stream(stream)),
          "lvq_codebook_update")


def lvq_decode_attn_workspace(g: lvq_geom, B: int, max_len: int, num_splits: int = 0) -> int:
    return int(lib.lvq_decode_attn_workspace(C.byref(g), int(B), int(max_len), int(num_splits)))


def lvq_decode_attn(g: lvq_geom, step: int, q: torch.Tensor, pool: torch.Tensor, page_table: torch.Tensor,
                    seq_len: torch.Tensor, max_len: int, win_k: torch.Tensor, win_v: torch.Tensor,
                    slices: torch.Tensor, rope_cos: torch.Tensor, rope_sin: torch.Tensor, sm_scale: float,
                    out: Optional[torch.Tensor] = None, lse_out: Optional[torch.Tensor] = None,
                    ws: Optional[torch.Tensor] = None, num_splits: int = 0,
                    stream=None, rope_f16: Optional[torch.Tensor] = None, order: Optional[torch.Tensor] = None,
                    k_scales: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Decode attention of loop step `step`; returns (out [B][H][D] fp32, lse [B][H] or None).
    rope_f16 (lvq_rope_table_f16) is optional: without it, bf16 codebooks have the packed table built from
    rope_cos / rope_sin in the workspace on every call; order (int32 [B], e.g. from
    lvq_request_order) groups the requests into workgroups (None: in batch order); k_scales (fp16
    [physical pages][T][8]) is the key scale stream of the index tokens (None: no scales)."""
    _need(q, "q", torch.bfloat16)
    B = q.shape[0]
    if tuple(q.shape) != (B, g.H, g.D):
        raise ValueError("q must be [B][H][D]")
    _need(pool, "pool", torch.uint8)
    _need(page_table, "page_table", torch.int32)
    _need(seq_len, "seq_len", torch.int32)
    for name, w in (("win_k", win_k), ("win_v", win_v)):
        _need(w, name, torch.bfloat16)
        if tuple(w.shape) != (B, g.T, g.H, g.sink + g.window + g.page, g.D):
            raise ValueError(f"{name} must be [B][T][H][sink+window+page][D]")
    _need(slices, "slices", _cb_torch_dtype(g))
    _need(rope_cos, "rope_cos", torch.float32)
    _need(rope_sin, "rope_sin", torch.float32)
    if seq_len.numel() != B or page_table.dim() != 2 or page_table.shape[0] != B:
        raise ValueError("seq_len / page_table batch does not match q")
    _need_order(order, B)
    _need_kscales(k_scales, g, pool)
    if out is None:
        out = torch.empty((B, g.H, g.D), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32)
    if lse_out is not None:
        _need(lse_out, "lse_out", torch.float32)
    need = lvq_decode_attn_workspace(g, B, max_len, num_splits)
    if ws is None:
        ws = torch.empty(max(need, 4), dtype=torch.uint8, device=q.device)
    _need(ws, "ws")
    check(lib.lvq_decode_attn(C.byref(g), int(step), q.data_ptr(), pool.data_ptr(), page_table.data_ptr(),
                              int(page_table.shape[1]), seq_len.data_ptr(), int(max_len),
                              order.data_ptr() if order is not None else None,
                              k_scales.data_ptr() if k_scales is not None else None, win_k.data_ptr(),
                              win_v.data_ptr(), slices.data_ptr(), rope_cos.data_ptr(), rope_sin.data_ptr(),
                              _rope_f16_ptr(rope_f16, rope_cos), int(rope_cos.shape[0]), float(sm_scale),
                              out.data_ptr(),
                              lse_out.data_ptr() if lse_out is not None else None, ws.data_ptr(),
                              ws.numel() * ws.element_size(), int(num_splits), int(B), _stream(stream)),
          "lvq_decode_attn")
    return out, lse_out


def lvq_decode_attn_noalloc(g: lvq_geom, step: int, q: torch.Tensor, pool: torch.Tensor, page_table: torch.Tensor,
                            seq_len: torch.Tensor, max_len: int, win_k: torch.Tensor, win_v: torch.Tensor,
                            slices: torch.Tensor, rope_cos: torch.Tensor, rope_sin: torch.Tensor, sm_scale: float,
                            out: torch.Tensor, lse_out: Optional[torch.Tensor] = None, num_splits: int = 0,
                            stream=None, rope_f16: Optional[torch.Tensor] = None,
                            order: Optional[torch.Tensor] = None,
                            k_scales: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """lvq_decode_attn with the library's own per-GPU workspace: the caller passes `out` (and `lse_out`) and
    nothing is allocated, here or in the library."""
    _need(q, "q", torch.bfloat16)
    B = q.shape[0]
    if tuple(q.shape) != (B, g.H, g.D):
        raise ValueError("q must be [B][H][D]")
    _need(pool, "pool", torch.uint8)
    _need(page_table, "page_table", torch.int32)
    _need(seq_len, "seq_len", torch.int32)
    for name, w in (("win_k", win_k), ("win_v", win_v)):
        _need(w, name, torch.bfloat16)
        if tuple(w.shape) != (B, g.T, g.H, g.sink + g.window + g.page, g.D):
            raise ValueError(f"{name} must be [B][T][H][sink+window+page][D]")
    _need(slices, "slices", _cb_torch_dtype(g))
    _need(rope_cos, "rope_cos", torch.float32)
    _need(rope_sin, "rope_sin", torch.float32)
    if seq_len.numel() != B or page_table.dim() != 2 or page_table.shape[0] != B:
        raise ValueError("seq_len / page_table batch does not match q")
    _need_order(order, B)
    _need_kscales(k_scales, g, pool)
    _need(out, "out", torch.float32)
    if tuple(out.shape) != (B, g.H, g.D):
        raise ValueError("out must be [B][H][D]")
    if lse_out is not None:
        _need(lse_out, "lse_out", torch.float32)
    check(lib.lvq_decode_attn_noalloc(C.byref(g), int(step), q.data_ptr(), pool.data_ptr(), page_table.data_ptr(),
                                      int(page_table.shape[1]), seq_len.data_ptr(), int(max_len),
                                      order.data_ptr() if order is not None else None,
                                      k_scales.data_ptr() if k_scales is not None else None, win_k.data_ptr(),
                                      win_v.data_ptr(), slices.data_ptr(), rope_cos.data_ptr(), rope_sin.data_ptr(),
                                      _rope_f16_ptr(rope_f16, rope_cos), int(rope_cos.shape[0]), float(sm_scale),
                                      out.data_ptr(), lse_out.data_ptr() if lse_out is not None else None,
                                      int(num_splits), int(B), _stream(stream)),
          "lvq_decode_attn_noalloc")
    return out, lse_out


def _need_kscales(k_scales: Optional[torch.Tensor], g: lvq_geom, pool: torch.Tensor):
    if k_scales is not None:
        _need(k_scales, "k_scales", torch.float16)
        if tuple(k_scales.shape) != (pool.shape[0], g.T, 8):
            raise ValueError("k_scales must be [physical pages][T][8], one page per pool page")


def _need_order(order: Optional[torch.Tensor], B: int):
    if order is not None:
        _need(order, "order", torch.int32)
        if order.numel() != B:
            raise ValueError("order must hold one entry per request")


def lvq_request_order(seq_len: torch.Tensor, max_len: int, out: Optional[torch.Tensor] = None,
                      stream=None) -> torch.Tensor:
    """The batch ranked by length, longest first (ties by index): int32 [B] for the `order` argument."""
    _need(seq_len, "seq_len", torch.int32)
    B = seq_len.numel()
    if out is None:
        out = torch.empty(B, dtype=torch.int32, device=seq_len.device)
    _need_order(out, B)
    check(lib.lvq_request_order(seq_len.data_ptr(), int(B), int(max_len), out.data_ptr(), _stream(stream)),
          "lvq_request_order")
    return out


def lvq_check_pages(g: lvq_geom, page_table: torch.Tensor, seq_len: torch.Tensor, max_len: int,
                    n_pool_pages: int, stream=None) -> Tuple[int, int, int]:
    """Debug check of a batch's page table and lengths (include/lvq.h): (offending page-table entries, the
    lowest request holding one or -1, requests whose seq_len lies outside [0, max_len]).  Waits for the
    result."""
    _need(page_table, "page_table", torch.int32)
    _need(seq_len, "seq_len", torch.int32)
    B = seq_len.numel()
    if page_table.dim() != 2 or page_table.shape[0] != B:
        raise ValueError("page_table must be [B][pt_stride] with the seq_len batch")
    bad = torch.zeros(3, dtype=torch.int32, device=seq_len.device)
    check(lib.lvq_check_pages(C.byref(g), page_table.data_ptr(), int(page_table.shape[1]), seq_len.data_ptr(),
                              int(max_len), int(n_pool_pages), int(B), bad.data_ptr(), _stream(stream)),
          "lvq_check_pages")
    n_bad, first, n_len = bad.tolist()
    return n_bad, first, n_len


def lvq_window_append(g: lvq_geom, step: int, k_new: Optional[torch.Tensor], v_new: Optional[torch.Tensor],
                      cache, max_len: int, stream=None):
    """One generated token (bf16 [B][H][D] pre-RoPE K and/or V of loop step `step`) into the window
    of `cache` (a layout.LoopVQCache) at position seq_len[b] - 1."""
    B = cache.B
    for name, x in (("k_new", k_new), ("v_new", v_new)):
        if x is not None:
            _need(x, name, torch.bfloat16)
            if tuple(x.shape) != (B, g.H, g.D):
                raise ValueError(f"{name} must be [B][H][D]")
    check(lib.lvq_window_append(C.byref(g), int(step), k_new.data_ptr() if k_new is not None else None,
                                v_new.data_ptr() if v_new is not None else None, cache.win_k.data_ptr(),
                                cache.win_v.data_ptr(), cache.seq_len.data_ptr(), int(max_len), int(B),
                                _stream(stream)), "lvq_window_append")


def lvq_decode_attn_splits(g: lvq_geom, B: int, max_len: int) -> int:
    """The split count lvq_decode_attn runs when num_splits = 0."""
    return int(lib.lvq_decode_attn_splits(C.byref(g), int(B), int(max_len)))


def lvq_quant_partial_workspace(g: lvq_geom, B: int, max_len: int) -> int:
    return int(lib.lvq_quant_partial_workspace(C.byref(g), int(B), int(max_len)))


def lvq_quant_partial(g: lvq_geom, step: int, q: torch.Tensor, pool: torch.Tensor, page_table: torch.Tensor,
                      seq_len: torch.Tensor, max_len: int, slices: torch.Tensor, rope_cos: torch.Tensor,
                      rope_sin: torch.Tensor, sm_scale: float, part_o: torch.Tensor, part_lse: torch.Tensor,
                      num_splits: int, ws: Optional[torch.Tensor] = None, stream=None,
                      rope_f16: Optional[torch.Tensor] = None, order: Optional[torch.Tensor] = None,
                      k_scales: Optional[torch.Tensor] = None):
    """Index-page partials into part_o [B*H][S_tot][D], part_lse [B*H][S_tot] (slots 0..num_splits-1)."""
    _need(q, "q", torch.bfloat16)
    _need(pool, "pool", torch.uint8)
    _need(page_table, "page_table", torch.int32)
    _need(seq_len, "seq_len", torch.int32)
    _need(slices, "slices", _cb_torch_dtype(g))
    _need(part_o, "part_o", torch.float32)
    _need(part_lse, "part_lse", torch.float32)
    B = q.shape[0]
    _need_order(order, B)
    _need_kscales(k_scales, g, pool)
    need = lvq_quant_partial_workspace(g, B, max_len)
    if ws is None:
        ws = torch.empty(max(need, 4), dtype=torch.uint8, device=q.device)
    _need(ws, "ws")
    check(lib.lvq_quant_partial(C.byref(g), int(step), q.data_ptr(), pool.data_ptr(), page_table.data_ptr(),
                                int(page_table.shape[1]), seq_len.data_ptr(), int(max_len),
                                order.data_ptr() if order is not None else None,
                                k_scales.data_ptr() if k_scales is not None else None, slices.data_ptr(),
                                rope_cos.data_ptr(), rope_sin.data_ptr(), _rope_f16_ptr(rope_f16, rope_cos),
                                int(rope_cos.shape[0]), float(sm_scale), part_o.data_ptr(), part_lse.data_ptr(),
                                int(num_splits), int(part_lse.shape[1]),
                                ws.data_ptr(), ws.numel() * ws.element_size(), int(B), _stream(stream)),
          "lvq_quant_partial")


def lvq_window_partial(g: lvq_geom, step: int, q: torch.Tensor, seq_len: torch.Tensor, max_len: int,
                       win_k: torch.Tensor, win_v: torch.Tensor, rope_cos: torch.Tensor, rope_sin: torch.Tensor,
                       sm_scale: float, part_o: torch.Tensor, part_lse: torch.Tensor, slot: int, stream=None):
    """bf16-window partial into slot `slot` of part_o / part_lse."""
    _need(q, "q", torch.bfloat16)
    _need(seq_len, "seq_len", torch.int32)
    _need(win_k, "win_k", torch.bfloat16)
    _need(win_v, "win_v", torch.bfloat16)
    _need(part_o, "part_o", torch.float32)
    _need(part_lse, "part_lse", torch.float32)
    B = q.shape[0]
    check(lib.lvq_window_partial(C.byref(g), int(step), q.data_ptr(), seq_len.data_ptr(), int(max_len),
                                 win_k.data_ptr(), win_v.data_ptr(), rope_cos.data_ptr(), rope_sin.data_ptr(),
                                 int(rope_cos.shape[0]), float(sm_scale), part_o.data_ptr(), part_lse.data_ptr(),
                                 int(slot), int(part_lse.shape[1]), int(B), _stream(stream)), "lvq_window_partial")


def splitk_lse_merge(part_o: torch.Tensor, part_lse: torch.Tensor, out: Optional[torch.Tensor] = None,
                     lse_out: Optional[torch.Tensor] = None, stream=None):
    """part_o fp32 [n][S][D], part_lse fp32 [n][S] -> (out [n][D], lse [n])."""
    _need(part_o, "part_o", torch.float32)
    _need(part_lse, "part_lse", torch.float32)
    n, S, D = part_o.shape
    if tuple(part_lse.shape) != (n, S):
        raise ValueError("part_lse must be [n][S]")
    if out is None:
        out = torch.empty((n, D), dtype=torch.float32, device=part_o.device)
    if lse_out is None:
        lse_out = torch.empty((n,), dtype=torch.float32, device=part_o.device)
    _need(out, "out", torch.float32)
    _need(lse_out, "lse_out", torch.float32)
    check(lib.splitk_lse_merge(part_o.data_ptr(), part_lse.data_ptr(), int(n), int(S), int(D), out.data_ptr(),
                               lse_out.data_ptr(), _stream(stream)), "splitk_lse_merge")
    return out, lse_out


# ---------------------------------------------------------------------------
# KIVI
# ---------------------------------------------------------------------------

class KiviCache:
    """Device buffers of a KIVI cache for B requests (layout in include/lvq.h)."""

    def __init__(self, g: kivi_geom, B: int, device="cuda"):
        self.g, self.B = g, B
        D, H, G, cap, ring = g.D, g.H, g.group, g.cap, g.R + g.group
        kb, vb, _ = kivi_widths(g)
        u8, f16 = torch.uint8, torch.float16
        self.k_codes = torch.zeros((B, H, cap, D * kb // 8), dtype=u8, device=device)
        self.k_scale = torch.zeros((B, H, cap // G, D), dtype=f16, device=device)
        self.k_zero = torch.zeros((B, H, cap // G, D), dtype=f16, device=device)
        self.v_codes = torch.zeros((B, H, cap, D * vb // 8), dtype=u8, device=device)
        self.v_scale = torch.zeros((B, H, cap, D // G), dtype=f16, device=device)
        self.v_zero = torch.zeros((B, H, cap, D // G), dtype=f16, device=device)
        self.k_res = torch.zeros((B, H, ring, D), dtype=f16, device=device)
        self.v_res = torch.zeros((B, H, ring, D), dtype=f16, device=device)
        self.len = torch.zeros((B,), dtype=torch.int32, device=device)
        self.n_kq = torch.zeros((B,), dtype=torch.int32, device=device)
        self.n_vq = torch.zeros((B,), dtype=torch.int32, device=device)
        self.c = kivi_cache(*[t.data_ptr() for t in (self.k_codes, self.k_scale, self.k_zero, self.v_codes,
                                                      self.v_scale, self.v_zero, self.k_res, self.v_res,
                                                      self.len, self.n_kq, self.n_vq)])


def kivi_append(g: kivi_geom, k_new: torch.Tensor, v_new: torch.Tensor, cache: KiviCache, prefill: bool,
                stream=None):
    """k_new, v_new fp16 [B][H][n][D] (unit stride on D)."""
    for name, x in (("k_new", k_new), ("v_new", v_new)):
        _need(x, name, torch.float16, contiguous=False)
        if x.dim() != 4 or x.shape[0] != cache.B or x.shape[1] != g.H or x.shape[3] != g.D or x.stride(3) != 1:
            raise ValueError(f"{name} must be [B][H][n][D] with unit stride on D")
    if k_new.stride() != v_new.stride() or k_new.shape != v_new.shape:
        raise ValueError("k_new and v_new must share shape and strides")
    strides = (C.c_int64 * 3)(*k_new.stride()[:3])
    check(lib.kivi_append(C.byref(g), k_new.data_ptr(), v_new.data_ptr(), strides, int(k_new.shape[2]),
                          int(bool(prefill)), C.byref(cache.c), int(cache.B), _stream(stream)), "kivi_append")


def kivi_decode_attn_workspace(g: kivi_geom, B: int, max_len: int, num_splits: int = 0) -> int:
    return int(lib.kivi_decode_attn_workspace(C.byref(g), int(B), int(max_len), int(num_splits)))


def kivi_decode_attn(g: kivi_geom, q: torch.Tensor, cache: KiviCache, max_len: int, sm_scale: float,
                     out: Optional[torch.Tensor] = None, lse_out: Optional[torch.Tensor] = None,
                     ws: Optional[torch.Tensor] = None, num_splits: int = 0, stream=None):
    _need(q, "q", torch.float16)
    B = cache.B
    Hq = kivi_widths(g)[2]
    if tuple(q.shape) != (B, Hq, g.D):
        raise ValueError("q must be [B][Hq][D]")
    if out is None:
        out = torch.empty((B, Hq, g.D), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32)
    if lse_out is not None:
        _need(lse_out, "lse_out", torch.float32)
    need = kivi_decode_attn_workspace(g, B, max_len, num_splits)
    if ws is None:
        ws = torch.empty(max(need, 4), dtype=torch.uint8, device=q.device)
    _need(ws, "ws")
    check(lib.kivi_decode_attn(C.byref(g), q.data_ptr(), C.byref(cache.c), int(max_len), float(sm_scale),
                               out.data_ptr(), lse_out.data_ptr() if lse_out is not None else None, ws.data_ptr(),
                               ws.numel() * ws.element_size(), int(num_splits), int(B), _stream(stream)),
          "kivi_decode_attn")
    return out, lse_out
