"""The C ABI on the host: the library loads, exports every symbol the header
declares, and rejects bad arguments with the documented status before any
device work.  No kernel is launched here (CPU only)."""

import ctypes as C
import os
import re

import pytest

import decode_attention_loopvq_amd as lvq
from decode_attention_loopvq_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "lvq.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FAKE = C.c_void_p(4096)      # never dereferenced: validation fails before any use


def _declared():
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"LVQ_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("lvq_encode", "lvq_decode_attn", "kivi_append", "kivi_decode_attn", "splitk_lse_merge"):
        assert n in names


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert names == sorted(_lib.EXPORTS)
    for n in names:
        assert hasattr(_lib.lib, n), n


def _geom(**kw):
    return lvq.make_geom(H=2, **kw)


def _attn(g, **over):
    args = dict(step=0, q=FAKE, pool=FAKE, pt=FAKE, pt_stride=1000, seq_len=FAKE, max_len=1024, wk=FAKE,
                wv=FAKE, slices=FAKE, cos=FAKE, sin=FAKE, rope16=FAKE, rope_len=2048, scale=0.1, out=FAKE,
                lse=None, ws=FAKE,
                ws_bytes=1 << 30, splits=0, B=4)
    args.update(over)
    gp = C.byref(g) if g is not None else None
    return _lib.lib.lvq_decode_attn(gp, args["step"], args["q"], args["pool"], args["pt"], args["pt_stride"],
                                    args["seq_len"], args["max_len"], None, args.get("kscale"), args["wk"], args["wv"],
                                    args["slices"],
                                    args["cos"], args["sin"], args["rope16"], args["rope_len"], args["scale"],
                                    args["out"],
                                    args["lse"], args["ws"], args["ws_bytes"], args["splits"], args["B"], None)


@pytest.mark.parametrize("over,status", [
    (dict(step=4), INVALID), (dict(step=-1), INVALID), (dict(max_len=0), INVALID),
    (dict(max_len=4096), INVALID),             # beyond the RoPE table
    (dict(splits=2000), INVALID), (dict(splits=-2), INVALID), (dict(q=None), INVALID), (dict(ws=None), INVALID),
    (dict(pool=None), INVALID), (dict(pt_stride=3), INVALID), (dict(scale=float("nan")), INVALID),
    (dict(ws_bytes=16), WORKSPACE),
    (dict(max_len=2048, splits=1), INVALID),   # 247 index pages in one split: over 1536 tokens per split
    (dict(ws=C.c_void_p(4096 + 16)), INVALID),  # workspace not 256-byte aligned
    (dict(splits=-1), INVALID),                # no single-pass kernel
])
def test_decode_attn_rejects(over, status):
    assert _attn(_geom(), **over) == status
    assert _lib.lib.lvq_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(D=64), UNSUPPORTED), (dict(K=128), UNSUPPORTED), (dict(page=16), UNSUPPORTED),
    (dict(T=4, Tc=3), INVALID), (dict(G=12, Tc=2), UNSUPPORTED), (dict(G=64, Tc=2), UNSUPPORTED),
    (dict(window=60), UNSUPPORTED), (dict(T=0), INVALID),
    (dict(T=8, Tc=8, G=64), UNSUPPORTED),    # c = 8, but codewords longer than 32 coordinates
])
def test_geometry_rejects(kw, status):
    assert _attn(_geom(**kw)) == status
    assert _attn(None) == INVALID


def test_decode_attn_without_packed_table_needs_room_for_one():
    """Called without the packed fp16 RoPE table, lvq_decode_attn builds one in the workspace (768 B per
    position below max_len), so the workspace query counts it and a workspace short of it is refused."""
    g = _geom()
    need = _lib.lib.lvq_decode_attn_workspace(C.byref(g), 4, 1024, 0)
    assert _attn(g, rope16=None, ws_bytes=need - 256) == WORKSPACE
    assert "workspace" in _lib.lib.lvq_last_error().decode()


def test_decode_attn_empty_batch_is_a_no_op():
    assert _attn(_geom(), B=0, q=None, ws=None) == OK


def test_workspace_query():
    g = _geom()
    n = _lib.lib.lvq_decode_attn_workspace(C.byref(g), 64, 6144, 3)
    # partials of 3 + 1 slots (rounded up to 256 B) + the packed fp16 query rows, 256 B per (request, head)
    # + room for a packed fp16 RoPE table of the positions below max_len, 768 B each (used by calls given none)
    scratch = 64 * 2 * 64 * 4
    table = 6144 * 768
    assert n == 64 * 2 * 4 * (128 + 1) * 4 + scratch + table
    assert (_lib.lib.lvq_decode_attn_workspace(C.byref(g), 3, 6144, 1) ==
            (3 * 2 * 2 * 129 * 4 + 255) // 256 * 256 + 3 * 2 * 256 + table)
    assert _lib.lib.lvq_quant_partial_workspace(C.byref(g), 64, 6144) == scratch + table
    assert _lib.lib.lvq_quant_partial_workspace(C.byref(g), 64, 1001) == scratch + (1001 * 768 + 255) // 256 * 256
    g32 = _geom(cb_dtype="fp32")
    assert _attn(g32, rope16=None, B=0) == OK
    assert _lib.lib.lvq_decode_attn_workspace(C.byref(g), 64, 6144, 0) > 0
    assert _lib.lib.lvq_decode_attn_workspace(None, 64, 6144, 0) == 0
    assert _lib.lib.lvq_decode_attn_workspace(C.byref(g), 64, 6144, -1) == 0


def test_encode_rejects():
    g = _geom()
    strides = (C.c_int64 * 4)(1, 1, 1, 1)
    f = _lib.lib.lvq_encode
    assert f(C.byref(g), 2, FAKE, FAKE, strides, None, FAKE, FAKE, FAKE, 8, FAKE, FAKE, 4, 8, None) == INVALID
    assert f(C.byref(g), 0, None, None, strides, None, FAKE, FAKE, FAKE, 8, FAKE, FAKE, 4, 8, None) == INVALID
    assert f(C.byref(g), 0, FAKE, None, strides, None, FAKE, None, FAKE, 8, FAKE, FAKE, 4, 8, None) == INVALID
    assert f(C.byref(g), 0, FAKE, None, strides, None, FAKE, FAKE, FAKE, 8, FAKE, FAKE, 0, 8, None) == OK
    g64 = _geom(T=8, Tc=8, G=64)
    assert f(C.byref(g64), 0, FAKE, None, strides, None, FAKE, FAKE, FAKE, 8, FAKE, FAKE, 4, 8, None) == UNSUPPORTED


def test_merge_and_tables_reject():
    assert _lib.lib.splitk_lse_merge(FAKE, FAKE, 4, 0, 128, FAKE, None, None) == INVALID
    assert _lib.lib.splitk_lse_merge(None, FAKE, 4, 2, 128, FAKE, None, None) == INVALID
    assert _lib.lib.splitk_lse_merge(None, None, 0, 2, 128, None, None, None) == OK
    assert _lib.lib.lvq_rope_table(0, 128, 10000.0, FAKE, FAKE, None) == INVALID
    assert _lib.lib.lvq_rope_table(16, 127, 10000.0, FAKE, FAKE, None) == INVALID
    assert _lib.lib.lvq_rope_table_f16(0, 128, 10000.0, FAKE, None) == INVALID
    assert _lib.lib.lvq_rope_table_f16(16, 64, 10000.0, FAKE, None) == UNSUPPORTED
    assert _lib.lib.lvq_rope_table_f16(16, 128, 1.0, FAKE, None) == INVALID
    assert _lib.lib.lvq_rope_table_f16(16, 128, 10000.0, None, None) == INVALID
    g = _geom(D=64)
    assert _lib.lib.lvq_slice_codebooks(C.byref(g), FAKE, FAKE, None) == UNSUPPORTED


def _kc():
    return _lib.kivi_cache(*([4096] * 11))


def test_kivi_rejects():
    g = lvq.make_kivi_geom(H=2, cap=4096)
    c = _kc()
    strides = (C.c_int64 * 3)(1, 1, 1)
    f = _lib.lib.kivi_append
    assert f(C.byref(g), FAKE, FAKE, strides, 2, 0, C.byref(c), 4, None) == UNSUPPORTED   # decode of 2 tokens
    assert f(C.byref(g), FAKE, FAKE, strides, 0, 1, C.byref(c), 4, None) == INVALID
    assert f(C.byref(g), FAKE, FAKE, strides, 5000, 1, C.byref(c), 4, None) == INVALID   # over capacity
    for kw in (dict(bits=3), dict(bits=8), dict(v_bits=3), dict(v_bits=1), dict(Hq=3), dict(Hq=2 * 64),
               dict(Hq=2 * 3), dict(Hq=-2)):
        bad = lvq.make_kivi_geom(H=2, **kw)
        assert f(C.byref(bad), FAKE, FAKE, strides, 1, 0, C.byref(c), 4, None) == UNSUPPORTED, kw
    # 2 splits + the residual slot, per (request, query head)
    assert _lib.lib.kivi_decode_attn_workspace(C.byref(lvq.make_kivi_geom(H=2)), 4, 4096, 2) == \
        4 * 2 * (2 + 1) * (128 + 1) * 4
    assert _lib.lib.kivi_decode_attn_workspace(C.byref(lvq.make_kivi_geom(H=2, Hq=8)), 4, 4096, 2) == \
        4 * 8 * (2 + 1) * (128 + 1) * 4
    bad = lvq.make_kivi_geom(H=2, R=100)
    assert f(C.byref(bad), FAKE, FAKE, strides, 1, 0, C.byref(c), 4, None) == INVALID
    c.len = None
    assert f(C.byref(g), FAKE, FAKE, strides, 1, 0, C.byref(c), 4, None) == INVALID
    c = _kc()
    a = _lib.lib.kivi_decode_attn
    assert a(C.byref(g), FAKE, C.byref(c), 4097, 0.1, FAKE, None, FAKE, 1 << 30, 0, 4, None) == INVALID
    assert a(C.byref(g), FAKE, C.byref(c), 4096, 0.1, FAKE, None, FAKE, 8, 0, 4, None) == WORKSPACE
    assert a(C.byref(g), None, C.byref(c), 4096, 0.1, FAKE, None, FAKE, 1 << 30, 0, 4, None) == INVALID


def test_python_binding_refuses_host_tensors():
    import torch
    g = _geom()
    with pytest.raises(ValueError):
        lvq.lvq_slice_codebooks(g, torch.zeros((2, 2, 2, 16, 256, 16), dtype=torch.bfloat16))


def test_request_order_rejects():
    """Argument checks of lvq_request_order (all fail before any launch); B = 0 is a no-op."""
    f = _lib.lib.lvq_request_order
    assert f(FAKE, -1, 100, FAKE, None) == INVALID
    assert f(FAKE, 4, 0, FAKE, None) == INVALID
    assert f(None, 4, 100, FAKE, None) == INVALID
    assert f(FAKE, 4, 100, None, None) == INVALID
    assert f(None, 0, 100, None, None) == OK


def test_window_append_rejects():
    """Argument checks of lvq_window_append (all fail before any launch); B = 0 is a no-op."""
    g = _geom(T=4, Tc=2)
    f = _lib.lib.lvq_window_append
    gp = C.byref(g)
    assert f(gp, 4, FAKE, FAKE, FAKE, FAKE, FAKE, 100, 2, None) == INVALID      # step out of range
    assert f(gp, 0, None, None, FAKE, FAKE, FAKE, 100, 2, None) == INVALID      # nothing to append
    assert f(gp, 0, FAKE, FAKE, None, FAKE, FAKE, 100, 2, None) == INVALID      # no window
    assert f(gp, 0, FAKE, FAKE, FAKE, FAKE, None, 100, 2, None) == INVALID      # no lengths
    assert f(gp, 0, C.c_void_p(4098), None, FAKE, None, FAKE, 100, 2, None) == INVALID   # misaligned
    assert f(gp, 0, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 2, None) == INVALID        # max_len < 1
    assert f(gp, 0, None, None, None, None, None, 100, 0, None) == OK


def test_codebook_update_rejects():
    """Argument checks of lvq_codebook_update (all fail before any launch)."""
    g = _geom(T=4, Tc=2)
    gp = C.byref(g)
    f = _lib.lib.lvq_codebook_update
    xs = (C.c_int64 * 4)(1, 1, 1, 1)
    wst = (C.c_int64 * 3)(1, 1, 1)

    def call(**o):
        a = dict(block=0, xk=FAKE, xv=FAKE, xs=xs, tok0=None, wk=FAKE, wv=FAKE, wst=wst, cb=FAKE, pool=FAKE,
                 pt=FAKE, pts=10, first=FAKE, n=FAKE, B=2, maxp=3)
        a.update(o)
        return f(gp, a["block"], a["xk"], a["xv"], a["xs"], a["tok0"], a["wk"], a["wv"], a["wst"], a["cb"],
                 a["pool"], a["pt"], a["pts"], a["first"], a["n"], a["B"], a["maxp"], None)

    assert call(block=2) == INVALID
    assert call(xk=None, xv=None) == INVALID
    assert call(wk=None) == INVALID
    assert call(cb=None) == INVALID
    assert call(B=-1) == INVALID
    assert call(maxp=-1) == INVALID
    assert call(B=0) == OK
    assert call(maxp=0) == OK


def test_context_beyond_the_split_limit_is_unsupported():
    """bf16 codebooks take at most 1024 splits of 192 index pages: a longer context is refused as unsupported,
    naming the context, whatever the split count asked for."""
    g = _geom()
    max_len = 8 + 64 + 8 * 1024 * 192 + 8
    for splits in (0, 1024):
        assert _attn(g, max_len=max_len, rope_len=max_len, pt_stride=1 << 20, splits=splits) == UNSUPPORTED
        assert "index pages" in _lib.lib.lvq_last_error().decode()


def test_noalloc_rejects_before_touching_the_device():
    """lvq_decode_attn_noalloc refuses a call whose workspace would exceed the scratch it holds per GPU, and
    passes argument errors through from lvq_decode_attn, all before any device call."""
    g = _geom()
    f = _lib.lib.lvq_decode_attn_noalloc
    def call(**over):
        a = dict(step=0, max_len=1024, splits=0, B=4, rope_len=2048, scale=0.1, rope16=FAKE)
        a.update(over)
        return f(C.byref(g), a["step"], FAKE, FAKE, FAKE, 1 << 20, FAKE, a["max_len"], None, None, FAKE, FAKE, FAKE,
                 FAKE, FAKE, a["rope16"], a["rope_len"], a["scale"], FAKE, None, a["splits"], a["B"], None)
    need = _lib.lib.lvq_decode_attn_workspace(C.byref(g), 60000, 1024, 0)
    assert need > 16 << 20
    assert call(B=60000) == WORKSPACE
    assert "16777216" in _lib.lib.lvq_last_error().decode()
    assert call(step=9) == INVALID
    assert call(B=0) == OK


def test_check_pages_rejects():
    """lvq_check_pages validates its sizes and pointers before launching anything."""
    g = _geom()
    f = _lib.lib.lvq_check_pages
    # 6K context: 759 index pages per request
    assert f(C.byref(g), FAKE, 758, FAKE, 6144, 100, 4, FAKE, None) == INVALID      # pt_stride below the pages
    assert f(C.byref(g), FAKE, 759, FAKE, 6144, 0, 4, FAKE, None) == INVALID        # no pool pages
    assert f(C.byref(g), None, 759, FAKE, 6144, 100, 4, FAKE, None) == INVALID      # NULL page table
    assert f(C.byref(g), FAKE, 759, FAKE, 6144, 100, 4, None, None) == INVALID      # NULL result
    assert f(C.byref(g), FAKE, 759, FAKE, 0, 100, 4, FAKE, None) == INVALID         # max_len < 1
    assert "lvq_check_pages" in _lib.lib.lvq_last_error().decode()
    assert f(None, FAKE, 759, FAKE, 6144, 100, 4, FAKE, None) == INVALID


def test_channel_perm_check():
    """lvq_channel_perm_check (host only): a permutation that maps RoPE pairs to RoPE pairs passes; swapping a
    pair's halves, putting both channels of a pair in one index group, or any other break of the pairing is
    unsupported; a non-permutation or NULL is an argument error.  lvq_rope_table_perm refuses the unsupported
    forms before touching the device."""
    import numpy as np
    g = _geom()
    f = _lib.lib.lvq_channel_perm_check

    def status(perm):
        p = np.ascontiguousarray(np.asarray(perm, dtype=np.int32))
        return f(C.byref(g), p.ctypes.data)

    rng = np.random.default_rng(4)
    pi = rng.permutation(64)
    assert status(np.arange(128)) == 0
    assert status(np.concatenate([pi, pi + 64])) == 0
    assert status(np.concatenate([np.arange(64, 128), np.arange(64)])) == UNSUPPORTED     # halves swapped
    # the pair-in-group form: stored channels 2u, 2u + 1 hold RoPE pair (u, u + 64)
    in_group = np.empty(128, dtype=np.int32)
    in_group[0::2], in_group[1::2] = np.arange(64), np.arange(64, 128)
    assert status(in_group) == UNSUPPORTED
    assert b"one index group" in _lib.lib.lvq_last_error()
    broken = np.concatenate([pi, pi + 64])
    broken[[64, 65]] = broken[[65, 64]]                                                      # hi halves crossed
    assert status(broken) == UNSUPPORTED
    dup = np.arange(128)
    dup[5] = 6
    assert status(dup) == INVALID
    assert f(C.byref(g), None) == INVALID
    p = np.ascontiguousarray(in_group)
    assert _lib.lib.lvq_rope_table_perm(C.byref(g), p.ctypes.data, 100, 10000.0, FAKE, FAKE, FAKE, None) == UNSUPPORTED
