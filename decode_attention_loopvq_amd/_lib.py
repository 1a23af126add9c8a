"""ctypes view of liblvq.so (the C ABI in include/lvq.h).

Loading fails loudly: there is no fallback path of any kind.
"""

from __future__ import annotations

import ctypes as C
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblvq.so")

EXPORTS = (
    "lvq_last_error", "lvq_slice_codebooks", "lvq_rope_table", "lvq_rope_table_f16", "lvq_channel_perm_check",
    "lvq_rope_table_perm", "lvq_encode",
    "lvq_decode_attn_workspace", "lvq_decode_attn_splits", "lvq_decode_attn", "lvq_decode_attn_noalloc",
    "lvq_request_order", "lvq_check_pages",
    "lvq_window_append", "lvq_codebook_update",
    "lvq_quant_partial",
    "lvq_quant_partial_workspace",
    "lvq_window_partial", "splitk_lse_merge",
    "kivi_append", "kivi_decode_attn_workspace", "kivi_decode_attn",
)

STATUS = {0: "LVQ_OK", 1: "LVQ_ERR_INVALID_ARG", 2: "LVQ_ERR_UNSUPPORTED", 3: "LVQ_ERR_WORKSPACE", 4: "LVQ_ERR_HIP"}
LVQ_BF16, LVQ_FP32 = 0, 1


class LvqError(RuntimeError):
    def __init__(self, status: int, fn: str, msg: str):
        super().__init__(f"{fn} -> {STATUS.get(status, status)}: {msg}")
        self.status = status


class lvq_geom(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("D", "T", "Tc", "G", "K", "page", "sink", "window", "H", "cb_dtype")]


class kivi_geom(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("D", "H", "bits", "group", "R", "cap", "v_bits", "Hq")]


class kivi_cache(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero",
                                          "k_res", "v_res", "len", "n_kq", "n_vq")]


_P = C.c_void_p
_I = C.c_int32
_S = C.c_size_t


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"liblvq.so is not built ({LIB_PATH}); run `python -m decode_attention_loopvq_amd.build`")
    lib = C.CDLL(LIB_PATH)
    lib.lvq_last_error.restype = C.c_char_p
    lib.lvq_last_error.argtypes = []
    lib.lvq_slice_codebooks.argtypes = [C.POINTER(lvq_geom), _P, _P, _P]
    lib.lvq_rope_table.argtypes = [_I, _I, C.c_double, _P, _P, _P]
    lib.lvq_rope_table_f16.argtypes = [_I, _I, C.c_double, _P, _P]
    lib.lvq_channel_perm_check.argtypes = [C.POINTER(lvq_geom), _P]
    lib.lvq_rope_table_perm.argtypes = [C.POINTER(lvq_geom), _P, _I, C.c_double, _P, _P, _P, _P]
    lib.lvq_encode.argtypes = [C.POINTER(lvq_geom), _I, _P, _P, C.POINTER(C.c_int64), _P, _P, _P, _P, _I,
                               _P, _P, _I, _I, _P]
    lib.lvq_decode_attn_workspace.restype = _S
    lib.lvq_decode_attn_workspace.argtypes = [C.POINTER(lvq_geom), _I, _I, _I]
    lib.lvq_decode_attn.argtypes = [C.POINTER(lvq_geom), _I, _P, _P, _P, _I, _P, _I, _P, _P, _P, _P, _P, _P, _P,
                                    _P, _I, C.c_float, _P, _P, _P, _S, _I, _I, _P]
    lib.lvq_decode_attn_noalloc.argtypes = [C.POINTER(lvq_geom), _I, _P, _P, _P, _I, _P, _I, _P, _P, _P, _P, _P,
                                            _P, _P, _P, _I, C.c_float, _P, _P, _I, _I, _P]
    lib.lvq_request_order.argtypes = [_P, _I, _I, _P, _P]
    lib.lvq_check_pages.argtypes = [C.POINTER(lvq_geom), _P, _I, _P, _I, _I, _I, _P, _P]
    lib.lvq_window_append.argtypes = [C.POINTER(lvq_geom), _I, _P, _P, _P, _P, _P, _I, _I, _P]
    lib.lvq_codebook_update.argtypes = [C.POINTER(lvq_geom), _I, _P, _P, C.POINTER(C.c_int64), _P, _P, _P,
                                        C.POINTER(C.c_int64), _P, _P, _P, _I, _P, _P, _I, _I, _P]
    lib.lvq_decode_attn_splits.restype = _I
    lib.lvq_decode_attn_splits.argtypes = [C.POINTER(lvq_geom), _I, _I]
    lib.lvq_quant_partial.argtypes = [C.POINTER(lvq_geom), _I, _P, _P, _P, _I, _P, _I, _P, _P, _P, _P, _P, _P,
                                      _I, C.c_float, _P, _P, _I, _I, _P, _S, _I, _P]
    lib.lvq_quant_partial_workspace.restype = _S
    lib.lvq_quant_partial_workspace.argtypes = [C.POINTER(lvq_geom), _I, _I]
    lib.lvq_window_partial.argtypes = [C.POINTER(lvq_geom), _I, _P, _P, _I, _P, _P, _P, _P, _I, C.c_float, _P, _P,
                                       _I, _I, _I, _P]
    lib.splitk_lse_merge.argtypes = [_P, _P, _I, _I, _I, _P, _P, _P]
    lib.kivi_append.argtypes = [C.POINTER(kivi_geom), _P, _P, C.POINTER(C.c_int64), _I, _I,
                                C.POINTER(kivi_cache), _I, _P]
    lib.kivi_decode_attn_workspace.restype = _S
    lib.kivi_decode_attn_workspace.argtypes = [C.POINTER(kivi_geom), _I, _I, _I]
    lib.kivi_decode_attn.argtypes = [C.POINTER(kivi_geom), _P, C.POINTER(kivi_cache), _I, C.c_float, _P, _P, _P,
                                     _S, _I, _I, _P]
    for name in ("lvq_slice_codebooks", "lvq_rope_table", "lvq_rope_table_f16", "lvq_channel_perm_check",
                 "lvq_rope_table_perm", "lvq_encode", "lvq_decode_attn",
                 "lvq_decode_attn_noalloc",
                 "lvq_request_order", "lvq_check_pages", "lvq_window_append", "lvq_codebook_update", "lvq_quant_partial",
                 "lvq_window_partial", "splitk_lse_merge",
                 "kivi_append", "kivi_decode_attn"):
        getattr(lib, name).restype = C.c_int
    return lib


lib = _load()


def check(status: int, fn: str):
    if status != 0:
        raise LvqError(status, fn, lib.lvq_last_error().decode(errors="replace"))
