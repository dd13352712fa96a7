"""ctypes declarations of libpa.so's C ABI (include/pa.h).

Loading fails loudly: there is no fallback implementation of any call.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpa.so")

PA_F32, PA_BF16, PA_FP8_E4M3 = 0, 1, 2
PA_OK, PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_DTYPE, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_HIP, \
    PA_ERR_NO_BLOCKS, PA_ERR_PENDING, PA_ERR_BOUNDS = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9

ERROR_NAMES = {
    PA_ERR_NULL: "PA_ERR_NULL", PA_ERR_SHAPE: "PA_ERR_SHAPE", PA_ERR_DTYPE: "PA_ERR_DTYPE",
    PA_ERR_UNSUPPORTED: "PA_ERR_UNSUPPORTED", PA_ERR_WORKSPACE: "PA_ERR_WORKSPACE", PA_ERR_HIP: "PA_ERR_HIP",
    PA_ERR_NO_BLOCKS: "PA_ERR_NO_BLOCKS", PA_ERR_PENDING: "PA_ERR_PENDING", PA_ERR_BOUNDS: "PA_ERR_BOUNDS",
}


class PaKvCache(C.Structure):
    _fields_ = [
        ("k_cache", C.c_void_p),
        ("v_cache", C.c_void_p),
        ("k_scale", C.c_void_p),
        ("v_scale", C.c_void_p),
        ("num_blocks", C.c_int32),
        ("num_kv_heads", C.c_int32),
        ("block_size", C.c_int32),
        ("head_dim", C.c_int32),
        ("dtype", C.c_int32),
    ]


# (name, restype, argtypes) for every symbol include/pa.h declares
_P = C.c_void_p
_I = C.c_int32
_CACHE = C.POINTER(PaKvCache)
_IP = C.POINTER(C.c_int32)
SIGNATURES = [
    ("pa_store_kv", C.c_int, [_CACHE, _P, _P, _I, _P, _I, _P]),
    ("pa_copy_blocks", C.c_int, [_CACHE, _P, _I, _P]),
    ("pa_decode_workspace_bytes", C.c_size_t, [_I, _I, _I, _I, _I]),
    ("pa_decode", C.c_int, [_CACHE, _P, _I, _P, _I, _I, _I, C.c_float, _P, _I, _P, _I, _I, _P, C.c_size_t, _P]),
    ("pa_decode_noalloc", C.c_int, [_CACHE, _P, _I, _P, _I, _I, _I, C.c_float, _P, _I, _P, _I, _I, _P]),
    ("pa_decode_append", C.c_int, [_CACHE, _P, _P, _P, _I, _P, _I, _I, _I, C.c_float, _P, _I, _P, _I, _I, _P,
                                   C.c_size_t, _P]),
    ("pa_decode_time_next", C.c_int, [_P, _P]),
    ("pa_prefill_chunk", C.c_int, [_CACHE, _P, _I, _P, _I, _I, _I, C.c_float, _P, _P, _P, _I, _I, _I, _P,
                                   C.c_size_t, _P]),
    ("pa_pack_kv", C.c_int, [_CACHE, _P, _I, _P, _P, _I, _I, _P, _P, _P]),
    ("pa_last_error", C.c_char_p, []),
    ("pa_check_slots", C.c_int, [_CACHE, _IP, _I]),
    ("pa_check_copy_pairs", C.c_int, [_CACHE, _IP, _I]),
    ("pa_check_tables", C.c_int, [_CACHE, _IP, _I, _IP, _I, _I]),
    ("pa_check_chunks", C.c_int, [_CACHE, _IP, _IP, _I, _I]),
    ("pa_check_scales", C.c_int, [_CACHE, C.POINTER(C.c_float), C.POINTER(C.c_float)]),
    ("pa_bm_create", C.c_void_p, [_I, _I, _IP]),
    ("pa_bm_destroy", None, [C.c_void_p]),
    ("pa_bm_seq_new", C.c_int32, [C.c_void_p]),
    ("pa_bm_append", C.c_int32, [C.c_void_p, _I, _I, _IP]),
    ("pa_bm_fork", C.c_int32, [C.c_void_p, _I]),
    ("pa_bm_release", C.c_int, [C.c_void_p, _I]),
    ("pa_bm_take_copies", C.c_int32, [C.c_void_p, _IP, _I]),
    ("pa_bm_seq_len", C.c_int32, [C.c_void_p, _I]),
    ("pa_bm_block_table", C.c_int32, [C.c_void_p, _I, _IP, _I]),
    ("pa_bm_used_blocks", C.c_int32, [C.c_void_p]),
    ("pa_bm_ref_count", C.c_int32, [C.c_void_p, _I]),
    ("pa_bm_prefix_cache_set_capacity", C.c_int, [C.c_void_p, _I]),
    ("pa_bm_prefix_lookup", C.c_int32, [C.c_void_p, _IP, _I, _IP, _I]),
    ("pa_bm_seq_new_prefixed", C.c_int32, [C.c_void_p, _IP, _I]),
    ("pa_bm_prefix_insert", C.c_int32, [C.c_void_p, _I, _IP, _I]),
    ("pa_bm_prefix_stats", C.c_int, [C.c_void_p, C.POINTER(C.c_int64)]),
]

_lib = None


def lib() -> C.CDLL:
    """The loaded libpa.so; raises if it is missing or incomplete."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libpa.so not found at {LIB_PATH}: build it with "
                              f"`python -m paged_kv_attention_26_amd.build` (hipcc, gfx950)")
        handle = C.CDLL(LIB_PATH)
        for name, res, args in SIGNATURES:
            fn = getattr(handle, name)          # AttributeError names a missing export
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


class PaError(RuntimeError):
    def __init__(self, code: int, where: str):
        msg = lib().pa_last_error().decode(errors="replace")
        super().__init__(f"{where} failed: {ERROR_NAMES.get(code, code)}: {msg}")
        self.code = code


def check(code: int, where: str) -> None:
    if code != PA_OK:
        raise PaError(code, where)
