"""ctypes declarations of libda.so (the C ABI in include/da.h)."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libda.so")

DA_OK, DA_E_INVALID, DA_E_UNSUPPORTED, DA_E_WORKSPACE, DA_E_NOT_PINNED, DA_E_HIP = range(6)
DA_F32, DA_F16, DA_BF16 = 0, 1, 2

c_i32, c_i64, c_f32, c_vp, c_sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t


class DaAttnShape(ctypes.Structure):
    _fields_ = [
        ("batch", c_i32),
        ("n_q_heads", c_i32),
        ("n_kv_heads", c_i32),
        ("head_dim", c_i32),
        ("n_ctx", c_i64),
        ("scale", c_f32),
        ("q_dtype", c_i32),
        ("kv_dtype", c_i32),
        ("split_tokens", c_i32),
    ]


class DaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_name(status)}: {message}")
        self.status = status


_P = ctypes.POINTER
SHAPE = _P(DaAttnShape)

# name -> (restype, argtypes)
SIGNATURES = {
    "da_version": (ctypes.c_int, []),
    "da_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "da_last_error": (ctypes.c_char_p, []),
    "da_decode_attention_workspace": (c_sz, [SHAPE]),
    "da_decode_attention": (ctypes.c_int, [SHAPE, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "da_decode_attention_n_split": (c_i32, [SHAPE]),
    "da_decode_attention_noalloc_max_scratch": (c_sz, []),
    "da_decode_attention_noalloc": (ctypes.c_int, [SHAPE, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "da_decode_attention_partials": (ctypes.c_int, [SHAPE, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "da_merge_partials": (ctypes.c_int, [c_i64, c_i32, c_i32, c_vp, c_vp, c_vp]),
    "da_build_page_meta": (ctypes.c_int, [SHAPE, c_i32, c_vp, c_vp, c_vp, c_vp]),
    "da_select_pages": (ctypes.c_int, [SHAPE, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "da_select_tokens": (ctypes.c_int, [SHAPE, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "da_token_keep_count": (c_i64, [c_i64]),
    "da_decode_attention_topk": (ctypes.c_int, [SHAPE, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "da_prefill_attention": (ctypes.c_int, [SHAPE, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "da_decode_attention_paged_workspace": (c_sz, [SHAPE, c_i32, c_i32]),
    "da_decode_attention_paged": (ctypes.c_int, [SHAPE, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                                 c_sz, c_vp]),
    "da_quantize_kv4": (ctypes.c_int, [c_i64, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "da_dequantize_kv4": (ctypes.c_int, [c_i64, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "da_decode_attention_kv4_workspace": (c_sz, [SHAPE]),
    "da_decode_attention_kv4": (ctypes.c_int, [SHAPE, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                               c_sz, c_vp]),
    "da_headwise_buffer_bytes": (c_sz, [SHAPE, c_i32]),
    "da_stream_create": (ctypes.c_int, [SHAPE, c_i32, _P(c_vp)]),
    "da_stream_buffer_bytes": (c_sz, [c_vp]),
    "da_stream_workspace": (c_sz, [c_vp]),
    "da_stream_headwise": (ctypes.c_int, [c_vp, c_i32, _P(c_vp), _P(c_vp), c_vp, c_vp, c_vp, c_vp, c_vp,
                                          c_sz, c_vp, c_vp]),
    "da_stream_length": (ctypes.c_int64, [c_vp]),
    "da_stream_set_length": (ctypes.c_int, [c_vp, ctypes.c_int64]),
    "da_stream_append": (ctypes.c_int, [c_vp, c_i32, c_vp, c_vp, _P(c_vp), _P(c_vp), c_vp]),
    "da_stream_destroy": (None, [c_vp]),
    "da_read_stream": (ctypes.c_int, [c_vp, ctypes.c_uint64, c_i32, c_vp, c_vp]),
    "da_decode_attention_sparse": (ctypes.c_int, [SHAPE, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                                  c_vp]),
}

_lib = None


def load(path: str | None = None):
    """Load libda.so (built in-tree); raise if it is missing."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is not built; run `python -m sparse_kv_cache_gqa_amd.build` "
                           "or __graft_entry__.build()")
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def status_name(status: int) -> str:
    names = {0: "DA_OK", 1: "DA_E_INVALID", 2: "DA_E_UNSUPPORTED", 3: "DA_E_WORKSPACE",
             4: "DA_E_NOT_PINNED", 5: "DA_E_HIP"}
    return names.get(status, f"status {status}")


def check(status: int) -> None:
    if status != DA_OK:
        msg = load().da_last_error().decode(errors="replace")
        raise DaError(status, msg)
