"""ctypes binding of libtq4.so (the C ABI in include/tq4.h).

Argument marshalling only: every step of encode and attention runs in the HIP
kernels of libtq4.so.  PyTorch supplies device memory and the current stream.
If the library is missing the first call raises; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB_PATH = os.path.join(PKG, "libtq4.so")
HEADER = os.path.join(ROOT, "include", "tq4.h")

TQ4_OK = 0
TQ4_F32, TQ4_BF16, TQ4_F16 = 0, 1, 2
STATUS_NAMES = {0: "TQ4_OK", 1: "TQ4_ERR_NULL", 2: "TQ4_ERR_SHAPE", 3: "TQ4_ERR_DTYPE",
                4: "TQ4_ERR_ALIGN", 5: "TQ4_ERR_WORKSPACE", 6: "TQ4_ERR_HIP", 7: "TQ4_ERR_CAPACITY",
                8: "TQ4_ERR_VALUE"}
TQ4_ERR_CAPACITY = 7
TQ4_DECODE_FUSED, TQ4_DECODE_VALU_ROTATED, TQ4_DECODE_VALU_LITERAL = 0, 1, 2


class Tq4Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class tq4_layer_pool(ctypes.Structure):
    _fields_ = [("k_words", ctypes.c_void_p), ("v_words", ctypes.c_void_p),
                ("k_norms", ctypes.c_void_p), ("v_norms", ctypes.c_void_p),
                ("num_pages", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32)]


class tq4_int8_pool(ctypes.Structure):
    _fields_ = [("k_codes", ctypes.c_void_p), ("v_codes", ctypes.c_void_p),
                ("k_scales", ctypes.c_void_p), ("v_scales", ctypes.c_void_p),
                ("num_pages", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32)]


_lib = None


def load_library(path: str | None = None):
    """Load libtq4.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m compressed_kv_attention_kvexec_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    pool_p = ctypes.POINTER(tq4_layer_pool)
    st = ctypes.c_int
    lib.tq4_abi_version.argtypes, lib.tq4_abi_version.restype = [], ctypes.c_int
    lib.tq4_status_string.argtypes, lib.tq4_status_string.restype = [st], ctypes.c_char_p
    lib.tq4_codebook.argtypes = [ctypes.POINTER(f32), ctypes.POINTER(f32)]
    lib.tq4_codebook.restype = st
    lib.tq4_encode_pages.argtypes = [pool_p, vp, vp, st, vp, i32, vp]
    lib.tq4_encode_pages.restype = st
    lib.tq4_attn_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    lib.tq4_attn_decode_workspace_size.restype = sz
    lib.tq4_attn_decode.argtypes = [pool_p, vp, st, vp, i32, vp, i32, i32, i32, f32, vp, vp, sz, vp]
    lib.tq4_attn_decode.restype = st
    lib.tq4_attn_decode_noalloc.argtypes = [pool_p, vp, st, vp, i32, vp, i32, i32, i32, f32, vp, vp]
    lib.tq4_attn_decode_noalloc.restype = st
    lib.tq4_attn_decode_variant.argtypes = [pool_p, vp, st, vp, i32, vp, i32, i32, i32, f32, ctypes.c_int, vp, vp,
                                            sz, vp]
    lib.tq4_attn_decode_variant.restype = st
    lib.tq4_attn_decode_append.argtypes = [pool_p, vp, vp, st, vp, vp, st, vp, i32, vp, i32, i32, i32, f32, vp,
                                           vp, sz, vp]
    lib.tq4_attn_decode_append.restype = st
    lib.tq4_attn_verify_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.tq4_attn_verify_workspace_size.restype = sz
    lib.tq4_attn_verify.argtypes = [pool_p, vp, st, i32, vp, i32, vp, i32, i32, i32, f32, vp, vp, sz, vp]
    lib.tq4_attn_verify.restype = st
    lib.tq4_reconstruct_pages.argtypes = [pool_p, vp, i32, vp, i32, i32, st, vp, vp, vp]
    lib.tq4_reconstruct_pages.restype = st
    lib.tq4_sdpa_decode_workspace_size.argtypes = [i32, i32, i32, i32]
    lib.tq4_sdpa_decode_workspace_size.restype = sz
    lib.tq4_sdpa_decode.argtypes = [vp, st, vp, vp, st, vp, i32, i32, i32, i32, f32, vp, vp, sz, vp]
    lib.tq4_sdpa_decode.restype = st
    lib.tq4_attn_prefill_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    lib.tq4_attn_prefill_workspace_size.restype = sz
    lib.tq4_attn_prefill_chunk.argtypes = [pool_p, vp, st, vp, i32, i32, i32, f32, vp, vp, sz, vp]
    lib.tq4_attn_prefill_chunk.restype = st
    i8p = ctypes.POINTER(tq4_int8_pool)
    lib.tq4_int8_encode_pages.argtypes = [i8p, vp, vp, st, vp, i32, vp]
    lib.tq4_int8_encode_pages.restype = st
    lib.tq4_int8_attn_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    lib.tq4_int8_attn_decode_workspace_size.restype = sz
    lib.tq4_int8_attn_decode.argtypes = [i8p, vp, st, vp, i32, vp, i32, i32, i32, f32, vp, vp, sz, vp]
    lib.tq4_int8_attn_decode.restype = st
    lib.tq4_int8_attn_decode_append.argtypes = [i8p, vp, vp, st, vp, vp, st, vp, i32, vp, i32, i32, i32, f32, vp,
                                                vp, sz, vp]
    lib.tq4_int8_attn_decode_append.restype = st
    lib.tq4_int8_attn_verify_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.tq4_int8_attn_verify_workspace_size.restype = sz
    lib.tq4_int8_attn_verify.argtypes = [i8p, vp, st, i32, vp, i32, vp, i32, i32, i32, f32, vp, vp, sz, vp]
    lib.tq4_int8_attn_verify.restype = st
    lib.tq4_int8_attn_prefill_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    lib.tq4_int8_attn_prefill_workspace_size.restype = sz
    lib.tq4_int8_attn_prefill_chunk.argtypes = [i8p, vp, st, vp, i32, i32, i32, f32, vp, vp, sz, vp]
    lib.tq4_int8_attn_prefill_chunk.restype = st
    pp = ctypes.c_void_p
    i64 = ctypes.c_int64
    lib.tq4_pages_create.argtypes = [i32, i32, ctypes.POINTER(pp)]
    lib.tq4_pages_create.restype = st
    lib.tq4_pages_destroy.argtypes = [pp]
    lib.tq4_pages_destroy.restype = None
    lib.tq4_pages_admission_need.argtypes = [i64, i64, i32]
    lib.tq4_pages_admission_need.restype = i64
    lib.tq4_pages_admit.argtypes = [pp, i64, i64, vp, i32, ctypes.POINTER(i32)]
    lib.tq4_pages_admit.restype = st
    lib.tq4_pages_extend.argtypes = [pp, i32, i64]
    lib.tq4_pages_extend.restype = st
    lib.tq4_pages_table.argtypes = [pp, i32, vp, i32]
    lib.tq4_pages_table.restype = i32
    lib.tq4_pages_finish.argtypes = [pp, i32]
    lib.tq4_pages_finish.restype = st
    lib.tq4_pages_boundary.argtypes = [pp]
    lib.tq4_pages_boundary.restype = st
    lib.tq4_pages_free_count.argtypes = [pp]
    lib.tq4_pages_free_count.restype = i32
    lib.tq4_pages_free_list.argtypes = [pp, vp, i32]
    lib.tq4_pages_free_list.restype = i32
    lib.tq4_pages_refcount.argtypes = [pp, i32]
    lib.tq4_pages_refcount.restype = i32
    lib.tq4_pages_reserved.argtypes = [pp]
    lib.tq4_pages_reserved.restype = i64
    _lib = lib
    return lib


def header_functions() -> list[str]:
    """Names of the functions include/tq4.h declares."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tq4_[a-z0-9_]+)\s*\(", text)))


def check(status: int) -> None:
    if status != TQ4_OK:
        msg = load_library().tq4_status_string(status).decode()
        raise Tq4Error(status, msg)
