"""ctypes view of the C-ABI in ``include/twotower_attn.h``.

Loads ``libtwotower_attn.so`` from this package directory. There is no
fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
# TT_LIBRARY selects another build of the library (the sanitizer test loads one)
LIB_PATH = os.environ.get("TT_LIBRARY") or os.path.join(PKG, "libtwotower_attn.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "twotower_attn.h")

TT_F32, TT_BF16 = 0, 1
STATUS = {0: "TT_OK", 1: "TT_ERR_NULL", 2: "TT_ERR_SHAPE", 3: "TT_ERR_DTYPE", 4: "TT_ERR_UNSUPPORTED",
          5: "TT_ERR_WORKSPACE", 6: "TT_ERR_ARG", 7: "TT_ERR_HIP"}

c_i32, c_i64, c_f32, c_ptr, c_size = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t


class BlockAttnParams(ctypes.Structure):
    _fields_ = [
        ("dtype", c_i32), ("o_dtype", c_i32),
        ("B", c_i32), ("S", c_i32), ("Hq", c_i32), ("Hkv", c_i32), ("head_dim", c_i32),
        ("softmax_scale", c_f32),
        ("Q", c_ptr), ("q_stride_b", c_i64), ("q_stride_s", c_i64), ("q_stride_h", c_i64),
        ("Kctx", c_ptr), ("Vctx", c_ptr),
        ("page_size", c_i32), ("num_pages", c_i32),
        ("page_table", c_ptr), ("max_pages", c_i32),
        ("ctx_len", c_ptr), ("max_ctx_len", c_i32),
        ("Kden", c_ptr), ("Vden", c_ptr),
        ("den_stride_b", c_i64), ("den_stride_s", c_i64), ("den_stride_h", c_i64),
        ("O", c_ptr), ("o_stride_b", c_i64), ("o_stride_s", c_i64), ("o_stride_h", c_i64),
        ("LSE", c_ptr), ("debug_flags", c_ptr),
    ]


class ConfUnmaskParams(ctypes.Structure):
    _fields_ = [
        ("dtype", c_i32), ("B", c_i32), ("S", c_i32), ("V", c_i32),
        ("logits", c_ptr), ("logits_stride_row", c_i64),
        ("mask_in", c_ptr), ("mask_out", c_ptr), ("tokens", c_ptr),
        ("gamma", c_f32), ("temperature", c_f32), ("steps_left", c_i32),
        ("conf", c_ptr), ("num_masked", c_ptr), ("uniforms", c_ptr),
    ]


class KvAppendParams(ctypes.Structure):
    _fields_ = [
        ("dtype", c_i32), ("B", c_i32), ("S", c_i32), ("Hkv", c_i32), ("head_dim", c_i32),
        ("Kctx", c_ptr), ("Vctx", c_ptr),
        ("page_size", c_i32), ("num_pages", c_i32), ("max_pages", c_i32),
        ("page_table", c_ptr), ("ctx_len", c_ptr),
        ("Knew", c_ptr), ("Vnew", c_ptr),
        ("new_stride_b", c_i64), ("new_stride_s", c_i64), ("new_stride_h", c_i64),
        ("pool", c_ptr), ("pool_count", c_ptr), ("status", c_ptr),
    ]


class MaskedNllParams(ctypes.Structure):
    _fields_ = [
        ("dtype", c_i32), ("B", c_i32), ("S", c_i32), ("V", c_i32),
        ("logits", c_ptr), ("logits_stride_row", c_i64),
        ("targets", c_ptr), ("mask", c_ptr),
        ("nll", c_ptr), ("loss", c_ptr), ("count", c_ptr),
    ]


class TTError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {STATUS.get(code, code)}")


# parameter-struct layouts above match this version of include/twotower_attn.h
ABI_VERSION = 3

_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m attention_eq_block_amd.build` "
                "(or __graft_entry__.build()); there is no fallback implementation")
        L = ctypes.CDLL(LIB_PATH)
        L.tt_abi_version.restype = ctypes.c_int
        if L.tt_abi_version() != ABI_VERSION:
            raise RuntimeError(f"{LIB_PATH} has ABI version {L.tt_abi_version()}, these bindings need "
                               f"{ABI_VERSION}: rebuild it with `python -m attention_eq_block_amd.build`")
        L.tt_status_string.restype = ctypes.c_char_p
        L.tt_status_string.argtypes = [ctypes.c_int]
        L.tt_block_attn_workspace_bytes.restype = c_size
        L.tt_block_attn_workspace_bytes.argtypes = [ctypes.POINTER(BlockAttnParams)]
        L.tt_block_attn.restype = ctypes.c_int
        L.tt_block_attn.argtypes = [ctypes.POINTER(BlockAttnParams), c_ptr, c_size, c_ptr]
        L.tt_block_attn_noalloc.restype = ctypes.c_int
        L.tt_block_attn_noalloc.argtypes = [ctypes.POINTER(BlockAttnParams), c_ptr]
        L.tt_lse_merge.restype = ctypes.c_int
        L.tt_lse_merge.argtypes = [ctypes.c_int, c_ptr, c_ptr, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, c_ptr, ctypes.c_int, c_ptr, c_ptr]
        L.tt_conf_unmask_workspace_bytes.restype = c_size
        L.tt_conf_unmask_workspace_bytes.argtypes = [ctypes.POINTER(ConfUnmaskParams)]
        L.tt_conf_unmask.restype = ctypes.c_int
        L.tt_conf_unmask.argtypes = [ctypes.POINTER(ConfUnmaskParams), c_ptr, c_size, c_ptr]
        L.tt_kv_append.restype = ctypes.c_int
        L.tt_kv_append.argtypes = [ctypes.POINTER(KvAppendParams), c_ptr]
        L.tt_masked_nll_workspace_bytes.restype = c_size
        L.tt_masked_nll_workspace_bytes.argtypes = [ctypes.POINTER(MaskedNllParams)]
        L.tt_masked_nll.restype = ctypes.c_int
        L.tt_masked_nll.argtypes = [ctypes.POINTER(MaskedNllParams), c_ptr, c_size, c_ptr]
        _lib = L
    return _lib


def header_functions():
    """Names of the functions declared in the public header."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(tt_\w+)\s*\(", text, flags=re.M)))


def check(code: int, what: str):
    if code != 0:
        raise TTError(code, what)
