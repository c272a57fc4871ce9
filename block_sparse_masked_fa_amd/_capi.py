"""ctypes view of include/flexattn.h: structs, enums and the loaded library.

Argument marshalling only. The library is loaded on first use; if it is
missing the call fails loudly (there is no other implementation to fall
back to).
"""
from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libflexattn.so")

# fa_status
FA_OK = 0
FA_ERR_NULL_POINTER = 1
FA_ERR_INVALID_VALUE = 2
FA_ERR_UNSUPPORTED = 3
FA_ERR_SHAPE_MISMATCH = 4
FA_ERR_HIP = 5

# fa_dtype
FA_BF16 = 0
FA_FP32 = 1

# fa_mask_kind
FA_MASK_NONE = 0
FA_MASK_CAUSAL = 1
FA_MASK_SLIDING_WINDOW = 2
FA_MASK_DOCUMENT = 3
FA_MASK_LOCAL_WINDOW = 4

# fa_score_kind
FA_SCORE_NONE = 0
FA_SCORE_SOFTCAP = 1
FA_SCORE_ALIBI = 2

# largest num_splits of fa_flex_attention_fwd_split
FA_MAX_SPLITS = 64

# bytes of the forward's scheduler workspace
FA_FWD_WORKSPACE_BYTES = 256

# bytes of fa_flex_attention_fwd_split_noalloc's fixed device scratch
FA_NOALLOC_SCRATCH_BYTES = 32 << 20

ABI_VERSION = 9


class fa_mask_mod(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32),
                ("window", ctypes.c_int32),
                ("doc_id", ctypes.c_void_p),
                ("doc_len", ctypes.c_int64),
                ("doc_stride", ctypes.c_int64)]


class fa_score_mod(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32),
                ("softcap", ctypes.c_float)]


class fa_block_mask(ctypes.Structure):
    _fields_ = [("mask", fa_mask_mod),
                ("B", ctypes.c_int32),
                ("H", ctypes.c_int32),
                ("q_len", ctypes.c_int32),
                ("kv_len", ctypes.c_int32),
                ("block_m", ctypes.c_int32),
                ("block_n", ctypes.c_int32),
                ("num_q_blocks", ctypes.c_int32),
                ("num_kv_blocks", ctypes.c_int32),
                ("separate_full_blocks", ctypes.c_int32),
                ("kv_num_blocks", ctypes.c_void_p),
                ("kv_indices", ctypes.c_void_p),
                ("full_kv_num_blocks", ctypes.c_void_p),
                ("full_kv_indices", ctypes.c_void_p)]


Stride3 = ctypes.c_int64 * 3
Stride2 = ctypes.c_int64 * 2

# name -> (restype, argtypes); every function include/flexattn.h declares
SIGNATURES = {
    "fa_block_mask_dims": (ctypes.c_int, [
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]),
    "fa_create_block_mask": (ctypes.c_int, [
        ctypes.POINTER(fa_mask_mod), ctypes.c_int32, ctypes.c_int32,
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_int32, ctypes.POINTER(fa_block_mask), ctypes.c_void_p]),
    "fa_flex_attention_fwd": (ctypes.c_int, [
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64),
        ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64),
        ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64),
        ctypes.c_float, ctypes.POINTER(fa_block_mask),
        ctypes.POINTER(fa_score_mod), ctypes.c_void_p, ctypes.c_uint64,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "fa_flex_attention_fwd_split": (ctypes.c_int, [
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64),
        ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64),
        ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64),
        ctypes.c_float, ctypes.POINTER(fa_block_mask),
        ctypes.POINTER(fa_score_mod), ctypes.c_int32, ctypes.c_void_p,
        ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "fa_flex_attention_fwd_split_noalloc": (ctypes.c_int, [
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64),
        ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64),
        ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64),
        ctypes.c_float, ctypes.POINTER(fa_block_mask),
        ctypes.POINTER(fa_score_mod), ctypes.c_int32, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p]),
    "fa_split_workspace_bytes": (ctypes.c_int, [
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_int32, ctypes.POINTER(ctypes.c_uint64)]),
    "fa_flex_attention_bwd": (ctypes.c_int, [
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64),
        ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64),
        ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64),
        ctypes.c_float, ctypes.POINTER(fa_block_mask),
        ctypes.POINTER(fa_score_mod), ctypes.c_int32, ctypes.c_int32,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p]),
    "fa_bwd_workspace_bytes": (ctypes.c_int, [
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(fa_block_mask),
        ctypes.c_int32, ctypes.POINTER(ctypes.c_uint64)]),
    "fa_flex_attention_decode_paged": (ctypes.c_int, [
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64),
        ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64),
        ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64),
        ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
        ctypes.c_void_p, ctypes.c_float, ctypes.POINTER(fa_mask_mod),
        ctypes.POINTER(fa_score_mod), ctypes.c_int32, ctypes.c_void_p,
        ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "fa_masked_softmax": (ctypes.c_int, [
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
        ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64),
        ctypes.POINTER(fa_mask_mod), ctypes.c_void_p, ctypes.c_void_p]),
    "fa_status_string": (ctypes.c_char_p, [ctypes.c_int32]),
    "fa_last_error": (ctypes.c_char_p, []),
    "fa_abi_version": (ctypes.c_int32, []),
}

_lock = threading.Lock()
_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libflexattn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with "
                    "`python -m block_sparse_masked_fa_amd.build` "
                    "(there is no non-HIP implementation)")
            handle = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(handle, name)
                fn.restype = res
                fn.argtypes = args
            if handle.fa_abi_version() != ABI_VERSION:
                raise RuntimeError("libflexattn.so ABI version mismatch")
            _lib = handle
    return _lib


class FlexAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        L = lib()
        name = L.fa_status_string(status).decode()
        detail = L.fa_last_error().decode()
        super().__init__(f"{where}: {name}: {detail}")
        self.status = status


def check(status: int, where: str) -> None:
    if status != FA_OK:
        raise FlexAttnError(status, where)
