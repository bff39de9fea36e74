"""ctypes view of libbca.so (include/bca.h).  Argument marshalling only."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbca.so")

BCA_OK = 0
BCA_ERR_ARG = 1
BCA_ERR_BLOCK_IDS = 2
BCA_ERR_UNSUPPORTED = 3
BCA_ERR_NO_DECODE = 4
BCA_ERR_ALLOC = 5
BCA_ERR_HIP = 6
BCA_PLAN_HOST_ONLY = 1
BCA_CACHE_BF16 = 0
BCA_CACHE_FP8_V = 1
BCA_CACHE_FP8_KV = 2

# every symbol include/bca.h declares
EXPORTED = ("bca_plan", "bca_plan_free", "bca_plan_get_info", "bca_plan_export", "bca_prefill",
            "bca_decode", "bca_prefill_ex", "bca_decode_ex", "bca_rope_positions", "bca_rope_table",
            "bca_qk_prologue", "bca_plan_varlen", "bca_prefill_varlen",
            "bca_decode_split_workspace", "bca_decode_split", "bca_cache_dequantize",
            "bca_decode_split_noalloc", "bca_plan_sequences", "bca_decode_varlen",
            "bca_decode_layout", "bca_prefill_layout", "bca_status_str", "bca_last_error")
BCA_SCRATCH_BYTES = 64 << 20


class BcaTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("stride_b", ctypes.c_int64),
                ("stride_s", ctypes.c_int64), ("stride_h", ctypes.c_int64)]


class BcaKvCache(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("k", BcaTensor), ("v", BcaTensor),
                ("k_scale", BcaTensor), ("v_scale", BcaTensor)]


class BcaPlanInfo(ctypes.Structure):
    _fields_ = [("seq_len", ctypes.c_int64), ("prefix_len", ctypes.c_int64),
                ("target_len", ctypes.c_int64), ("useful_pairs", ctypes.c_int64),
                ("n_segments", ctypes.c_int32), ("block_m", ctypes.c_int32),
                ("block_n", ctypes.c_int32), ("n_qtiles", ctypes.c_int32),
                ("decode_ok", ctypes.c_int32), ("host_only", ctypes.c_int32),
                ("n_sequences", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("rows", ctypes.c_int64)]


_lib = None


def load() -> ctypes.CDLL:
    """Load the HIP library; raises if it has not been built (there is no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libbca.so not found at {LIB_PATH}: build it with "
                          "`python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    T = ctypes.POINTER(BcaTensor)
    i32p = ctypes.POINTER(ctypes.c_int32)
    lib.bca_plan.argtypes = [i32p, ctypes.c_int64, ctypes.c_uint32, ctypes.POINTER(P)]
    lib.bca_plan_free.argtypes = [P]
    lib.bca_plan_get_info.argtypes = [P, ctypes.POINTER(BcaPlanInfo)]
    lib.bca_plan_export.argtypes = [P, i32p, i32p, i32p, i32p, i32p]
    lib.bca_prefill.argtypes = [P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_float,
                                T, T, T, T, T, T, P]
    lib.bca_decode.argtypes = [P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_float,
                               T, T, T, T, T, T, P]
    C = ctypes.POINTER(BcaKvCache)
    lib.bca_prefill_ex.argtypes = [P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_float, T, T, T, T, C, P]
    lib.bca_decode_ex.argtypes = [P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                  ctypes.c_float, T, C, T, T, T, P]
    f32p = ctypes.POINTER(ctypes.c_float)
    lib.bca_rope_positions.argtypes = [i32p, ctypes.c_int64, i32p, ctypes.c_int32, i32p]
    lib.bca_rope_table.argtypes = [i32p, ctypes.c_int64, ctypes.c_double, f32p]
    lib.bca_qk_prologue.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_float, T, T, T, T, P, P, P, P]
    i64p = ctypes.POINTER(ctypes.c_int64)
    lib.bca_plan_varlen.argtypes = [i32p, i64p, i64p, ctypes.c_int32, ctypes.c_uint32,
                                    ctypes.POINTER(P)]
    lib.bca_prefill_varlen.argtypes = [P, ctypes.c_int32, ctypes.c_int32, ctypes.c_float,
                                       T, T, T, T, T, T, P]
    lib.bca_plan_sequences.argtypes = [P, i64p]
    lib.bca_decode_varlen.argtypes = [P, ctypes.c_int32, ctypes.c_int32, ctypes.c_float,
                                      T, T, T, T, T, T, P]
    lib.bca_decode_split_workspace.argtypes = [P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                               i64p, i32p]
    lib.bca_decode_split.argtypes = [P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_float, T, C, T, T, T, ctypes.c_int32, P,
                                     ctypes.c_int64, P]
    lib.bca_cache_dequantize.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                         ctypes.c_int32, C, T, T, P]
    lib.bca_decode_split_noalloc.argtypes = [P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_float, T, C, T, T, T, ctypes.c_int32, P]
    lib.bca_decode_layout.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.c_int32, i32p]
    lib.bca_prefill_layout.argtypes = [P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, i32p]
    lib.bca_status_str.argtypes = [ctypes.c_int]
    lib.bca_status_str.restype = ctypes.c_char_p
    lib.bca_last_error.argtypes = []
    lib.bca_last_error.restype = ctypes.c_char_p
    for name in ("bca_plan", "bca_plan_free", "bca_plan_get_info", "bca_plan_export",
                 "bca_prefill", "bca_decode", "bca_prefill_ex", "bca_decode_ex",
                 "bca_rope_positions", "bca_rope_table", "bca_qk_prologue", "bca_plan_varlen",
                 "bca_prefill_varlen", "bca_decode_split_workspace", "bca_decode_split",
                 "bca_cache_dequantize", "bca_decode_split_noalloc", "bca_plan_sequences",
                 "bca_decode_varlen", "bca_decode_layout", "bca_prefill_layout"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib
