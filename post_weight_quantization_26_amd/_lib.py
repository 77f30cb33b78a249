"""ctypes binding of ``libawq_mi355x.so`` (the C ABI declared in include/awq.h).

Argument marshalling only: every step of the computation runs in the HIP
library. Loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
import threading

from .build_lib import LIB_PATH

c_i32, c_i64, c_sz, c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p
c_fp, c_dp = ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_double)

AWQ_OK, AWQ_E_INVALID, AWQ_E_UNSUPPORTED, AWQ_E_WORKSPACE, AWQ_E_RANGE, AWQ_E_HIP = 0, -1, -2, -3, -4, -5
STATUS_NAMES = {0: "AWQ_OK", -1: "AWQ_E_INVALID", -2: "AWQ_E_UNSUPPORTED", -3: "AWQ_E_WORKSPACE",
                -4: "AWQ_E_RANGE", -5: "AWQ_E_HIP"}
AWQ_F32, AWQ_BF16, AWQ_F16 = 0, 1, 2
AWQ_OP_STATS, AWQ_OP_SEARCH_SCALE, AWQ_OP_SEARCH_CLIP, AWQ_OP_PACK = 0, 1, 2, 3
AWQ_OP_SEARCH_SCALE_GRAM, AWQ_OP_SEARCH_CLIP_GRAM = 4, 5
AWQ_OP_GRAM_BUILD, AWQ_OP_SEARCH_SCALE_GRAM_G, AWQ_OP_SEARCH_CLIP_GRAM_G = 6, 7, 8
AWQ_OP_SEARCH_SCALE_SPLIT_E, AWQ_OP_SEARCH_CLIP_SPLIT_E = 9, 10
AWQ_OP_SEARCH_SCALE_FUSED, AWQ_OP_SEARCH_CLIP_FUSED = 11, 12
AWQ_SEARCH_SPLIT_E = 1
AWQ_SEARCH_FUSED = 2
KERNEL_KINDS = {"stats": 0, "scale": 1, "transform": 2, "gemm": 3, "reduce": 4, "pack": 5,
                "fold": 6, "dequant": 7, "w4a16": 8, "w4a16_reduce": 9, "gram_build": 10,
                "gram_search": 11}


class QConfig(ctypes.Structure):
    _fields_ = [("w_bit", c_i32), ("group_size", c_i32), ("zero_point", c_i32),
                ("flags", c_i32)]


class AwqError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


# name -> (restype, argtypes); mirrors include/awq.h
SIGNATURES = {
    "awq_workspace_bytes": (c_sz, [ctypes.c_int, c_i64, c_i64, c_i64, c_i32, ctypes.c_int]),
    "awq_workspace_bytes_batch": (c_sz, [ctypes.c_int, c_i64, c_i64, c_i64, c_i32, c_i32,
                                         ctypes.c_int]),
    "awq_gram_bytes": (c_sz, [c_i64]),
    "awq_gram_build": (ctypes.c_int, [c_vp, ctypes.c_int, c_i64, c_i64, c_vp, c_sz, c_vp, c_sz,
                                      c_vp]),
    "awq_act_stats": (ctypes.c_int, [c_vp, ctypes.c_int, c_i64, c_i64, c_vp, c_vp, c_sz, c_vp]),
    "awq_act_stats_noalloc": (ctypes.c_int, [c_vp, ctypes.c_int, c_i64, c_i64, c_vp, c_vp]),
    "awq_act_stats_accumulate": (ctypes.c_int,
                                 [c_vp, ctypes.c_int, c_i64, c_i64, c_vp, c_vp, c_sz, c_vp]),
    "awq_act_stats_finalize": (ctypes.c_int, [c_vp, c_i64, c_i64, c_vp, c_vp]),
    "awq_scale_table": (ctypes.c_int, [c_vp, c_i64, c_fp, c_i32, c_vp, c_vp]),
    "awq_search_scale": (ctypes.c_int, [c_vp, c_vp, ctypes.c_int, c_i64, c_i64, c_i64, c_vp, c_fp,
                                        c_i32, QConfig, c_vp, c_fp, c_dp, c_vp, c_vp, c_sz, c_vp]),
    "awq_search_clip": (ctypes.c_int, [c_vp, c_vp, ctypes.c_int, c_i64, c_i64, c_i64, c_vp, c_fp,
                                       c_i32, QConfig, c_vp, c_dp, c_vp, c_vp, c_sz, c_vp]),
    "awq_quantize_pack": (ctypes.c_int, [c_vp, ctypes.c_int, c_i64, c_i64, c_vp, c_vp, QConfig,
                                         c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "awq_search_scale_gram": (ctypes.c_int, [c_vp, c_vp, ctypes.c_int, c_i64, c_i64, c_i64, c_vp,
                                             c_fp, c_i32, QConfig, c_vp, c_fp, c_dp, c_vp, c_vp,
                                             c_sz, c_vp]),
    "awq_search_scale_gram_g": (ctypes.c_int, [c_vp, c_vp, ctypes.c_int, c_i64, c_i64, c_i64, c_vp,
                                             c_fp, c_i32, QConfig, c_vp, c_fp, c_dp, c_vp, c_vp,
                                             c_sz, c_vp]),
    "awq_search_clip_gram": (ctypes.c_int, [c_vp, c_vp, ctypes.c_int, c_i64, c_i64, c_i64, c_vp,
                                            c_fp, c_i32, QConfig, c_vp, c_dp, c_vp, c_vp, c_sz,
                                            c_vp]),
    "awq_search_clip_gram_g": (ctypes.c_int, [c_vp, c_vp, ctypes.c_int, c_i64, c_i64, c_i64, c_vp,
                                            c_fp, c_i32, QConfig, c_vp, c_dp, c_vp, c_vp, c_sz,
                                            c_vp]),
    "awq_search_scale_group": (ctypes.c_int, [c_vp, ctypes.POINTER(c_vp), ctypes.POINTER(c_i64),
                                              c_i32, ctypes.c_int, c_i64, c_i64, c_vp, c_fp,
                                              c_i32, QConfig, c_vp, c_fp, c_dp, c_vp, c_vp,
                                              c_sz, c_vp]),
    "awq_search_scale_group_gram": (ctypes.c_int, [c_vp, ctypes.POINTER(c_vp),
                                                   ctypes.POINTER(c_i64), c_i32, ctypes.c_int,
                                                   c_i64, c_i64, c_vp, c_fp, c_i32, QConfig, c_vp,
                                                   c_fp, c_dp, c_vp, c_vp, c_sz, c_vp]),
    "awq_search_scale_group_gram_g": (ctypes.c_int, [c_vp, ctypes.POINTER(c_vp),
                                                   ctypes.POINTER(c_i64), c_i32, ctypes.c_int,
                                                   c_i64, c_i64, c_vp, c_fp, c_i32, QConfig, c_vp,
                                                   c_fp, c_dp, c_vp, c_vp, c_sz, c_vp]),
    "awq_fold_norm": (ctypes.c_int, [c_vp, c_vp, ctypes.c_int, c_i64, c_vp, c_vp]),
    "awq_fold_linear": (ctypes.c_int, [c_vp, c_vp, ctypes.c_int, c_i64, c_i64, c_vp, c_vp]),
    "awq_w4a16_workspace_bytes": (c_sz, [c_i64, c_i64, c_i64, ctypes.c_int]),
    "awq_w3a16_workspace_bytes": (c_sz, [c_i64, c_i64, c_i64, ctypes.c_int]),
    "awq_w4a16_matmul": (ctypes.c_int, [c_vp, ctypes.c_int, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp,
                                        c_i32, c_vp, c_vp, c_sz, c_vp]),
    "awq_w3a16_matmul": (ctypes.c_int, [c_vp, ctypes.c_int, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp,
                                        c_i32, c_vp, c_vp, c_sz, c_vp]),
    "awq_last_error": (ctypes.c_char_p, []),
    "awq_profile_enable": (None, [ctypes.c_int]),
    "awq_profile_reset": (None, []),
    "awq_profile_read": (ctypes.c_int, [ctypes.c_int, c_dp, ctypes.POINTER(c_i64)]),
}

_lib = None
_lock = threading.Lock()


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it was never built)."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise RuntimeError(f"AWQ HIP library not built: {LIB_PATH} is missing "
                                       "(run __graft_entry__.build())")
                L = ctypes.CDLL(LIB_PATH)
                for name, (res, args) in SIGNATURES.items():
                    fn = getattr(L, name)
                    fn.restype = res
                    fn.argtypes = args
                _lib = L
    return _lib


def last_error() -> str:
    msg = lib().awq_last_error()
    return msg.decode() if msg else ""


def check(status: int) -> None:
    if status != AWQ_OK:
        raise AwqError(status, last_error())


def float_array(values):
    vals = [float(v) for v in values]
    return (ctypes.c_float * len(vals))(*vals)
