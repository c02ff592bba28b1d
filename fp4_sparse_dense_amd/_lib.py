"""ctypes view of libsharq.so (the C ABI in include/sharq.h).

Loading fails loudly when the library has not been built: there is no
fallback path of any kind.
"""
from __future__ import annotations

import ctypes as C
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsharq.so")

SHARQ_ABI_VERSION = 1

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = range(5)
FMT_MXFP4, FMT_NVFP4, FMT_HIF4 = 0, 1, 2
OUT_F32, OUT_BF16 = 0, 1
PATH_SPARSE, PATH_DENSE = 0, 1


class ScaleView(C.Structure):
    _fields_ = [("base", C.c_void_p), ("ld", C.c_int64), ("block", C.c_int32), ("reserved", C.c_int32)]


class WeightDesc(C.Structure):
    _fields_ = [
        ("struct_size", C.c_uint32), ("layout_version", C.c_uint32),
        ("N", C.c_int64), ("K", C.c_int64),
        ("fmt", C.c_int32), ("reserved", C.c_int32),
        ("codes", C.c_void_p), ("scales", C.c_void_p),
        ("view", ScaleView * 2),
    ]


class ActDesc(C.Structure):
    _fields_ = [
        ("struct_size", C.c_uint32), ("layout_version", C.c_uint32),
        ("M", C.c_int64), ("K", C.c_int64),
        ("n", C.c_int32), ("m", C.c_int32),
        ("fmt", C.c_int32), ("reserved", C.c_int32),
        ("s_codes", C.c_void_p), ("s_meta", C.c_void_p), ("s_scales", C.c_void_p),
        ("r_codes", C.c_void_p), ("r_scales", C.c_void_p),
    ]


# name -> (restype, argtypes); mirrors include/sharq.h, sharq_peak.h and sharq_check.h
PROTOTYPES = {
    "sharq_abi_version": (C.c_int, []),
    "sharq_status_str": (C.c_char_p, [C.c_int]),
    "sharq_last_error": (C.c_char_p, []),
    "sharq_weight_bytes": (C.c_int, [C.c_int64, C.c_int64, C.c_int32,
                                     C.POINTER(C.c_size_t), C.POINTER(C.c_size_t)]),
    "sharq_act_bytes": (C.c_int, [C.c_int64, C.c_int64, C.c_int32, C.c_int32, C.c_int32,
                                  C.POINTER(C.c_size_t)]),
    "sharq_pack_weight": (C.c_int, [C.c_void_p, C.c_int64, C.c_int64, C.c_int64, C.c_int32,
                                    C.POINTER(WeightDesc), C.c_void_p]),
    "sharq_prepare": (C.c_int, [C.c_void_p, C.c_int64, C.c_int64, C.c_int64, C.c_void_p, C.c_float,
                                C.c_int32, C.c_int32, C.c_int32, C.POINTER(ActDesc), C.c_void_p]),
    "sharq_linear": (C.c_int, [C.POINTER(ActDesc), C.POINTER(WeightDesc), C.c_void_p, C.c_int64,
                               C.c_int32, C.c_void_p]),
    "sharq_grouped_workspace_bytes": (C.c_int, [C.c_int64, C.c_int32, C.c_int64, C.POINTER(C.c_size_t)]),
    "sharq_linear_grouped": (C.c_int, [C.POINTER(ActDesc), C.c_void_p, C.c_int64, C.c_void_p, C.c_int32,
                                       C.POINTER(WeightDesc), C.c_void_p, C.c_int64, C.c_int32,
                                       C.c_void_p, C.c_size_t, C.c_void_p]),
    "sharq_linear_grouped_noalloc": (C.c_int, [C.POINTER(ActDesc), C.c_void_p, C.c_int64, C.c_void_p, C.c_int32,
                                               C.POINTER(WeightDesc), C.c_void_p, C.c_int64, C.c_int32,
                                               C.c_void_p]),
    "sharq_linear_grouped_swiglu_prep": (C.c_int, [C.POINTER(ActDesc), C.c_void_p, C.c_int64, C.c_void_p,
                                                   C.c_int32, C.POINTER(WeightDesc), C.POINTER(ActDesc),
                                                   C.c_void_p, C.c_size_t, C.c_void_p]),
    "sharq_noalloc_scratch_bytes": (C.c_size_t, []),
    "sharq_rmsnorm": (C.c_int, [C.c_void_p, C.c_int64, C.c_int64, C.c_int64, C.c_void_p, C.c_float,
                                C.c_void_p, C.c_int64, C.c_void_p]),
    "sharq_add_f32": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int64, C.c_void_p]),
    "sharq_add_bf16_f32": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int64, C.c_void_p]),
    "sharq_linear_swiglu_prep": (C.c_int, [C.POINTER(ActDesc), C.POINTER(WeightDesc), C.POINTER(ActDesc),
                                           C.c_void_p]),
    "sharq_linear_residual": (C.c_int, [C.POINTER(ActDesc), C.POINTER(WeightDesc), C.c_void_p, C.c_int64,
                                        C.c_void_p, C.c_int64, C.c_void_p]),
    "sharq_linear_swiglu": (C.c_int, [C.POINTER(ActDesc), C.POINTER(WeightDesc), C.c_void_p, C.c_int64,
                                      C.c_void_p]),
    "sharq_peak_fp4_mfma": (C.c_int, [C.c_void_p, C.c_size_t, C.c_int32, C.c_void_p, C.POINTER(C.c_double),
                                      C.c_void_p]),
    "sharq_peak_read": (C.c_int, [C.c_void_p, C.c_size_t, C.c_void_p, C.POINTER(C.c_double), C.c_void_p]),
    "sharq_check_e2m1": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int64, C.c_int32, C.c_void_p, C.c_void_p,
                                   C.c_void_p, C.c_void_p, C.c_void_p]),
    "sharq_check_e4m3": (C.c_int, [C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]),
    "sharq_check_mfma_fp4": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p,
                                       C.c_void_p]),
    "sharq_linear_fused": (C.c_int, [C.c_void_p, C.c_int64, C.c_int64, C.c_int64, C.c_void_p, C.c_float,
                                     C.c_int32, C.c_int32, C.c_int32, C.POINTER(WeightDesc), C.c_void_p,
                                     C.c_int64, C.c_int32, C.c_void_p]),
}

_LIB = None


def load() -> C.CDLL:
    """Load libsharq.so once; raises if it is missing."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m fp4_sparse_dense_amd.build`")
        lib = C.CDLL(LIB_PATH)
        for name, (res, args) in PROTOTYPES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        if lib.sharq_abi_version() != SHARQ_ABI_VERSION:
            raise RuntimeError("libsharq.so ABI version mismatch")
        _LIB = lib
    return _LIB


class SharqError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = load()
        detail = lib.sharq_last_error().decode()
        super().__init__(f"{where}: {lib.sharq_status_str(status).decode()} ({detail})")
        self.status = status


def check(status: int, where: str) -> None:
    if status != OK:
        raise SharqError(status, where)
