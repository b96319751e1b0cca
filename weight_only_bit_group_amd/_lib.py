"""ctypes loader for libaq.so (the C ABI declared in include/aq.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation anywhere in the package.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libaq.so")

AQ_OK, AQ_EINVAL, AQ_ERUNTIME = 0, 1, 2
AQ_F32, AQ_BF16 = 0, 1

# name -> (restype, argtypes); mirrors include/aq.h
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t
SIGNATURES = {
    "aq_quantize_pack": (_I32, [_P, _I32, _I64, _I64, _I32, _P, _P, _P, _P, _P]),
    "aq_quantize_pack_sym": (_I32, [_P, _I32, _I64, _I64, _I32, _P, _P, _P, _P, _P]),
    "aq_quantize_pack8": (_I32, [_P, _I32, _I64, _I64, _I32, _P, _P, _P, _P, _P]),
    "aq_w8a16_gemv": (_I32, [_P, _I64, _I64, _P, _P, _P, _I64, _I32, _P, _P]),
    "aq_w8a16_gemm_workspace": (_SZ, [_I64, _I64, _I64, _I32]),
    "aq_w8a16_gemm": (_I32, [_P, _I64, _I64, _P, _P, _P, _I64, _I32, _P, _P, _SZ, _P]),
    "aq_w4a16_gemv": (_I32, [_P, _I64, _I64, _P, _P, _P, _I64, _I32, _P, _P]),
    "aq_w4a16_gemm_workspace": (_SZ, [_I64, _I64, _I64, _I32]),
    "aq_w4a16_gemm": (_I32, [_P, _I64, _I64, _P, _P, _P, _I64, _I32, _P, _P, _SZ, _P]),
    "aq_act_absmean_workspace": (_SZ, [_I64, _I64]),
    "aq_act_absmean": (_I32, [_P, _I64, _I64, _P, _P, _I64, _P, _SZ, _P]),
    "aq_act_absmean_noalloc": (_I32, [_P, _I64, _I64, _P, _P, _I64, _P]),
    "aq_awq_search_workspace": (_SZ, [_I64, _I64, _I64, _I32, _I32]),
    "aq_awq_search": (_I32, [_P, _I64, _P, _P, _I32, _I64, _I64, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "aq_awq_fold_norm": (_I32, [_P, _I32, _P, _I64, _P, _P]),
    "aq_fp4_gemm_workspace": (_SZ, [_I64, _I64, _I64]),
    "aq_fp4_gemm": (_I32, [_P, _I64, _I64, _P, _P, ctypes.c_float, _I64, _P, _P, _SZ, _P]),
    "aq_fp4_quantize_workspace": (_SZ, [_I64, _I64]),
    "aq_fp4_quantize": (_I32, [_P, _I32, _I64, _I64, _P, _P, _P, _P, _SZ, _P]),
    "aq_last_error": (ctypes.c_char_p, []),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load libaq.so once and attach the prototypes; raises OSError if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise OSError(f"libaq.so not found at {LIB_PATH}; build it with "
                      "`python -m weight_only_bit_group_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def last_error() -> str:
    msg = load().aq_last_error()
    return msg.decode() if msg else ""


def check(status: int, name: str) -> None:
    """Map a status code to the Python convention: 1 -> ValueError, 2 -> RuntimeError."""
    if status == AQ_OK:
        return
    msg = f"{name}: {last_error()}"
    if status == AQ_EINVAL:
        raise ValueError(msg)
    raise RuntimeError(msg)
