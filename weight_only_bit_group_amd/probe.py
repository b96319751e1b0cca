"""ctypes loader of libaq_probe.so: the ceiling microbenchmarks (empty kernel, pure
streaming read, MFMA-only loop) that the benchmark measures beside the hot path, so
its roofline fractions can be stated against measured as well as nameplate peaks.
Not part of the library's C ABI."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libaq_probe.so")

_P, _I32, _I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
SIGNATURES = {
    "aqp_empty": (_I32, [_I32, _I32, _P]),
    "aqp_stream_read": (_I32, [_P, _I64, _I32, _I32, _P, _P]),
    "aqp_mfma_loop": (_I32, [_I32, _I32, _I32, _P, _P]),
}
_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise OSError(f"libaq_probe.so not found at {LIB_PATH}; run `python -m weight_only_bit_group_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            getattr(lib, name).restype = res
            getattr(lib, name).argtypes = args
        _lib = lib
    return _lib


def _check(st: int, name: str) -> None:
    if st != 0:
        raise RuntimeError(f"{name}: HIP error {st}")


def empty(blocks: int, threads: int, stream: int) -> None:
    _check(load().aqp_empty(blocks, threads, stream), "aqp_empty")


def stream_read(src_ptr: int, nbytes: int, blocks: int, unroll: int, sink_ptr: int, stream: int) -> None:
    _check(load().aqp_stream_read(src_ptr, nbytes, blocks, unroll, sink_ptr, stream), "aqp_stream_read")


def mfma_loop(big: bool, blocks: int, iters: int, sink_ptr: int, stream: int) -> None:
    _check(load().aqp_mfma_loop(1 if big else 0, blocks, iters, sink_ptr, stream), "aqp_mfma_loop")
