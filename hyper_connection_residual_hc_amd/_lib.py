"""ctypes declarations of the C ABI in include/hc_mi355x.h.

Loading needs only the built library and the HIP runtime it links; nothing here touches the
GPU. A missing library is an error: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhc_mi355x.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "hc_mi355x.h")

HC_OK = 0

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_f32 = ctypes.c_float
_sz = ctypes.c_size_t
_int = ctypes.c_int

SIGNATURES = {
    "hc_status_string": (ctypes.c_char_p, [_int]),
    "hc_abi_version": (_int, []),
    "hc_fn_packed_bytes": (_sz, [_i32]),
    "hc_fn_pack": (_int, [_p, _i32, _p, _p]),
    "hc_pre_stats_workspace_bytes": (_sz, [_i64, _i32]),
    "hc_pre_stats": (_int, [_p, _i64, _p, _i64, _i32, _f32, _p, _p, _p, _sz, _p]),
    "hc_sinkhorn": (_int, [_p, _i64, _p, _p, _i32, _f32, _f32, _f32, _p, _p, _p, _p]),
    "hc_combine_norm": (_int, [_p, _i64, _p, _i64, _p, _i64, _i32, _f32, _p, _i64, _p]),
    "hc_post": (_int, [_p, _i64, _p, _i64, _p, _p, _i64, _i32, _p, _i64, _p]),
    "mxfp8_quant_rows": (_int, [_p, _i64, _i64, _i32, _p, _i64, _p, _i64, _p]),
    "hc_pre_workspace_bytes": (_sz, [_i64, _i32]),
    "hc_pre": (_int, [_p, _i64, _p, _p, _p, _p, _i64, _i32, _f32, _f32, _f32, _i32, _f32, _f32,
                      _p, _i64, _p, _p, _p, _p, _sz, _p]),
    "hc_post_pre_workspace_bytes": (_sz, [_i64, _i32]),
    "hc_post_pre": (_int, [_p, _i64, _p, _i64, _p, _p, _p, _p, _p, _p, _i64, _i32, _f32, _f32,
                           _f32, _i32, _f32, _f32, _p, _i64, _p, _i64, _p, _p, _p, _p, _sz,
                           _p]),
    "hc_post_pre_noalloc": (_int, [_p, _i64, _p, _i64, _p, _p, _p, _p, _p, _p, _i64, _i32, _f32,
                                   _f32, _f32, _i32, _f32, _f32, _p, _i64, _p, _i64, _p, _p, _p,
                                   _p]),
    "hc_post_stats": (_int, [_p, _i64, _p, _i64, _p, _p, _p, _i64, _i32, _p, _i64, _p, _sz, _p]),
    "hc_pre_finish": (_int, [_p, _i64, _p, _p, _p, _i64, _i32, _f32, _f32, _f32, _i32, _f32, _f32,
                             _p, _i64, _p, _p, _p, _p, _sz, _p]),
    "hc_pre_mxfp8": (_int, [_p, _i64, _p, _p, _p, _p, _i64, _i32, _f32, _f32, _f32, _i32, _f32,
                            _f32, _p, _i64, _p, _i64, _p, _i64, _p, _p, _p, _p, _sz, _p]),
    "hc_post_pre_mxfp8": (_int, [_p, _i64, _p, _i64, _p, _p, _p, _p, _p, _p, _i64, _i32, _f32,
                                 _f32, _f32, _i32, _f32, _f32, _p, _i64, _p, _i64, _p, _i64, _p,
                                 _i64, _p, _p, _p, _p, _sz, _p]),
    "hc_pre_finish_mxfp8": (_int, [_p, _i64, _p, _p, _p, _i64, _i32, _f32, _f32, _f32, _i32,
                                   _f32, _f32, _p, _i64, _p, _i64, _p, _i64, _p, _p, _p, _p, _sz,
                                   _p]),
    "mxfp8_swizzled_bytes": (_sz, [_i64, _i32]),
    "hc_head_fn_pack": (_int, [_p, _i32, _p, _p]),
    "hc_head_workspace_bytes": (_sz, [_i64, _i32]),
    "hc_head": (_int, [_p, _i64, _p, _p, _p, _i64, _i32, _f32, _f32, _p, _i64, _p, _sz, _p]),
    "mxfp8_swizzle_128x4": (_int, [_p, _i64, _i64, _i32, _p, _p]),
}

_LIB = None


class HCError(RuntimeError):
    """A C-ABI call returned a status other than HC_OK."""

    def __init__(self, fn: str, status: int, name: str):
        super().__init__(f"{fn} returned {status} ({name})")
        self.status = status
        self.status_name = name


def header_symbols() -> list[str]:
    """Names of every entry point declared with HC_API in include/hc_mi355x.h."""
    with open(HEADER) as fh:
        text = fh.read()
    return re.findall(r"HC_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


def lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m hyper_connection_residual_hc_amd.build` "
                "(the mHC path has no implementation other than the HIP library)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


def check(fn: str, status: int) -> None:
    if status != HC_OK:
        raise HCError(fn, status, lib().hc_status_string(status).decode())


def call(fn: str, *args) -> None:
    check(fn, getattr(lib(), fn)(*args))
