"""ctypes binding of the C ABI in include/fa2.h (argument marshalling only).

The library is loaded from ``libfa2.so`` in this package directory.  There is
no fallback: if the library is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

from ._build import LIB_PATH

FA2_DTYPE_FP16 = 0
FA2_DTYPE_BF16 = 1

FA2_OK = 0
FA2_ERR_NULL_POINTER = 1
FA2_ERR_BAD_SHAPE = 2
FA2_ERR_UNSUPPORTED_HEAD_DIM = 3
FA2_ERR_UNSUPPORTED_DTYPE = 4
FA2_ERR_BAD_SCALE = 5
FA2_ERR_MISALIGNED = 6
FA2_ERR_OVERLAP = 7
FA2_ERR_HIP = 8
FA2_ERR_TOO_LARGE = 9

# Every symbol include/fa2.h declares.
EXPORTED = ("fa2_fwd", "fa2_fwd_masked", "fa2_bwd", "fa2_bwd_masked", "fa2_bwd_noalloc", "fa2_status_string",
            "fa2_launch_info")

_lock = threading.Lock()
_lib = None


class Fa2Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({fa2_status_string(status)})")


def open_library(path: str) -> ctypes.CDLL:
    """Load a build of the library from `path` with the C signatures declared."""
    lib = ctypes.CDLL(path)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.fa2_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64,
                            ctypes.c_float, ctypes.c_int, ctypes.c_int, vp]
    lib.fa2_fwd.restype = ctypes.c_int
    lib.fa2_fwd_masked.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_float,
                                   i64, i64, vp, ctypes.c_int, vp]
    lib.fa2_fwd_masked.restype = ctypes.c_int
    lib.fa2_bwd.argtypes = [vp] * 10 + [i64, i64, i64, i64, ctypes.c_float, ctypes.c_int, ctypes.c_int, vp]
    lib.fa2_bwd.restype = ctypes.c_int
    lib.fa2_bwd_masked.argtypes = [vp] * 10 + [i64, i64, i64, i64, ctypes.c_float, i64, i64, vp, ctypes.c_int, vp]
    lib.fa2_bwd_masked.restype = ctypes.c_int
    lib.fa2_bwd_noalloc.argtypes = [vp] * 9 + [i64, i64, i64, i64, ctypes.c_float, ctypes.c_int, ctypes.c_int, vp]
    lib.fa2_bwd_noalloc.restype = ctypes.c_int
    lib.fa2_status_string.argtypes = [ctypes.c_int]
    lib.fa2_status_string.restype = ctypes.c_char_p
    lib.fa2_launch_info.argtypes = [i64, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                    ctypes.POINTER(i64), ctypes.POINTER(ctypes.c_int),
                                    ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int),
                                    ctypes.POINTER(ctypes.c_int)]
    lib.fa2_launch_info.restype = ctypes.c_int
    return lib


def library() -> ctypes.CDLL:
    """Load libfa2.so once; raise if it is not built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
            _lib = open_library(LIB_PATH)
        return _lib


def fa2_fwd(Q: int, K: int, V: int, O: int, LSE: int, B: int, H: int, N: int, d: int,
            scale: float, is_causal: int, dtype: int, stream: int) -> int:
    """Same arguments and status as the C function; pointers are integers."""
    return library().fa2_fwd(Q, K, V, O, LSE, B, H, N, d, scale, int(is_causal), int(dtype), stream)


def fa2_fwd_masked(Q: int, K: int, V: int, O: int, LSE: int, B: int, H: int, N: int, d: int,
                   scale: float, window_left: int, window_right: int, key_lens: int | None,
                   dtype: int, stream: int) -> int:
    """Same arguments and status as the C function; pointers are integers (key_lens may be None)."""
    return library().fa2_fwd_masked(Q, K, V, O, LSE, B, H, N, d, scale, int(window_left), int(window_right),
                                    key_lens, int(dtype), stream)


def fa2_bwd(Q: int, K: int, V: int, O: int, dO: int, LSE: int, dQ: int, dK: int, dV: int, workspace: int,
            B: int, H: int, N: int, d: int, scale: float, is_causal: int, dtype: int, stream: int) -> int:
    """Same arguments and status as the C function; pointers are integers."""
    return library().fa2_bwd(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, B, H, N, d, scale, int(is_causal),
                             int(dtype), stream)


def fa2_bwd_masked(Q: int, K: int, V: int, O: int, dO: int, LSE: int, dQ: int, dK: int, dV: int, workspace: int,
                   B: int, H: int, N: int, d: int, scale: float, window_left: int, window_right: int,
                   key_lens: int | None, dtype: int, stream: int) -> int:
    """Same arguments and status as the C function; pointers are integers (key_lens may be None)."""
    return library().fa2_bwd_masked(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, B, H, N, d, scale,
                                    int(window_left), int(window_right), key_lens, int(dtype), stream)


def fa2_bwd_noalloc(Q: int, K: int, V: int, O: int, dO: int, LSE: int, dQ: int, dK: int, dV: int,
                    B: int, H: int, N: int, d: int, scale: float, is_causal: int, dtype: int, stream: int) -> int:
    """Same arguments and status as the C function; pointers are integers."""
    return library().fa2_bwd_noalloc(Q, K, V, O, dO, LSE, dQ, dK, dV, B, H, N, d, scale, int(is_causal),
                                     int(dtype), stream)


def fa2_status_string(status: int) -> str:
    return library().fa2_status_string(int(status)).decode()


def fa2_launch_info(B: int, H: int, N: int, d: int, is_causal: int, dtype: int) -> dict:
    wg = ctypes.c_int64()
    th, rows, keys, lds = ctypes.c_int(), ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    st = library().fa2_launch_info(B, H, N, d, int(is_causal), int(dtype), ctypes.byref(wg),
                                   ctypes.byref(th), ctypes.byref(rows), ctypes.byref(keys),
                                   ctypes.byref(lds))
    if st != FA2_OK:
        raise Fa2Error(st, "fa2_launch_info")
    return {"workgroups": wg.value, "threads": th.value, "rows_per_wg": rows.value,
            "keys_per_tile": keys.value, "lds_bytes": lds.value}
