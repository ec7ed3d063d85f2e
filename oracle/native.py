"""TEST INFRASTRUCTURE ONLY: builds and loads the oracle's C attention.

The library is compiled with the system C compiler from ``attn_ref.c`` in this
directory; nothing here is shared with the GPU library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_ref.c")
# ORACLE_ATTN_LIBRARY names a prebuilt copy instead (the sanitizer run builds
# one with AddressSanitizer and UBSan and runs the oracle's pins on it)
_LIB = os.environ.get("ORACLE_ATTN_LIBRARY") or os.path.join(_HERE, "liboracle_attn.so")
_SAN_LIB = os.path.join(_HERE, "_san", "liboracle_attn.so")
_lib = None


def build(force: bool = False) -> str:
    if os.environ.get("ORACLE_ATTN_LIBRARY"):
        return _LIB
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def build_sanitized() -> str:
    """The same C reference built with AddressSanitizer and UBSan (host only),
    for a run of the oracle's pins under the gcc sanitizer runtime."""
    os.makedirs(os.path.dirname(_SAN_LIB), exist_ok=True)
    tmp = _SAN_LIB + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-pthread",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                           "-fno-omit-frame-pointer", "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _SAN_LIB)
    return _SAN_LIB


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        L.oracle_attend_batch.restype = ctypes.c_int
        L.oracle_attend_batch.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_double, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int]
        _lib = L
    return _lib


def attend_batch(n_heads: int, d_qk: int, v_off: int, d_v: int, row_elems: int, scale: float,
                 q_ptrs: np.ndarray, row_begin: np.ndarray, row_ptrs: np.ndarray,
                 n_threads: int = 1) -> np.ndarray:
    """Calls the C reference; pointer arrays are uint64 addresses of bf16 data
    that the caller keeps alive for the duration of the call."""
    q_ptrs = np.ascontiguousarray(q_ptrs, dtype=np.uint64)
    row_begin = np.ascontiguousarray(row_begin, dtype=np.int64)
    row_ptrs = np.ascontiguousarray(row_ptrs, dtype=np.uint64)
    n_q = q_ptrs.size
    out = np.zeros((n_q, n_heads, d_v), dtype=np.float64)
    if n_q == 0:
        return out
    rc = lib().oracle_attend_batch(n_q, n_heads, d_qk, v_off, d_v, row_elems, float(scale),
                                   q_ptrs.ctypes.data, row_begin.ctypes.data,
                                   row_ptrs.ctypes.data if row_ptrs.size else None,
                                   out.ctypes.data, int(n_threads))
    if rc != 0:
        raise RuntimeError("oracle_attend_batch failed (%d)" % rc)
    return out
