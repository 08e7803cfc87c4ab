"""ctypes access to the C replay of the oracle's EXP and LOG (oracle/explog.c, built by
oracle/build.py).  TEST INFRASTRUCTURE: only tests/ use it.  The constants passed in are
the Python oracle's (oracle.logsoftmax.K), so both replays share one derivation."""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .logsoftmax import K

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def _consts() -> np.ndarray:
    return np.asarray([K["LOG2E"], K["LN2_HI"], K["LN2_LO"], *K["EXP_C"], K["SQRT2"], *K["LOG_B"]],
                      dtype=np.float32)


def _lib():
    global _LIB
    if _LIB is None:
        path = os.path.join(HERE, "libexplog.so")
        if not os.path.exists(path):
            from .build import build
            build()
        lib = ctypes.CDLL(path)
        P, I64, U32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32
        for name in ("oracle_exp_bits", "oracle_log_bits"):
            getattr(lib, name).argtypes = [U32, I64, P, P]
        for name in ("oracle_exp", "oracle_log"):
            getattr(lib, name).argtypes = [P, I64, P, P]
        _LIB = lib
    return _LIB


_K = None


def _k():
    global _K
    if _K is None:
        _K = _consts()
    return _K


def _bits_call(name, first: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    getattr(_lib(), name)(ctypes.c_uint32(first), n, _k().ctypes.data, out.ctypes.data)
    return out


def _vals_call(name, x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty_like(x)
    getattr(_lib(), name)(x.ctypes.data, x.size, _k().ctypes.data, out.ctypes.data)
    return out


def exp_bits(first: int, n: int) -> np.ndarray:
    """EXP of the n floats whose bit patterns are first, first + 1, ..."""
    return _bits_call("oracle_exp_bits", first, n)


def log_bits(first: int, n: int) -> np.ndarray:
    return _bits_call("oracle_log_bits", first, n)


def EXP(x) -> np.ndarray:
    return _vals_call("oracle_exp", x)


def LOG(x) -> np.ndarray:
    return _vals_call("oracle_log", x)
