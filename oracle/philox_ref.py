"""Loader for the C Philox cross-check (oracle side, test infrastructure only)."""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "philox_ref.c")
_LIB = os.path.join(_HERE, "libphilox_ref.so")


def build(force: bool = False) -> str:
    """Compile philox_ref.c with gcc into oracle/libphilox_ref.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-shared", "-fPIC", "-o", tmp, _SRC])
        os.replace(tmp, _LIB)
    return _LIB


def batch(ctr: np.ndarray, k0: int, k1: int) -> np.ndarray:
    """ctr uint32 [n, 4] -> uint32 [n, 4] outputs."""
    lib = ctypes.CDLL(build())
    ctr = np.ascontiguousarray(ctr, dtype=np.uint32)
    out = np.empty_like(ctr)
    lib.philox4x32_10_batch(ctr.ctypes.data_as(ctypes.c_void_p), ctypes.c_size_t(ctr.shape[0]),
                            ctypes.c_uint32(k0), ctypes.c_uint32(k1),
                            out.ctypes.data_as(ctypes.c_void_p))
    return out
