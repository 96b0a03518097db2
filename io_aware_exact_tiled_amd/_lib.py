"""ctypes view of libfa.so (the C ABI declared in include/fa.h).

Argument marshalling only.  If the library is missing this module raises:
there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfa.so")

FA_F32, FA_F16, FA_BF16 = 0, 1, 2
FA_FLAG_RECORD_TILES = 1 << 0
FA_FLAG_REVERSE_KV = 1 << 1
FA_BWD_SCRATCH_BYTES = 16 << 20   # the static scratch of fa_bwd_noalloc

STATUS = {
    0: "FA_OK", -1: "FA_ERR_NULL", -2: "FA_ERR_SHAPE", -3: "FA_ERR_HEAD_DIM", -4: "FA_ERR_DTYPE",
    -5: "FA_ERR_DROPOUT", -6: "FA_ERR_SCALE", -7: "FA_ERR_ALIGN", -8: "FA_ERR_WORKSPACE",
    -9: "FA_ERR_HIP", -10: "FA_ERR_OPTS", -11: "FA_ERR_SCRATCH",
}

# every symbol include/fa.h declares
EXPORTS = ("fa_fwd", "fa_fwd_workspace_bytes", "fa_bwd", "fa_bwd_workspace_bytes", "fa_bwd_noalloc", "fa_decode",
           "fa_decode_workspace_bytes", "fa_fwd_kv_outer", "fa_fwd_kv_outer_workspace_bytes",
           "fa_dropout_keep_mask", "fa_tile_shape",
           "fa_status_string", "fa_last_hip_error", "fa_abi_version")


class FaOpts(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("o_fp32", ctypes.c_int32),
        ("key_lens", ctypes.c_void_p),
        ("rng_offset", ctypes.c_uint64),
        ("flags", ctypes.c_uint32),
        ("tile_visits", ctypes.c_void_p),
        ("tile_visits2", ctypes.c_void_p),
        ("main_begin", ctypes.c_void_p),
        ("main_end", ctypes.c_void_p),
        ("main_mid", ctypes.c_void_p),
        ("kv_heads", ctypes.c_int32),
    ]


class FaError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {STATUS.get(code, code)} ({lib().fa_status_string(code).decode()})"
                         + (f" [{lib().fa_last_hip_error().decode()}]" if code == -9 else ""))


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m io_aware_exact_tiled_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, u64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64, ctypes.c_float, ctypes.c_size_t
        L.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, f32, u64, vp,
                             ctypes.POINTER(FaOpts), vp, sz, vp]
        L.fa_fwd.restype = i32
        L.fa_fwd_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
        L.fa_fwd_workspace_bytes.restype = sz
        L.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, f32, u64,
                             vp, ctypes.POINTER(FaOpts), vp, sz, vp]
        L.fa_bwd.restype = i32
        L.fa_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, f32,
                                     u64, vp, ctypes.POINTER(FaOpts), vp]
        L.fa_bwd_noalloc.restype = i32
        L.fa_bwd_workspace_bytes.argtypes = [i32, i32, i32, i32]
        L.fa_bwd_workspace_bytes.restype = sz
        L.fa_decode.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, i32, vp, vp, vp, sz, vp]
        L.fa_decode.restype = i32
        L.fa_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
        L.fa_decode_workspace_bytes.restype = sz
        L.fa_fwd_kv_outer.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, i32, i32, vp, vp, sz,
                                      vp]
        L.fa_fwd_kv_outer.restype = i32
        L.fa_fwd_kv_outer_workspace_bytes.argtypes = [i32, i32, i32, i32]
        L.fa_fwd_kv_outer_workspace_bytes.restype = sz
        L.fa_dropout_keep_mask.argtypes = [u64, u64, f32, i32, i32, i32, vp, vp]
        L.fa_dropout_keep_mask.restype = i32
        L.fa_tile_shape.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(i32), ctypes.POINTER(i32)]
        L.fa_tile_shape.restype = i32
        L.fa_status_string.argtypes = [i32]
        L.fa_status_string.restype = ctypes.c_char_p
        L.fa_last_hip_error.argtypes = []
        L.fa_last_hip_error.restype = ctypes.c_char_p
        L.fa_abi_version.argtypes = []
        L.fa_abi_version.restype = i32
        _lib = L
    return _lib


def check(code: int, what: str) -> None:
    if code != 0:
        raise FaError(code, what)
