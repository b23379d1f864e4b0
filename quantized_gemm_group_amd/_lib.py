"""ctypes loader of libqgemm.so and the C ABI prototypes (include/qgemm.h).

The library is loaded from this package directory only; there is no other
implementation to fall back to, so a missing or stale build raises.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqgemm.so")

# qg_format
INT4_SYM, INT4_ASYM, INT8_SYM, INT8_ASYM, FP8_E4M3, BF16_ACT, MXFP4 = range(7)
# qg_dtype
BF16, F32 = 0, 1
# qg_norm
NORM_LAYER, NORM_RMS = 0, 1
# qg_calib_kind
CALIB_BF16, CALIB_FP8, CALIB_FP4, CALIB_INT8 = range(4)
# qg_status
OK, ERR_GEOMETRY, ERR_ALIGN, ERR_FORMAT, ERR_NULL, ERR_HIP, ERR_UNSUPPORTED = range(7)

EXPORTS = [
    "qg_quantize_pack", "qg_dequant", "qg_qgemv", "qg_qgemm", "qg_mx_quant", "qg_mx_gemm",
    "qg_norm_quant", "qg_qgemm_swiglu", "qg_quantize_pack_smooth", "qg_channel_absmax",
    "qg_smooth_scales", "qg_channel_scales", "qg_kv_cache_store", "qg_status_str",
    "qg_last_error", "qg_abi_version", "qg_calib_stream_read", "qg_calib_mfma",
    "qg_tile_gemv_weights", "qg_qgemv_tiled", "qg_qgemv_swiglu", "qg_qgemm_swiglu_fp8",
    "qg_debug_fp32_output", "qg_debug_build",
]

_lib = None


LIB_DEBUG_PATH = os.path.join(HERE, "libqgemm_debug.so")
_lib_debug = None


def load() -> ctypes.CDLL:
    """Load libqgemm.so (once) and declare its prototypes."""
    global _lib
    if _lib is None:
        _lib = _open(LIB_PATH)
    return _lib


def load_debug() -> ctypes.CDLL:
    """Load the debug library libqgemm_debug.so (once): the same entry points,
    plus fp32 output recording (qg_debug_fp32_output).  For tests and bug
    hunts; the binding in api.py always uses the product library."""
    global _lib_debug
    if _lib_debug is None:
        _lib_debug = _open(LIB_DEBUG_PATH)
    return _lib_debug


def _open(path: str) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m quantized_gemm_group_amd.build` "
            "(the HIP library is the only implementation)")
    lib = ctypes.CDLL(path)
    i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.qg_quantize_pack.argtypes = [i32, vp, i32, i64, i64, i64, vp, vp, vp, vp]
    lib.qg_dequant.argtypes = [i32, vp, vp, vp, i64, i64, i64, vp, i32, vp]
    lib.qg_qgemv.argtypes = [i32, vp, i64, vp, vp, vp, i64, i64, i64, vp, vp]
    lib.qg_qgemm.argtypes = [i32, i32, vp, vp, vp, i64, vp, vp, vp, i64, i64, i64, vp, vp]
    lib.qg_mx_quant.argtypes = [vp, i32, i64, i64, vp, vp, vp]
    lib.qg_mx_gemm.argtypes = [vp, vp, i64, vp, vp, i64, i64, vp, vp]
    lib.qg_norm_quant.argtypes = [i32, i32, vp, i32, vp, vp, ctypes.c_float, i64, i64, vp, vp,
                                  vp, vp]
    lib.qg_qgemm_swiglu.argtypes = [i32, i32, vp, i64, vp, vp, vp, i64, i64, i64, vp, vp]
    lib.qg_quantize_pack_smooth.argtypes = [i32, vp, i32, i64, i64, i64, vp, i32, vp, vp, vp, vp]
    lib.qg_channel_absmax.argtypes = [vp, i32, i64, i64, i32, vp, vp]
    lib.qg_smooth_scales.argtypes = [vp, vp, ctypes.c_float, i64, vp, vp]
    lib.qg_channel_scales.argtypes = [vp, i64, ctypes.c_float, vp, vp]
    lib.qg_kv_cache_store.argtypes = [vp, i32, i64, i64, i64, vp, i64, vp, vp, vp, vp]
    lib.qg_calib_stream_read.argtypes = [vp, i64, vp, vp]
    lib.qg_tile_gemv_weights.argtypes = [vp, i64, i64, vp, vp]
    lib.qg_qgemv_tiled.argtypes = [i32, vp, i64, vp, vp, vp, i64, i64, i64, vp, vp]
    lib.qg_qgemv_swiglu.argtypes = [i32, vp, i64, vp, vp, vp, i64, i64, i64, i32, vp, vp]
    lib.qg_qgemm_swiglu_fp8.argtypes = [vp, vp, i64, vp, vp, i64, i64, vp, vp]
    lib.qg_calib_mfma.argtypes = [i32, i64, i64, vp, vp]
    for name in ["qg_quantize_pack", "qg_dequant", "qg_qgemv", "qg_qgemm", "qg_mx_quant",
                 "qg_mx_gemm", "qg_norm_quant", "qg_qgemm_swiglu", "qg_quantize_pack_smooth",
                 "qg_channel_absmax", "qg_smooth_scales", "qg_channel_scales",
                 "qg_kv_cache_store", "qg_calib_stream_read", "qg_calib_mfma",
                 "qg_tile_gemv_weights", "qg_qgemv_tiled", "qg_qgemv_swiglu",
                 "qg_qgemm_swiglu_fp8"]:
        getattr(lib, name).restype = i32
    lib.qg_status_str.argtypes = [i32]
    lib.qg_status_str.restype = ctypes.c_char_p
    lib.qg_last_error.argtypes = []
    lib.qg_last_error.restype = ctypes.c_char_p
    lib.qg_abi_version.argtypes = []
    lib.qg_abi_version.restype = i32
    lib.qg_debug_fp32_output.argtypes = [vp, vp]
    lib.qg_debug_fp32_output.restype = i32
    lib.qg_debug_build.argtypes = []
    lib.qg_debug_build.restype = i32
    return lib


class QGError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(detail)


def check(status: int) -> None:
    """Raise on a non-OK status: ValueError for invalid geometry (the
    convention of the lesson's exercise), QGError otherwise."""
    if status == OK:
        return
    lib = load()
    name = lib.qg_status_str(status).decode()
    detail = lib.qg_last_error().decode()
    if status == ERR_GEOMETRY:
        raise ValueError(f"invalid quantization geometry: {detail}")
    raise QGError(status, f"{name}: {detail}")
