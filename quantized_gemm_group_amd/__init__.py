"""Quantized linear layer for AMD Instinct MI355X (gfx950).

Each operation is one call into the HIP library libqgemm.so (C ABI in
include/qgemm.h): ``quantize_pack``, ``dequant``, ``qgemv``, ``qgemm``,
``mx_quant``, ``mx_gemm``; two fused steps: ``norm_quant`` (row
normalization + per-row dynamic quantization) and ``qgemm_swiglu`` (the gate
and up projections of a SwiGLU FFN in one W4A16 GEMM with SiLU(gate) * up in
its epilogue); SmoothQuant smoothing: ``channel_absmax`` (calibration
statistics), ``smooth_scales`` and ``quantize_pack_smooth`` (the factors
folded into the quantizer); and the FP8 KV cache: ``channel_scales``
(static per-channel scales) and ``kv_cache_store`` (quantize new keys or
values into a paged cache).  The library is the only implementation: importing
works without it, but every operation raises if it is missing.
"""

from .api import (dequant, mx_gemm, mx_quant, norm_quant, qgemm, qgemm_swiglu, qgemv,  # noqa: F401
                  quantize_pack, default_group, quantize_pack_smooth, channel_absmax,
                  smooth_scales, channel_scales, kv_cache_store, calib_stream_read, calib_mfma,
                  CALIB_K, TiledCodes, tile_gemv_weights, qgemv_tiled, qgemv_swiglu,
                  qgemm_swiglu_fp8)
from ._lib import LIB_PATH, QGError, load as load_library  # noqa: F401

__all__ = ["quantize_pack", "dequant", "qgemv", "qgemm", "mx_quant", "mx_gemm", "norm_quant",
           "qgemm_swiglu", "quantize_pack_smooth", "channel_absmax", "smooth_scales",
           "channel_scales", "kv_cache_store",
           "load_library", "LIB_PATH", "QGError", "default_group"]
