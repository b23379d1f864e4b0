"""Quantized linear layer for AMD Instinct MI355X (gfx950).

Eight operations, each one call into the HIP library libqgemm.so (C ABI in
include/qgemm.h): ``quantize_pack``, ``dequant``, ``qgemv``, ``qgemm``,
``mx_quant``, ``mx_gemm``, and two fused steps: ``norm_quant`` (row
normalization + per-row dynamic quantization) and ``qgemm_swiglu`` (the gate
and up projections of a SwiGLU FFN in one W4A16 GEMM with SiLU(gate) * up in
its epilogue).  The library is the only implementation: importing
works without it, but every operation raises if it is missing.
"""

from .api import (dequant, mx_gemm, mx_quant, norm_quant, qgemm, qgemm_swiglu, qgemv,  # noqa: F401
                  quantize_pack, default_group)
from ._lib import LIB_PATH, QGError, load as load_library  # noqa: F401

__all__ = ["quantize_pack", "dequant", "qgemv", "qgemm", "mx_quant", "mx_gemm", "norm_quant",
           "qgemm_swiglu",
           "load_library", "LIB_PATH", "QGError", "default_group"]
