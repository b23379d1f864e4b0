"""Per-row FP8 E4M3 quantization (weights per output channel, activations per
token, dynamically at run time).

Test infrastructure only (see the package docstring).

Definitions followed: 《第 6 课：量化源码走读》 section 2 (W8A8/FP8 paradigm:
activations are quantized on line just before the GEMM with a scale s_x
derived from the tensor's absolute maximum, the codes clipped to
[-q_max, q_max]; the GEMM output is rescaled by scale_x * scale_w, figure 6-2);
《推理优化与量化算子深度技术调研》 section 1.4 (E4M3 for forward activations and
weights, an fp32 scale tensor beside the codes); 《量化与加速》 format table
(E4M3 range +-448, so q_max = 448).

Readings: the scale is absmax / 448 computed in fp32 (one IEEE division) per
row; an all-zero row uses scale 1; the code is the saturating,
ties-to-even nearest E4M3 value of x / s (one IEEE fp32 division).
"""

from __future__ import annotations

import numpy as np

from .formats import decode, encode

E4M3_MAX = 448.0


def quantize_rows(x):
    """x: [rows][K] values (fp32 or bf16 widened to fp32).
    Returns (codes uint8 [rows][K], scales float32 [rows])."""
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 2 or x.shape[1] == 0:
        raise ValueError("invalid quantization geometry")
    amax = np.max(np.abs(x), axis=1)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    s = np.where(s == 0, np.float32(1.0), s).astype(np.float32)
    v = (x / s[:, None]).astype(np.float32)
    return encode(v, "e4m3"), s


def dequantize_rows(codes, scales) -> np.ndarray:
    """x_hat = s * dec(code), exact, float64."""
    return decode(codes, "e4m3") * np.asarray(scales, dtype=np.float64)[:, None]
