"""Group-wise integer quantization, nibble packing and dequantization.

Test infrastructure only (see the package docstring).

Definitions followed:

* Symmetric: scale = max|x| / q_max, q = clip(round(x / scale), lo, hi),
  x_hat = q * scale.  《推理优化与量化算子深度技术调研》 section 1.2 (INT8,
  max|x|/127, clamp to +-127); 《第 6 课：量化源码走读》 worked example and
  practice exercise (scale = max_abs / q_max, a zero block uses scale 1).
  The INT4 range [-8, 7] is the format table of 《量化与加速》.
* Asymmetric: scale = (x_max - x_min) / (2^b - 1), z = round(-x_min / scale),
  q = clip(round(x / scale) + z, 0, 2^b - 1), x_hat = scale * (q - z).
  《量化与加速》 "INT8 量化原理" equations; 《推理优化与量化算子深度技术调研》
  section 1.2 code; 《第 1 章：推理加速全景》 section 4.1.

Readings where the pages are silent (each also listed in the design notes):

* round() is round-half-to-even (the pages' code only uses half-even
  rounding functions).
* Quantization decides integers in the kernel's precision: the scale is
  computed in fp32, rounded to its storage dtype first, and x is divided by
  the stored value with one IEEE fp32 division.  ``scale_dtype="f64"`` instead
  runs the same steps in float64 (the pages' Python exercise).
* Order is round, then add z, then clip (the affine equation of 《量化与加速》).
* A zero (or underflowed) scale becomes 1 (the exercise's zero-block rule).
* fp16 storage saturates at +-65504 instead of overflowing to infinity.
* The zero point is not clamped; it is stored in the scale's dtype.
* INT4 packing: element k = 8j + i sits in bits 4i..4i+3 of int32 word j of
  its row (LSB first), as the two's-complement nibble for signed codes.  The
  lesson's registry section says eight INT4 values are packed per int32; the
  order within the word is this reading.
"""

from __future__ import annotations

import numpy as np

from .formats import round_to_fp16_saturating

INT_RANGES = {
    # (lo, hi) code ranges
    "int4_sym": (-8, 7),
    "int4_asym": (0, 15),
    "int8_sym": (-127, 127),
    "int8_asym": (0, 255),
}
Q_MAX = {"int4_sym": 7, "int8_sym": 127}
LEVELS = {"int4_asym": 15, "int8_asym": 255}
SCALE_DTYPE = {"int4_sym": "f16", "int4_asym": "f16", "int8_sym": "f32", "int8_asym": "f32"}


def _store_scale(v: np.ndarray, scale_dtype: str) -> np.ndarray:
    """Round computed scales to their storage dtype; return them in the
    arithmetic dtype used for the following division (fp32 or fp64)."""
    if scale_dtype == "f16":
        return round_to_fp16_saturating(v).astype(np.float32)
    if scale_dtype == "f32":
        return np.asarray(v, dtype=np.float32)
    if scale_dtype == "f64":
        return np.asarray(v, dtype=np.float64)
    raise ValueError(scale_dtype)


def _groups(x: np.ndarray, group: int) -> np.ndarray:
    rows, k = x.shape
    if group <= 0 or k % group != 0:
        raise ValueError("invalid quantization geometry")
    return x.reshape(rows, k // group, group)


def quantize_sym(x, group: int, fmt: str = "int4_sym", scale_dtype: str | None = None,
                 qmax: int | None = None):
    """Symmetric group quantization of a [rows][K] array along K.

    Returns (codes int32 [rows][K], scales [rows][K/group] in the storage
    dtype: float16, float32 or float64).  ``qmax`` overrides the format with
    the range [-qmax, qmax] (the exercise's generic form).
    """
    scale_dtype = scale_dtype or SCALE_DTYPE[fmt]
    ar = np.float64 if scale_dtype == "f64" else np.float32
    x = np.asarray(x, dtype=ar)
    if x.ndim != 2:
        raise ValueError("invalid quantization geometry")
    lo, hi = INT_RANGES[fmt]
    q_max = Q_MAX[fmt]
    if qmax is not None:
        lo, hi, q_max = -qmax, qmax, qmax
    g = _groups(x, group)
    amax = np.max(np.abs(g), axis=2)                       # exact
    s = _store_scale(amax / ar(q_max), scale_dtype)        # divide, then store
    s = np.where(s == 0, ar(1.0), s).astype(ar)            # zero block -> 1
    q = np.rint(g / s[:, :, None])                         # one IEEE division, RNE
    q = np.clip(q, lo, hi).astype(np.int32)
    out_dtype = {"f16": np.float16, "f32": np.float32, "f64": np.float64}[scale_dtype]
    return q.reshape(x.shape), s.astype(out_dtype)


def quantize_asym(x, group: int, fmt: str = "int4_asym", scale_dtype: str | None = None):
    """Asymmetric group quantization of a [rows][K] array along K.

    Returns (codes int32 [rows][K], scales, zeros), scales and zeros in the
    storage dtype (zeros hold integer values).
    """
    scale_dtype = scale_dtype or SCALE_DTYPE[fmt]
    ar = np.float64 if scale_dtype == "f64" else np.float32
    x = np.asarray(x, dtype=ar)
    if x.ndim != 2:
        raise ValueError("invalid quantization geometry")
    lo_c, hi_c = INT_RANGES[fmt]
    levels = LEVELS[fmt]
    g = _groups(x, group)
    x_min = np.min(g, axis=2)
    x_max = np.max(g, axis=2)
    s = _store_scale((x_max - x_min) / ar(levels), scale_dtype)
    s = np.where(s == 0, ar(1.0), s).astype(ar)
    z = _store_scale(np.rint(-x_min / s), scale_dtype).astype(ar)
    q = np.rint(g / s[:, :, None]) + z[:, :, None]         # round, then add z
    q = np.clip(q, lo_c, hi_c).astype(np.int32)            # then clip
    out_dtype = {"f16": np.float16, "f32": np.float32, "f64": np.float64}[scale_dtype]
    return q.reshape(x.shape), s.astype(out_dtype), z.astype(out_dtype)


def dequantize(q, scales, zeros, group: int, out: str = "f64") -> np.ndarray:
    """x_hat = s * (q - z) per group (《量化与加速》 "INT8 量化原理").

    ``out="f64"`` returns the exact value (the product of a <= 24-bit scale and
    a small integer is exact in float64); ``out="f32"`` rounds that exact value
    once to fp32, which is what one fp32 multiply of the stored operands gives.
    """
    q = np.asarray(q, dtype=np.float64)
    rows, k = q.shape
    s = np.repeat(np.asarray(scales, dtype=np.float64), group, axis=1)
    z = 0.0 if zeros is None else np.repeat(np.asarray(zeros, dtype=np.float64), group, axis=1)
    v = s * (q - z)
    if out == "f64":
        return v
    if out == "f32":
        return v.astype(np.float32)
    raise ValueError(out)


# ----------------------------------------------------------------------------
# nibble packing


def pack_int4(q) -> np.ndarray:
    """Pack int4 codes [rows][K] (K % 8 == 0) into int32 words [rows][K/8]:
    element 8j+i -> bits 4i..4i+3 of word j; the nibble is q & 0xF."""
    q = np.asarray(q, dtype=np.int64)
    rows, k = q.shape
    if k % 8 != 0:
        raise ValueError("invalid quantization geometry")
    nib = (q & 0xF).reshape(rows, k // 8, 8)
    word = np.zeros((rows, k // 8), dtype=np.int64)
    for i in range(8):
        word |= nib[:, :, i] << (4 * i)
    return word.astype(np.uint32).view(np.int32)


def unpack_int4(words, signed: bool) -> np.ndarray:
    """Inverse of pack_int4: int32 words [rows][K/8] -> codes int32 [rows][K]."""
    w = np.asarray(words).view(np.uint32).astype(np.int64)
    rows, kw = w.shape
    out = np.zeros((rows, kw, 8), dtype=np.int64)
    for i in range(8):
        nib = (w >> (4 * i)) & 0xF
        if signed:
            nib = np.where(nib >= 8, nib - 16, nib)
        out[:, :, i] = nib
    return out.reshape(rows, kw * 8).astype(np.int32)


# ----------------------------------------------------------------------------
# the lesson's practice exercise, as a plain function of the same behaviour


def blockwise_symmetric_fake_quant(values, block_size, qmax):
    """Symmetric per-block fake quantization in Python floats, with the
    behaviour the practice exercise of 《第 6 课：量化源码走读》 specifies:
    consecutive blocks of ``block_size`` (the last may be shorter), scale
    max|x| / qmax (1 for an all-zero block), codes clipped to [-qmax, qmax],
    values restored as q * scale; a non-positive block size or qmax raises
    ValueError("invalid quantization geometry").  Returns (restored, scales).
    Built on ``quantize_sym`` in float64 mode."""
    if block_size <= 0 or qmax <= 0:
        raise ValueError("invalid quantization geometry")
    x = np.asarray(values, dtype=np.float64)
    restored, scales = [], []
    for b in range(0, len(x), block_size):
        blk = x[b:b + block_size]
        q, s = quantize_sym(blk[None, :], len(blk), scale_dtype="f64", qmax=qmax)
        scales.append(float(s[0, 0]))
        restored.extend(float(v) * float(s[0, 0]) for v in q[0])
    return restored, scales
