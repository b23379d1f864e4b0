"""OCP MXFP4 quantization: 32-element blocks along K share one E8M0 exponent,
elements are FP4 E2M1 codes.

Test infrastructure only (see the package docstring).

Definitions followed: 《大模型量化推理引擎全景大复盘》 section 2, equation 3
(32 four-bit elements share one E8M0 exponent) and section 3 code (shared
scale 2^ceil(log2(max|x| / 6))); 《第 6 课：量化源码走读》 section 2 (micro-block
scaling, outliers confined to their block) and section 3 (K must be a
multiple of the block size).

Readings:

* The exponent is the smallest integer e with max|x| <= 6 * 2^e, which is
  what ceil(log2(max/6)) means, decided exactly instead of through a
  floating-point log.  It is clamped to [-127, 127]; the stored byte is
  e + 127.  An all-zero block gets e = 0 (the exercise's zero-block rule;
  any e gives the same all-zero codes).
* Each element is divided by 2^e (exact) and encoded to the nearest E2M1
  value, ties to the even code, saturating at 6; the sign is kept.
* Two codes per byte along K: element 2j in the low nibble of byte j.
"""

from __future__ import annotations

import math

import numpy as np

from .formats import decode, encode

BLOCK = 32
E2M1_MAX = 6.0


def shared_exponent(m: float) -> int:
    """Smallest integer e such that m <= 6 * 2^e (m > 0), clamped to
    [-127, 127]; 0 for m == 0.  Start from a floating-point estimate and step
    until the defining inequalities hold exactly (6 * 2^e is exact in fp64)."""
    m = float(m)
    if m == 0.0:
        return 0
    e = math.ceil(math.log2(m / E2M1_MAX))
    while m > E2M1_MAX * 2.0 ** e:
        e += 1
    while m <= E2M1_MAX * 2.0 ** (e - 1):
        e -= 1
    return max(-127, min(127, e))


def quantize(x):
    """x: [rows][K], K % 32 == 0 (fp32 or bf16 widened to fp32).
    Returns (packed uint8 [rows][K/2], e8m0 uint8 [rows][K/32])."""
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 2 or x.shape[1] % BLOCK != 0 or x.shape[1] == 0:
        raise ValueError("invalid quantization geometry")
    rows, k = x.shape
    nb = k // BLOCK
    blocks = x.reshape(rows, nb, BLOCK).astype(np.float64)
    amax = np.max(np.abs(blocks), axis=2)
    e = np.vectorize(shared_exponent, otypes=[np.int64])(amax) if amax.size else \
        np.zeros_like(amax, dtype=np.int64)
    v = blocks / np.exp2(e.astype(np.float64))[:, :, None]      # exact power-of-two scaling
    codes = encode(v, "e2m1").astype(np.uint8).reshape(rows, k)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, (e + 127).astype(np.uint8)


def unpack_codes(packed) -> np.ndarray:
    """uint8 [rows][K/2] -> E2M1 codes uint8 [rows][K]."""
    p = np.asarray(packed, dtype=np.uint8)
    rows, kh = p.shape
    out = np.empty((rows, 2 * kh), dtype=np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


def dequantize(packed, e8m0) -> np.ndarray:
    """x_hat = 2^(byte - 127) * e2m1(code), exact, float64 [rows][K]."""
    codes = unpack_codes(packed)
    rows, k = codes.shape
    e = np.asarray(e8m0, dtype=np.float64) - 127.0
    scale = np.repeat(np.exp2(e), BLOCK, axis=1)
    return decode(codes, "e2m1") * scale
