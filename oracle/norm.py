"""Row normalization (LayerNorm, RMSNorm) followed by per-row dynamic
quantization, as one fused step.

Test infrastructure only (see the package docstring).

Definition followed: 《推理优化与量化算子深度技术调研》 section 4.4 (LayerNorm +
quantization fusion).  Per row: mean and variance, the normalized value
(x - mean) / sqrt(var + eps) * gamma + beta, then the row's absmax scale and
the codes, written once instead of writing the normalized activations and
reading them back.  The same section names RMSNorm + quantization as an
equally valid variant; RMSNorm here is x / sqrt(mean(x^2) + eps) * gamma.

Readings where the section's sketch is loose or silent (each also listed in
the design notes):

* The variance is the biased one (divide by K), as in the layer norm the
  sketch's unfused path calls: the fused step must equal that path followed
  by quantization.  (The sketch's ``x.var`` would be the unbiased estimator.)
* Precision.  The row statistics (sum of x and of (x - mean)^2, or sum of
  x^2) are accumulated in float64; mean and r = 1 / sqrt(var + eps) are
  computed in float64 and rounded once to float32.  The normalized value is
  then formed in float32, one rounding per operation and no fused
  multiply-add: t = x - mean, u = t * r, y = u * gamma, y = y + beta
  (LayerNorm); u = x * r, y = u * gamma (RMSNorm).  Float64 statistics make
  the float32 mean and r independent of the summation order except when a
  float64 result lies within a few float64 units of a float32 rounding
  boundary.
* The quantization is the per-row dynamic quantization of the activations
  (fp8.quantize_rows; intquant.quantize_sym / quantize_asym with one group
  per row): round half to even, then clip.  The sketch's ``.to(torch.int8)``
  truncation is not used: it would disagree with the unfused path's
  quantizer.
* eps is given as a float32 value and widened exactly to float64.
* MXFP4 output (the same section's fusion applied to the block-scaled
  format of 《大模型量化推理引擎全景大复盘》 section 2, eq. 3): the normalized
  float32 row goes through the MX quantizer of this package unchanged, 32
  elements along K per E8M0 exponent; there is then no per-row scale, the
  per-block exponents take its place.
"""
from __future__ import annotations

import numpy as np

from . import fp8, intquant, mx

KINDS = ("layer", "rms")
FORMATS = ("fp8_e4m3", "int8_sym", "int8_asym", "mxfp4")


def row_stats(x, kind: str, eps: float):
    """Float32 mean (zero for RMSNorm) and reciprocal root r of each row of
    x [rows][K] (float32 values), from float64 sums."""
    if kind not in KINDS:
        raise ValueError(f"unknown normalization {kind!r}")
    x64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    if x64.ndim != 2 or x64.shape[1] == 0:
        raise ValueError("invalid quantization geometry")
    k = x64.shape[1]
    e64 = float(np.float32(eps))
    if kind == "layer":
        mean = x64.sum(axis=1) / k
        var = ((x64 - mean[:, None]) ** 2).sum(axis=1) / k
        r = 1.0 / np.sqrt(var + e64)
        return mean.astype(np.float32), r.astype(np.float32)
    ms = (x64 * x64).sum(axis=1) / k
    r = 1.0 / np.sqrt(ms + e64)
    return np.zeros(x64.shape[0], np.float32), r.astype(np.float32)


def normalize(x, gamma, beta, kind: str, eps: float) -> np.ndarray:
    """The normalized rows y [rows][K] in float32 (readings above)."""
    x = np.asarray(x, dtype=np.float32)
    g = np.asarray(gamma, dtype=np.float32).reshape(-1)
    mean, r = row_stats(x, kind, eps)
    if g.shape[0] != x.shape[1]:
        raise ValueError("invalid quantization geometry")
    if kind == "layer":
        b = np.asarray(beta, dtype=np.float32).reshape(-1)
        t = (x - mean[:, None]).astype(np.float32)
        u = (t * r[:, None]).astype(np.float32)
        y = (u * g[None, :]).astype(np.float32)
        return (y + b[None, :]).astype(np.float32)
    u = (x * r[:, None]).astype(np.float32)
    return (u * g[None, :]).astype(np.float32)


def norm_quant(x, gamma, beta, kind: str, fmt: str, eps: float):
    """Normalize, then quantize per row.  Returns (codes [rows][K], scales
    float32 [rows], zeros float32 [rows] or None); for "mxfp4" (codes uint8
    [rows][K/2], E8M0 exponents uint8 [rows][K/32], None)."""
    if fmt not in FORMATS:
        raise ValueError(f"unknown format {fmt!r}")
    y = normalize(x, gamma, beta, kind, eps)
    k = y.shape[1]
    if fmt == "mxfp4":
        codes, e8m0 = mx.quantize(y)
        return codes, e8m0, None
    if fmt == "fp8_e4m3":
        codes, s = fp8.quantize_rows(y)
        return codes, np.asarray(s, np.float32).reshape(-1), None
    if fmt == "int8_sym":
        q, s = intquant.quantize_sym(y, k, "int8_sym")
        return q.astype(np.int8), np.asarray(s, np.float32).reshape(-1), None
    q, s, z = intquant.quantize_asym(y, k, "int8_asym")
    return (q.astype(np.uint8), np.asarray(s, np.float32).reshape(-1),
            np.asarray(z, np.float32).reshape(-1))
