"""SmoothQuant per-channel smoothing: channel statistics, the smoothing
factors, and quantization of the smoothed operands.

Test infrastructure only (see the package docstring).

Definitions followed: 《第 1 章：推理加速全景：从计算瓶颈到多路突围》 section 4.3
(the equivalence X W = (X diag(s)^-1)(diag(s) W), and the factor
s_j = max|X_j|^alpha / max|W_j|^(1-alpha) with X_j the calibration
activations of input channel j and W_j the weights that multiply it, alpha in
[0, 1]); 《推理优化与量化算子深度技术调研》 section 1.5 (the same factor,
X_hat = X / s and W_hat = W * s, the factor folded into the weights offline so
that inference only quantizes activations).

Readings (each also listed in the design notes):

* Layout: weights are stored [N][K], one row per output channel, so the
  weights that multiply input channel j form column j and W_hat = W diag(s)
  scales columns; activations X [M][K] have X_hat = X diag(s)^-1, column j
  divided by s_j.
* Channel statistic: the maximum of |x| over the rows (exact).  Calibration
  over several batches keeps the running maximum.
* The factor is evaluated in float64 from the float32 statistics and alpha (a
  float32 value widened exactly), a^alpha / w^(1 - alpha), and rounded once to
  float32.  A channel whose statistic is zero on either side, or whose factor
  is not a positive normal float32, gets s_j = 1 (no migration), as a zero
  block gets scale 1 in the quantizers.
* Folding: w_hat = fl32(w * s_j), x_hat = fl32(x / s_j), one float32 rounding
  each (inputs are float32, or bf16 widened exactly), then the unchanged
  group quantizers of ``intquant`` and ``fp8``.
"""
from __future__ import annotations

import numpy as np

from . import fp8, intquant

FORMATS = ("int4_sym", "int4_asym", "int8_sym", "int8_asym", "fp8_e4m3")
F32_TINY = float(np.finfo(np.float32).tiny)
F32_MAX = float(np.finfo(np.float32).max)


def channel_absmax(x, running=None) -> np.ndarray:
    """max over rows of |x| per column of x [rows][K] (float32), combined with
    a previous running maximum when given."""
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 2 or x.shape[0] == 0 or x.shape[1] == 0:
        raise ValueError("invalid quantization geometry")
    m = np.max(np.abs(x), axis=0)
    if running is not None:
        m = np.maximum(np.asarray(running, dtype=np.float32), m)
    return m.astype(np.float32)


def smooth_scales(act_max, w_max, alpha: float) -> np.ndarray:
    """s_j = act_max_j^alpha / w_max_j^(1 - alpha), float64, rounded once to
    float32; 1 where either statistic is zero or the result is not a positive
    normal float32."""
    a = np.asarray(act_max, dtype=np.float32).astype(np.float64)
    w = np.asarray(w_max, dtype=np.float32).astype(np.float64)
    if a.shape != w.shape or a.ndim != 1:
        raise ValueError("invalid quantization geometry")
    al = float(np.float32(alpha))
    if not 0.0 <= al <= 1.0:
        raise ValueError("alpha must lie in [0, 1]")
    s = np.ones_like(a)
    ok = (a > 0) & (w > 0)
    with np.errstate(over="ignore", under="ignore", divide="ignore"):
        s[ok] = np.power(a[ok], al) / np.power(w[ok], 1.0 - al)
    with np.errstate(over="ignore"):
        s32 = s.astype(np.float32)
    good = ok & (s32 >= np.float32(F32_TINY)) & (s32 <= np.float32(F32_MAX))
    return np.where(good, s32, np.float32(1.0)).astype(np.float32)


def fold(x, s, divide: bool) -> np.ndarray:
    """x [rows][K] with column j multiplied (weights) or divided
    (activations) by s_j, one float32 rounding."""
    x = np.asarray(x, dtype=np.float32)
    s = np.asarray(s, dtype=np.float32).reshape(-1)
    if x.ndim != 2 or s.shape[0] != x.shape[1]:
        raise ValueError("invalid quantization geometry")
    with np.errstate(over="ignore"):
        y = x / s[None, :] if divide else x * s[None, :]
    return y.astype(np.float32)


def quantize(x, fmt: str, group: int):
    """The group quantizer of the library's storage formats on x [rows][K]:
    (codes, scales [rows][K/group], zeros or None); INT4 codes packed."""
    x = np.asarray(x, dtype=np.float32)
    rows, k = x.shape
    if fmt == "int4_sym":
        q, s = intquant.quantize_sym(x, group, "int4_sym")
        return intquant.pack_int4(q), s, None
    if fmt == "int4_asym":
        q, s, z = intquant.quantize_asym(x, group, "int4_asym")
        return intquant.pack_int4(q), s, z
    if fmt == "int8_sym":
        q, s = intquant.quantize_sym(x, group, "int8_sym")
        return q.astype(np.int8), s, None
    if fmt == "int8_asym":
        q, s, z = intquant.quantize_asym(x, group, "int8_asym")
        return q.astype(np.uint8), s, z
    if fmt == "fp8_e4m3":
        if group <= 0 or k % group:
            raise ValueError("invalid quantization geometry")
        codes, s = fp8.quantize_rows(x.reshape(rows * (k // group), group))
        return codes.reshape(rows, k), np.asarray(s).reshape(rows, k // group), None
    raise ValueError(f"unknown format {fmt!r}")


def smooth_quantize(x, s, divide: bool, fmt: str, group: int):
    """Quantize the smoothed operand fold(x, s, divide) with the format's
    group quantizer."""
    return quantize(fold(x, s, divide), fmt, group)
