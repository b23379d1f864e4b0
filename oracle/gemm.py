"""Reference products of the quantized linear layer and the error metric.

Test infrastructure only (see the package docstring).

Y = X * W^T with W stored [N][K] (row n = output channel) and X [M][K].  Every
reference is the float64 product of the exactly dequantized operands, so it
carries no rounding beyond fp64 summation:

* W4A16 (GEMV and prefill GEMM): X is bf16 (exact), W_hat = s * (q - z) per
  group.  《第 6 课：量化源码走读》 section 2 (W4A16: weights dequantized inside
  the GEMM, activations stay 16-bit) and section 3 (the asymmetric zero-point
  cross term must be kept).
* W8A8 (FP8 / INT8): X_hat = s_x * dec(xq) per token, W_hat = s_w * dec(wq)
  per output channel; figure 6-2 of the same lesson (Out = acc * scale_x *
  scale_w).
* MXFP4: both operands 2^e * e2m1(code) per 32-block.
* SwiGLU (《推理优化与量化算子深度技术调研》 section 4.6): the gate and up
  projections as one product over the concatenation [W_gate; W_up] (rows
  0 .. I - 1 gate, I .. 2I - 1 up), then h = SiLU(gate) * up with
  SiLU(g) = g / (1 + exp(-g)), all in float64.

``rel_fro`` is ||Y - Y_ref||_F / ||Y_ref||_F in float64.
"""

from __future__ import annotations

import numpy as np

from . import fp8 as _fp8
from . import intquant as _iq
from . import mx as _mx


def reference_product(a_hat, w_hat) -> np.ndarray:
    """float64(A_hat) @ float64(W_hat)^T (BLAS dgemm)."""
    return np.asarray(a_hat, dtype=np.float64) @ np.asarray(w_hat, dtype=np.float64).T


def brute_force_product(a, w) -> np.ndarray:
    """Pure-Python triple loop, for tiny shapes only."""
    a = [[float(v) for v in row] for row in np.asarray(a, dtype=np.float64)]
    w = [[float(v) for v in row] for row in np.asarray(w, dtype=np.float64)]
    m, k, n = len(a), len(a[0]) if a else 0, len(w)
    out = [[0.0] * n for _ in range(m)]
    for i in range(m):
        for j in range(n):
            acc = 0.0
            for t in range(k):
                acc += a[i][t] * w[j][t]
            out[i][j] = acc
    return np.array(out, dtype=np.float64).reshape(m, n)


def rel_fro(y, y_ref) -> float:
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    den = np.linalg.norm(y_ref)
    num = np.linalg.norm(y - y_ref)
    return float(num / den) if den > 0 else float(num)


# ----------------------------------------------------------------------------
# per-format references (operands in their stored forms)


def w4a16_reference(x, packed, scales, zeros, group: int, rows=None) -> np.ndarray:
    """x: [M][K] bf16 values (as fp32); packed int32 [N][K/8]; scales (and
    zeros for the asymmetric format) fp16 [N][K/group].  ``rows`` optionally
    selects output channels (columns of Y) to compute."""
    packed = np.asarray(packed)
    scales = np.asarray(scales)
    if rows is not None:
        packed, scales = packed[rows], scales[rows]
        zeros = None if zeros is None else np.asarray(zeros)[rows]
    q = _iq.unpack_int4(packed, signed=zeros is None)
    w_hat = _iq.dequantize(q, scales, zeros, group)
    return reference_product(x, w_hat)


def fp8_reference(xq, sx, wq, sw) -> np.ndarray:
    return reference_product(_fp8.dequantize_rows(xq, sx), _fp8.dequantize_rows(wq, sw))


def int8_reference(xq, sx, zx, wq, sw, zw) -> np.ndarray:
    """Per-row INT8 operands (group = K): x_hat = s_x (q_x - z_x), likewise W."""
    k = np.asarray(xq).shape[1]
    sx = np.asarray(sx).reshape(-1, 1)
    sw = np.asarray(sw).reshape(-1, 1)
    zx = None if zx is None else np.asarray(zx).reshape(-1, 1)
    zw = None if zw is None else np.asarray(zw).reshape(-1, 1)
    a_hat = _iq.dequantize(xq, sx, zx, k)
    w_hat = _iq.dequantize(wq, sw, zw, k)
    return reference_product(a_hat, w_hat)


def mx_reference(a_packed, a_e8m0, b_packed, b_e8m0) -> np.ndarray:
    return reference_product(_mx.dequantize(a_packed, a_e8m0), _mx.dequantize(b_packed, b_e8m0))


def silu(g) -> np.ndarray:
    """SiLU(g) = g * sigmoid(g) = g / (1 + exp(-g)), float64."""
    g = np.asarray(g, dtype=np.float64)
    return g / (1.0 + np.exp(-g))


def swiglu_reference(x, packed, scales, zeros, group: int, channels=None) -> np.ndarray:
    """h [M][I] = SiLU(x W_gate^T) * (x W_up^T) for the quantized [2I][K]
    concatenation [W_gate; W_up] (W4A16 operands as in w4a16_reference).
    ``channels`` optionally selects intermediate channels (columns of h)."""
    n2 = np.asarray(packed).shape[0]
    if n2 % 2:
        raise ValueError("invalid quantization geometry")
    i = n2 // 2
    ch = np.arange(i) if channels is None else np.asarray(channels)
    gate = w4a16_reference(x, packed, scales, zeros, group, rows=ch)
    up = w4a16_reference(x, packed, scales, zeros, group, rows=ch + i)
    return silu(gate) * up


def fp8_swiglu_reference(xq, sx, wq, sw, channels=None) -> np.ndarray:
    """h [M][I] = SiLU(g) * u for FP8 W8A8 operands: per-token activation
    codes xq [M][K] with scales sx, and the per-row quantized [2I][K]
    concatenation [W_gate; W_up] (codes wq, scales sw), gate rows first.  g
    and u are the fp64 products of the dequantized operands, i.e. the
    rescaled code products of figure 6-2 of 《第 6 课：量化源码走读》, and the
    activation follows 《推理优化与量化算子深度技术调研》 section 4.6 (the
    W8A8 GEMM with dequantization and activation fused).  ``channels``
    optionally selects intermediate channels (columns of h)."""
    wq = np.asarray(wq)
    sw = np.asarray(sw).reshape(-1)
    n2 = wq.shape[0]
    if n2 % 2:
        raise ValueError("invalid quantization geometry")
    i = n2 // 2
    ch = np.arange(i) if channels is None else np.asarray(channels)
    gate = fp8_reference(xq, sx, wq[ch], sw[ch])
    up = fp8_reference(xq, sx, wq[ch + i], sw[ch + i])
    return silu(gate) * up
