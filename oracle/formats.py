"""Floating-point formats of the quantized path, written from their definition.

Test infrastructure only (see the package docstring).

Source: 《量化与加速》 (docs.ifdog.com), section "浮点数的数学表示": a float with
E exponent bits and M mantissa bits has the value (-1)^s * 2^(e - bias) * (1 + m)
with bias = 2^(E-1) - 1; its format table lists E4M3 at +-448, E5M2 at
+-57344, FP16 at +-65504.  The page states only the normal-number formula;
the reading adopted here is the usual IEEE extension to subnormals (exponent
field 0 encodes 2^(1-bias) * m), and per-format special codes:

* E4M3 (OCP "FN" variant): no infinities; only exponent 15 with mantissa 111
  is NaN, so the largest finite value is 1.75 * 2^8 = 448 (the table's +-448).
* E5M2 and FP16: IEEE, exponent all-ones is inf/NaN (maxima 57344 and 65504).
* E2M1 (FP4): no special codes; magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}, the
  maximum 6 being the divisor of the MX scale rule in
  《大模型量化推理引擎全景大复盘》 section 3 code.

Codes are sign-magnitude: bit (E+M) is the sign, the low E+M bits the
magnitude code, and magnitude codes are ordered by value.

Encoding is "nearest representable value, ties to the even code", with
saturation to the largest finite magnitude (the FP8 workload of the
quantized GEMM is stated as saturating); the sign of the input is kept, so a
negative input that rounds to zero encodes as negative zero.
"""

from __future__ import annotations

import numpy as np

# (exponent bits, mantissa bits, kind of special codes)
FORMATS = {
    "e4m3": (4, 3, "fn"),      # OCP E4M3FN: only S.1111.111 is NaN
    "e5m2": (5, 2, "ieee"),    # IEEE-like
    "fp16": (5, 10, "ieee"),   # IEEE binary16
    "e2m1": (2, 1, "none"),    # OCP FP4, all codes finite
}


def format_bias(name: str) -> int:
    """bias = 2^(E-1) - 1 (《量化与加速》, "浮点数的数学表示")."""
    e_bits, _, _ = FORMATS[name]
    return 2 ** (e_bits - 1) - 1


def value_table(name: str) -> np.ndarray:
    """Value of every code of the format, as float64, NaN for NaN codes and
    +-inf for infinity codes.  Index = code (sign bit included)."""
    e_bits, m_bits, kind = FORMATS[name]
    bias = format_bias(name)
    n_mag = 2 ** (e_bits + m_bits)
    e_max_field = 2 ** e_bits - 1
    mags = np.empty(n_mag, dtype=np.float64)
    for code in range(n_mag):
        e_field = code >> m_bits
        m_field = code & (2 ** m_bits - 1)
        frac = m_field / 2.0 ** m_bits
        if kind == "ieee" and e_field == e_max_field:
            mags[code] = np.inf if m_field == 0 else np.nan
            continue
        if kind == "fn" and e_field == e_max_field and m_field == 2 ** m_bits - 1:
            mags[code] = np.nan
            continue
        if e_field == 0:                       # subnormal: 2^(1-bias) * m
            mags[code] = 2.0 ** (1 - bias) * frac
        else:                                  # normal: 2^(e-bias) * (1+m)
            mags[code] = 2.0 ** (e_field - bias) * (1.0 + frac)
    return np.concatenate([mags, -mags])


def max_finite(name: str) -> float:
    t = value_table(name)
    return float(np.max(t[np.isfinite(t)]))


def _finite_magnitudes(name: str) -> tuple[np.ndarray, np.ndarray]:
    """Non-negative finite magnitudes with their codes (sorted by value)."""
    e_bits, m_bits, _ = FORMATS[name]
    n_mag = 2 ** (e_bits + m_bits)
    t = value_table(name)[:n_mag]
    codes = np.arange(n_mag)
    keep = np.isfinite(t)
    order = np.argsort(t[keep], kind="stable")
    return t[keep][order], codes[keep][order]


def encode(x, name: str) -> np.ndarray:
    """Round each value to the nearest finite value of the format, ties to the
    even code, saturating at the largest finite magnitude; keep the sign.

    ``x`` is converted to float64 (exact for fp32/bf16 inputs).  Returns the
    codes as uint8 (uint16 for fp16).  NaN inputs are outside the contract.
    """
    e_bits, m_bits, _ = FORMATS[name]
    x = np.asarray(x, dtype=np.float64)
    mags, codes = _finite_magnitudes(name)
    a = np.abs(x)
    # candidate below (largest magnitude <= a) and above (smallest >= a)
    hi = np.searchsorted(mags, a, side="left")
    hi_c = np.minimum(hi, len(mags) - 1)
    lo_c = np.maximum(hi - 1, 0)
    v_hi, v_lo = mags[hi_c], mags[lo_c]
    d_hi, d_lo = np.abs(v_hi - a), np.abs(a - v_lo)
    c_hi, c_lo = codes[hi_c], codes[lo_c]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (c_hi % 2 == 0))
    mag_code = np.where(pick_hi, c_hi, c_lo)
    mag_code = np.where(a >= mags[-1], codes[-1], mag_code)      # saturate
    sign = np.signbit(x).astype(np.int64)
    out = (sign << (e_bits + m_bits)) | mag_code
    return out.astype(np.uint16 if e_bits + m_bits + 1 > 8 else np.uint8)


def decode(codes, name: str) -> np.ndarray:
    """Value of each code (float64)."""
    return value_table(name)[np.asarray(codes, dtype=np.int64)]


# ----------------------------------------------------------------------------
# bf16 / fp16 rounding of fp32 values


def round_to_bf16(x) -> np.ndarray:
    """Round fp32 values to the nearest bf16 value, ties to even, returned as
    fp32.  bf16 values are exactly the fp32 values whose low 16 bits are zero;
    the two candidates around x are its truncation and the next bf16 away from
    zero, and the nearer one wins (on a tie, the one whose bit 16 is clear).
    Values beyond the largest bf16 round to infinity as IEEE rounding does.
    """
    x = np.asarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    trunc = bits & 0xFFFF0000
    up = trunc + 0x10000                       # next magnitude (may reach inf)
    v_t = trunc.astype(np.uint32).view(np.float32).astype(np.float64)
    v_u = up.astype(np.uint32).view(np.float32).astype(np.float64)
    # rounding up past the largest bf16 gives infinity; for the distance it
    # stands at the next step of the grid, 2^128 (as in IEEE rounding)
    v_u = np.where(np.isinf(v_u), np.copysign(2.0 ** 128, v_u), v_u)
    xf = x.astype(np.float64)
    d_t = np.abs(xf - v_t)
    d_u = np.abs(v_u - xf)
    even_t = (trunc & 0x10000) == 0
    take_up = (d_u < d_t) | ((d_u == d_t) & ~even_t)
    res = np.where(take_up, up, trunc).astype(np.uint32)
    res = np.where(np.isfinite(x), res, bits.astype(np.uint32))
    return res.view(np.float32)


def bf16_bits(x) -> np.ndarray:
    """uint16 bit patterns of round_to_bf16(x)."""
    return (round_to_bf16(x).view(np.uint32) >> 16).astype(np.uint16)


def round_to_fp16_saturating(x) -> np.ndarray:
    """fp32 -> fp16 with IEEE round-to-nearest-even (numpy's conversion), with
    results that overflow to infinity clamped to +-65504 (the format table's
    FP16 range).  Returned as float16."""
    x = np.asarray(x, dtype=np.float32)
    with np.errstate(over="ignore"):
        h = x.astype(np.float16)
    fmax = np.float16(65504.0)
    h = np.where(np.isinf(h) & np.isfinite(x), np.copysign(fmax, x).astype(np.float16), h)
    return h.astype(np.float16)
