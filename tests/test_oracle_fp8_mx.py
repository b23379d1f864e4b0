"""Pins of the oracle's FP8 per-row quantization and MXFP4 block quantization:
exact rational evaluation of the shared-exponent rule, the invariants that
rule implies, error bounds, and library conversions for the E4M3 codes."""

import math
from fractions import Fraction

import numpy as np
import torch

from oracle import formats as F
from oracle import fp8, mx


def _exact_ceil_log2_ratio(m: float, d: int = 6) -> int:
    """ceil(log2(m/d)) evaluated with exact rationals."""
    r = Fraction(m) / d
    e = 0
    while Fraction(2) ** e < r:
        e += 1
    while Fraction(2) ** (e - 1) >= r:
        e -= 1
    return e


def test_shared_exponent_exact_rule():
    rng = np.random.default_rng(21)
    vals = list((rng.standard_normal(2000) * 10.0 ** rng.integers(-20, 20, 2000)).astype(np.float32))
    edges = []
    for k in range(-40, 40):
        b = np.float32(6.0 * 2.0 ** k)
        edges += [b, np.nextafter(b, np.float32(np.inf)), np.nextafter(b, np.float32(0)),
                  np.float32(3.0 * 2.0 ** k), np.nextafter(np.float32(3.0 * 2.0 ** k), np.float32(np.inf))]
    for v in vals + edges:
        m = abs(float(v))
        if m == 0:
            continue
        assert mx.shared_exponent(m) == max(-127, min(127, _exact_ceil_log2_ratio(m))), m


def test_shared_exponent_zero_and_clamps():
    assert mx.shared_exponent(0.0) == 0
    assert mx.shared_exponent(1e-45) == -127
    assert mx.shared_exponent(3.0e38) == 126


def _blocks(seed, rows=64, k=1024):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, k)).astype(np.float32)
    x[:, 7] *= 50
    x[3, 64:96] = 0.0                     # an all-zero block
    return x


def test_mx_block_invariants():
    x = _blocks(22)
    packed, e8 = mx.quantize(x)
    e = e8.astype(np.int64) - 127
    m = np.abs(x.reshape(64, 32, 32)).max(axis=2).astype(np.float64)
    nz = m > 0
    assert ((3 * np.exp2(e) < m) | ~nz).all() and ((m <= 6 * np.exp2(e)) | ~nz).all()
    assert (e[~nz] == 0).all()
    codes = mx.unpack_codes(packed).reshape(64, 32, 32)
    mags = F.decode(codes & 7, "e2m1").max(axis=2)
    assert np.isin(mags[nz], [3.0, 4.0, 6.0]).all()
    assert (mags[~nz] == 0).all()
    # error bound: at most half the grid spacing at the value, <= 2^e overall,
    # and <= 2^(e-2) for |x|/2^e < 2
    x_hat = mx.dequantize(packed, e8)
    se = np.repeat(np.exp2(e.astype(np.float64)), 32, axis=1)
    err = np.abs(x - x_hat)
    assert (err <= se).all()
    small = np.abs(x) / se < 2
    assert (err[small] <= se[small] / 4).all()


def test_mx_idempotent_iff_block_max_code_is_4_or_6():
    x = _blocks(23)
    packed, e8 = mx.quantize(x)
    x_hat = mx.dequantize(packed, e8).astype(np.float32)
    p2, e2 = mx.quantize(x_hat)
    mags = F.decode(mx.unpack_codes(packed) & 7, "e2m1").reshape(64, 32, 32).max(axis=2)
    same_block = (mx.unpack_codes(p2).reshape(64, 32, 32) == mx.unpack_codes(packed).reshape(
        64, 32, 32)).all(axis=2) & (e2 == e8)
    assert (same_block == np.isin(mags, [0.0, 4.0, 6.0])).all()


def test_mx_packing_low_nibble_first_and_sign():
    x = np.zeros((1, 32), np.float32)
    x[0, 0], x[0, 1], x[0, 2], x[0, 3] = 6.0, -0.5, 1.0, -6.0
    packed, e8 = mx.quantize(x)
    assert e8[0, 0] == 127
    assert packed[0, 0] == (0x7 | (0x9 << 4)) and packed[0, 1] == (0x2 | (0xF << 4))


def test_mx_geometry_error():
    import pytest
    with pytest.raises(ValueError, match="invalid quantization geometry"):
        mx.quantize(np.zeros((2, 48), np.float32))


def test_fp8_rows_codes_match_torch_and_scale_rule():
    rng = np.random.default_rng(24)
    x = rng.standard_normal((32, 512)).astype(np.float32)
    x.reshape(-1)[rng.choice(x.size, 20, replace=False)] *= 100
    x[5] = 0.0
    codes, s = fp8.quantize_rows(x)
    amax = np.abs(x).max(axis=1)
    assert s[5] == 1.0
    assert (s[amax > 0] == (amax[amax > 0] / np.float32(448)).astype(np.float32)).all()
    v = np.clip(x / s[:, None], -448, 448)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (codes == ref).all()
    # every non-zero row reaches the top code exactly (the absmax maps to 448)
    mags = codes & 0x7F
    assert (mags.max(axis=1)[amax > 0] == 0x7E).all()
    # relative error of E4M3 with RNE: at most 2^-4 of the value for normals
    x_hat = fp8.dequantize_rows(codes, s)
    normal = np.abs(x / s[:, None]) >= 2.0 ** -6
    assert (np.abs(x - x_hat)[normal] <= np.abs(x)[normal] * 2.0 ** -4 * (1 + 1e-6)).all()
