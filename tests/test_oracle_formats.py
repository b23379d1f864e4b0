"""Pins of the oracle's float formats: value tables against the format table
printed on 《量化与加速》, encoders against independent library conversions
and hand-derived tie cases, bf16 rounding against torch."""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_format_maxima_match_the_page_table():
    g = _gold("format_table.json")
    for name, spec in g["float_formats"].items():
        e, m, _ = F.FORMATS[name]
        assert (e, m) == (spec["exponent_bits"], spec["mantissa_bits"])
        assert F.max_finite(name) == spec["max"]
    assert F.format_bias("fp16") == g["float_formats"]["fp16"]["bias"]


def test_e2m1_grid_by_hand():
    # E=2, M=1, bias 1: subnormals 0, 0.5; normals 1, 1.5, 2, 3, 4, 6
    assert list(F.value_table("e2m1")[:8]) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert list(F.value_table("e2m1")[8:]) == [-0.0, -0.5, -1, -1.5, -2, -3, -4, -6]


def test_e4m3_table_special_codes():
    t = F.value_table("e4m3")
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.isfinite(t[:0x7F]).all()
    assert t[0x7E] == 448.0 and t[0x01] == 2.0 ** -9 and t[0x08] == 2.0 ** -6


def test_e4m3_encoder_matches_torch_cast_after_clamp():
    # torch's float8_e4m3fn conversion is an independent RNE implementation; it
    # yields NaN beyond the range, so compare after clamping to +-448.
    rng = np.random.default_rng(11)
    x = np.concatenate([
        rng.standard_normal(400_000).astype(np.float32) * np.float32(50),
        rng.standard_normal(200_000).astype(np.float32) * np.float32(0.01),
        (rng.random(100_000, dtype=np.float32) * np.float32(480)),
    ])
    # every bf16 bit pattern that is finite
    allbf = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    x = np.concatenate([x, allbf[np.isfinite(allbf)]])
    xc = np.clip(x, -448, 448)
    ours = F.encode(xc, "e4m3")
    ref = torch.from_numpy(xc).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (ours == ref).all()


def test_e4m3_saturates_and_round_trips():
    assert F.encode(np.float32(1e6), "e4m3") == 0x7E
    assert F.encode(np.float32(-500), "e4m3") == 0xFE
    assert F.encode(np.float32(464), "e4m3") == 0x7E     # above the last midpoint too
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    assert (F.encode(F.decode(codes, "e4m3"), "e4m3") == codes).all()
    assert F.encode(np.float32(-1e-30), "e4m3") == 0x80  # sign kept on zero


def test_fp16_encoder_matches_numpy_conversion():
    rng = np.random.default_rng(12)
    x = np.concatenate([rng.standard_normal(300_000).astype(np.float32) * 1000,
                        rng.standard_normal(300_000).astype(np.float32) * 1e-5])
    x = x[np.abs(x) < 65504]
    assert (F.encode(x, "fp16") == x.astype(np.float16).view(np.uint16)).all()


def test_e5m2_encoder_matches_torch_cast():
    rng = np.random.default_rng(13)
    x = np.clip(rng.standard_normal(300_000).astype(np.float32) * 3000, -57344, 57344)
    ref = torch.from_numpy(x).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert (F.encode(x, "e5m2") == ref).all()


def test_e2m1_ties_go_to_the_even_code():
    # midpoints of the grid, derived by hand: (0|0.5) (1|1.5) ... (4|6)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    expect_vals = [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]
    got = F.decode(F.encode(mids, "e2m1"), "e2m1")
    assert list(got) == expect_vals
    assert list(F.decode(F.encode(-mids, "e2m1"), "e2m1")) == [-v for v in expect_vals]
    assert F.encode(7.0, "e2m1") == 7 and F.encode(-100.0, "e2m1") == 15


def test_e2m1_agrees_with_the_half_step_rounding_on_0_to_2():
    # 《大模型量化推理引擎全景大复盘》 section 3 code rounds x/s on a 0.5 grid
    # (round(2v)/2, half-even); on [0, 2) that grid is exactly E2M1's.
    v = np.linspace(0, 1.999, 20001)
    half_grid = np.rint(2 * v) / 2
    assert (F.decode(F.encode(v, "e2m1"), "e2m1") == half_grid).all()


def test_e2m1_is_nearest_by_exact_search():
    grid = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2),
            Fraction(3), Fraction(4), Fraction(6)]
    rng = np.random.default_rng(14)
    vals = rng.random(3000) * 7
    got = F.decode(F.encode(vals, "e2m1"), "e2m1")
    for v, g in zip(vals, got):
        fv = Fraction(float(v))
        best = min(grid, key=lambda c: (abs(c - fv), grid.index(c) % 2))
        if fv > 6:
            best = Fraction(6)
        assert Fraction(float(g)) == best


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(15)
    x = np.concatenate([
        rng.standard_normal(500_000).astype(np.float32),
        (rng.integers(0, 2 ** 32, 500_000, dtype=np.uint64).astype(np.uint32)).view(np.float32),
    ])
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    got = F.round_to_bf16(x)
    same = (got.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def test_bf16_tie_cases_by_hand():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: the even one (1.0) wins;
    # 1 + 3*2^-8 lies halfway between 1+2^-7 (odd) and 1+2^-6 (even).
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8)], dtype=np.float32)
    assert list(F.round_to_bf16(x)) == [1.0, 1 + 2 ** -6, -1.0]


def test_fp16_scale_storage_saturates():
    h = F.round_to_fp16_saturating(np.array([1e6, -1e6, 65504, 65519, 1.0], dtype=np.float32))
    assert list(h.astype(np.float64)) == [65504, -65504, 65504, 65504, 1.0]


@pytest.mark.parametrize("name", ["e4m3", "e5m2", "e2m1"])
def test_tables_are_monotonic_in_code(name):
    e, m, _ = F.FORMATS[name]
    t = F.value_table(name)[: 2 ** (e + m)]
    fin = t[np.isfinite(t)]
    assert (np.diff(fin) > 0).all()
