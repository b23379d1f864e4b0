"""Pins of the oracle's fused normalization + per-row quantization
(《推理优化与量化算子深度技术调研》 section 4.4): torch's own layer_norm and
rms_norm (independent library routines, float64), a hand-worked example,
exact scaling identities and invariants that a dropped term, the unbiased
variance or a wrong operand order breaks."""

import numpy as np
import pytest
import torch

from oracle import fp8 as F8
from oracle import intquant as IQ
from oracle import mx as MX
from oracle import norm as NQ


def _case(rows, k, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((rows, k)) * 1.5 + 0.3).astype(np.float32)
    g = (1.0 + 0.1 * rng.standard_normal(k)).astype(np.float32)
    b = (0.05 * rng.standard_normal(k)).astype(np.float32)
    return x, g, b


@pytest.mark.parametrize("k", [8, 64, 1000])
def test_layer_norm_matches_torch(k):
    x, g, b = _case(5, k, k)
    y = NQ.normalize(x, g, b, "layer", 1e-5)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x).double(), (k,),
                                         torch.from_numpy(g).double(),
                                         torch.from_numpy(b).double(), eps=1e-5).numpy()
    # float32 steps after float64 statistics: a few float32 units of the
    # largest term of the row
    tol = 8 * np.finfo(np.float32).eps * (np.abs(ref).max(axis=1, keepdims=True) + 1)
    assert (np.abs(y - ref) <= tol).all()


@pytest.mark.parametrize("k", [8, 64, 1000])
def test_rms_norm_matches_torch(k):
    x, g, _ = _case(4, k, 100 + k)
    y = NQ.normalize(x, g, None, "rms", 1e-6)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x).double(), (k,),
                                       torch.from_numpy(g).double(), eps=1e-6).numpy()
    tol = 8 * np.finfo(np.float32).eps * (np.abs(ref).max(axis=1, keepdims=True) + 1)
    assert (np.abs(y - ref) <= tol).all()


def test_worked_example_int8():
    # x = [1, 2, 3, 4], gamma 1, beta 0, eps 0: mean 2.5, biased variance
    # 1.25, normalized (x - 2.5) / sqrt(1.25); the absmax scale is
    # 1.5 / sqrt(1.25) / 127 and the codes 127 * [-1, -1/3, 1/3, 1] rounded
    x = np.array([[1, 2, 3, 4]], np.float32)
    q, s, z = NQ.norm_quant(x, np.ones(4, np.float32), np.zeros(4, np.float32), "layer",
                            "int8_sym", 0.0)
    assert z is None
    assert list(q[0]) == [-127, -42, 42, 127]
    assert abs(float(s[0]) - 1.5 / np.sqrt(1.25) / 127) < 1e-7
    # the unbiased variance (5 / 3) would give a scale 1.5 / sqrt(5 / 3) / 127
    assert abs(float(s[0]) - 1.5 / np.sqrt(5.0 / 3.0) / 127) > 1e-3


def test_biased_variance():
    # gamma 1, beta 0, eps 0: the normalized row has mean 0 and mean square 1
    # (the unbiased variance would give (K - 1) / K)
    x, _, _ = _case(3, 8, 7)
    y = NQ.normalize(x, np.ones(8, np.float32), np.zeros(8, np.float32), "layer", 0.0)
    assert np.allclose(y.astype(np.float64).mean(axis=1), 0.0, atol=1e-6)
    assert np.allclose((y.astype(np.float64) ** 2).mean(axis=1), 1.0, atol=1e-6)


def test_constant_row_gives_beta():
    # t = x - mean = 0 exactly, so y = 0 * gamma + beta = beta bit for bit
    k = 64
    _, g, b = _case(1, k, 3)
    x = np.full((2, k), 0.75, np.float32)
    y = NQ.normalize(x, g, b, "layer", 1e-5)
    assert (y == b[None, :]).all()
    q, s, _ = NQ.norm_quant(x, g, b, "layer", "fp8_e4m3", 1e-5)
    qb, sb = F8.quantize_rows(b[None, :])
    assert (q == qb).all() and (s == np.asarray(sb).reshape(-1)).all()


@pytest.mark.parametrize("kind", ["layer", "rms"])
def test_power_of_two_scaling_is_exact(kind):
    # with eps = 0, x -> 4 x scales mean by 4 and r by 1/4 exactly, so every
    # float32 step repeats bit for bit
    x, g, b = _case(3, 96, 11)
    y1 = NQ.normalize(x, g, b, kind, 0.0)
    y4 = NQ.normalize(4 * x, g, b, kind, 0.0)
    assert (y1 == y4).all()


def test_rms_closed_form():
    # rows of +-a (a a power of two), eps 0: r = 1 / a, u = +-1 exactly, so
    # y = +-gamma and the codes are those of +-gamma
    k = 32
    _, g, _ = _case(1, k, 5)
    signs = np.where(np.arange(k) % 3 == 0, -1.0, 1.0).astype(np.float32)
    x = np.stack([0.25 * signs, 8.0 * signs]).astype(np.float32)
    y = NQ.normalize(x, g, None, "rms", 0.0)
    assert (y == (signs * g)[None, :]).all()
    q, s, _ = NQ.norm_quant(x, g, None, "rms", "int8_sym", 0.0)
    q0, s0 = IQ.quantize_sym((signs * g)[None, :], k, "int8_sym")
    assert (q == q0).all() and (s == np.asarray(s0).reshape(-1)).all()


def test_asym_codes_span_the_range():
    x, g, b = _case(6, 256, 21)
    q, s, z = NQ.norm_quant(x, g, b, "layer", "int8_asym", 1e-5)
    assert q.dtype == np.uint8 and z is not None
    assert (q.min(axis=1) == 0).all() and (q.max(axis=1) >= 254).all()


def test_invalid_geometry():
    with pytest.raises(ValueError, match="invalid quantization geometry"):
        NQ.normalize(np.zeros((2, 8), np.float32), np.ones(4, np.float32), None, "rms", 1e-6)
    with pytest.raises(ValueError):
        NQ.norm_quant(np.zeros((2, 8), np.float32), np.ones(8), None, "rms", "int4_sym", 1e-6)


# --------------------------------------------------------------- MXFP4 output

def test_mx_output_hand_worked_rms_block():
    # RMSNorm of rows +-a (a a power of two), eps 0: u = +-1 exactly, so y =
    # +-gamma.  gamma puts one 32-element block on the E2M1 grid times 2^-3
    # (block max 6 * 2^-3 = 0.75, so e = -3, byte 124) and a second block
    # that rounds (max 0.3: e = -4, byte 123, values / 2^-4 = 4.8 -> 4 and
    # the rest of that block at 0.05 / 2^-4 = 0.8 -> 1 (code 2), 0.02 ->
    # 0.32 -> 0.5 (code 1), -0.1 -> -1.6 -> -1.5 (code 8 | 3))
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32)
    g0 = np.concatenate([grid, -grid, grid[::-1], -grid[::-1]]) * np.float32(2.0 ** -3)
    g1 = np.full(32, 0.05, np.float32)
    g1[0], g1[1], g1[2] = 0.3, 0.02, -0.1
    gamma = np.concatenate([g0, g1]).astype(np.float32)
    x = np.full((2, 64), 0.5, np.float32)
    x[1] *= -1.0
    codes, e8m0, z = NQ.norm_quant(x, gamma, None, "rms", "mxfp4", 0.0)
    assert z is None
    assert e8m0.tolist() == [[124, 123], [124, 123]]
    mag = [0, 1, 2, 3, 4, 5, 6, 7]
    b0 = mag + [8 | m for m in mag] + mag[::-1] + [8 | m for m in mag[::-1]]
    b0[8] = 8                                  # -0 keeps its sign bit
    b0[31] = 8
    b1 = [2] * 32
    b1[0], b1[1], b1[2] = 6, 1, 8 | 3          # 4.8 -> 4 (code 6), 0.32 -> 0.5, -1.6 -> -1.5
    want = np.array(b0 + b1, np.uint8)
    nib = np.stack([codes[0] & 15, codes[0] >> 4], axis=1).reshape(-1)
    assert nib.tolist() == want.tolist()
    # the negated row flips every sign bit, zeros included
    nib1 = np.stack([codes[1] & 15, codes[1] >> 4], axis=1).reshape(-1)
    assert (nib1 == (want ^ 8)).all()


def test_mx_output_constant_row_is_beta():
    # LayerNorm of a constant row is beta bit for bit, so the MX codes and
    # exponents are those of beta itself
    k = 96
    _, g, b = _case(1, k, 31)
    x = np.full((3, k), -1.25, np.float32)
    codes, e8m0, _ = NQ.norm_quant(x, g, b, "layer", "mxfp4", 1e-5)
    cb, eb = MX.quantize(b[None, :])
    assert (codes == cb).all() and (e8m0 == eb).all()


@pytest.mark.parametrize("kind", ["layer", "rms"])
def test_mx_output_agrees_with_torch_norm(kind):
    # torch's float64 normalization, rounded to float32, through the MX
    # quantizer: the codes agree except where float32 rounding moves a value
    # across an E2M1 midpoint or a block maximum across 6 * 2^e (then the two
    # sides may differ by one code step); a dropped term or a transposed
    # gamma would change most of them
    k = 256
    x, g, b = _case(64, k, 40 + len(kind))
    tx = torch.from_numpy(x).double()
    if kind == "layer":
        ref = torch.nn.functional.layer_norm(tx, (k,), torch.from_numpy(g).double(),
                                             torch.from_numpy(b).double(), eps=1e-5)
    else:
        ref = torch.nn.functional.rms_norm(tx, (k,), torch.from_numpy(g).double(), eps=1e-5)
    ref = ref.numpy().astype(np.float32)
    codes, e8m0, _ = NQ.norm_quant(x, g, b if kind == "layer" else None, kind, "mxfp4", 1e-5)
    rc, re = MX.quantize(ref)
    assert (e8m0 == re).mean() > 0.99
    same = (codes == rc).mean()
    assert same > 0.995, same
    # dequantized, the fused output is within one MX step of torch's values
    deq = MX.dequantize(codes, e8m0)
    step = np.repeat(2.0 ** (e8m0.astype(np.float64) - 127), 32, axis=1)
    assert (np.abs(deq - ref) <= 1.01 * step).all()
