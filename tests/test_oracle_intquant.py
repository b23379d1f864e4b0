"""Pins of the oracle's integer quantization: the lesson's worked example and
exercise (values printed on 《第 6 课：量化源码走读》), hand-derived cases, and
invariants that a dropped term, a wrong divisor or a wrong rounding breaks."""

import json
import os

import numpy as np
import pytest

from oracle import intquant as IQ

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_worked_example_exact_scale():
    g = _gold("lesson6_worked_example.json")
    x = np.array([g["x"]], dtype=np.float64)
    q, s = IQ.quantize_sym(x, len(g["x"]), scale_dtype="f64", qmax=g["q_max"])
    assert float(s[0, 0]) == 8.0 / 7
    assert list(q[0]) == g["q"]
    x_hat = q[0] * s[0, 0]
    assert np.allclose(x_hat, g["x_hat_printed"], atol=0.5 * 10 ** -g["printed_decimals"])
    assert abs(x_hat[-1] - 8.0) < 1e-12            # the maximum is reproduced


def test_worked_example_with_fp16_scale():
    # the stored-scale form used by the INT4 format: same codes, the scale is
    # fp16(8/7) = 1.142578125 and the maximum comes back as 7.998046875.
    g = _gold("lesson6_worked_example.json")
    q, s = IQ.quantize_sym(np.array([g["x"]], dtype=np.float32), 4, "int4_sym")
    assert list(q[0]) == g["q"]
    assert float(s[0, 0]) == 1.142578125
    x_hat = IQ.dequantize(q, s, None, 4)[0]
    assert np.allclose(x_hat, g["x_hat_printed"], atol=3e-3)


def test_exercise_cases():
    g = _gold("lesson6_exercise.json")
    c0, c1 = g["cases"]
    restored, scales = IQ.blockwise_symmetric_fake_quant(c0["values"], c0["block_size"], c0["qmax"])
    assert scales == [1 / 7, 8 / 7]
    assert abs(restored[1] - c0["restored_index_1"]) < c0["abs_tol"]
    assert abs(restored[-1] - c0["restored_last"]) < c0["abs_tol"]
    assert IQ.blockwise_symmetric_fake_quant(c1["values"], c1["block_size"], c1["qmax"]) == (
        c1["restored"], c1["scales"])
    for vals, bs, qm in g["invalid_geometry"]:
        with pytest.raises(ValueError, match=g["error"]):
            IQ.blockwise_symmetric_fake_quant(vals, bs, qm)


def test_symmetric_ties_round_half_even():
    # group max 7 -> scale exactly 1 (fp16); ties at .5 go to the even integer
    x = np.array([[7.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5]], dtype=np.float32)
    q, s = IQ.quantize_sym(x, 8, "int4_sym")
    assert float(s[0, 0]) == 1.0
    assert list(q[0]) == [7, 0, 2, 2, 0, -2, -2, 4]


def test_asymmetric_hand_case():
    # min -1, max 14 -> scale (15)/15 = 1, z = round(1) = 1; q = round(x) + 1
    x = np.array([[-1.0, 14.0, 0.0, 0.5, 2.5, 13.4, -0.6, 6.5]], dtype=np.float32)
    q, s, z = IQ.quantize_asym(x, 8, "int4_asym")
    assert float(s[0, 0]) == 1.0 and float(z[0, 0]) == 1.0
    assert list(q[0]) == [0, 15, 1, 1, 3, 14, 0, 7]


def test_zero_group_uses_scale_one():
    x = np.zeros((2, 256), dtype=np.float32)
    q, s = IQ.quantize_sym(x, 128)
    assert (s == 1).all() and (q == 0).all()
    q, s, z = IQ.quantize_asym(x, 128)
    assert (s == 1).all() and (z == 0).all() and (q == 0).all()


def _rand(rows, k, seed, scale=0.02):
    return (np.random.default_rng(seed).standard_normal((rows, k)) * scale).astype(np.float32)


def test_symmetric_invariants():
    x = _rand(64, 1024, 1)
    q, s = IQ.quantize_sym(x, 128)
    g = q.reshape(64, 8, 128)
    assert (np.abs(g).max(axis=2) == 7).all()          # every group reaches q_max
    x_hat = IQ.dequantize(q, s, None, 128)
    s_rep = np.repeat(s.astype(np.float64), 128, axis=1)
    assert (np.abs(x - x_hat) <= s_rep / 2 * (1 + 2 ** -10)).all()  # in-range bound
    # idempotence: quantizing the dequantized values reproduces the codes
    q2, s2 = IQ.quantize_sym(x_hat.astype(np.float32), 128)
    assert (q2 == q).all() and (s2 == s).all()


def test_asymmetric_invariants():
    x = _rand(64, 1024, 2)
    x[:, :40] *= 20                                     # outlier input channels
    q, s, z = IQ.quantize_asym(x, 128)
    assert (z == np.rint(z)).all()                      # integer zero point
    g = x.reshape(64, 8, 128)
    gq = q.reshape(64, 8, 128)
    lo_idx = g.argmin(axis=2)
    assert (np.take_along_axis(gq, lo_idx[:, :, None], 2) == 0).all()   # q(min) == 0
    hi_idx = g.argmax(axis=2)
    assert np.isin(np.take_along_axis(gq, hi_idx[:, :, None], 2), [14, 15]).all()
    # in range (the unclipped code lies in [0, 15]) the error is at most s/2;
    # the clip at the top costs at most the rounding of s and z on top of it
    x_hat = IQ.dequantize(q, s, z, 128)
    s_rep = np.repeat(s.astype(np.float64), 128, axis=1)
    z_rep = np.repeat(z.astype(np.float32), 128, axis=1)
    raw = np.rint(x / s_rep.astype(np.float32)) + z_rep
    inside = (raw >= 0) & (raw <= 15)
    err = np.abs(x - x_hat)
    assert (err[inside] <= s_rep[inside] / 2 * (1 + 2 ** -10)).all()
    assert (err <= s_rep * (0.5 + 2 ** -6)).all()
    assert inside.mean() > 0.99
    # q(0) == z whenever 0 <= z <= 15, and 0 dequantizes to exactly 0
    x0 = x.copy()
    x0[:, 5] = 0.0
    q0, s0, z0 = IQ.quantize_asym(x0, 128)
    assert (q0[:, 5] == z0[:, 0]).all()
    assert (IQ.dequantize(q0, s0, z0, 128)[:, 5] == 0).all()


def test_quantization_error_variance_is_s2_over_12():
    # 《第 1 章：推理加速全景》 section 4.1: in-range error variance s^2 / 12
    x = _rand(256, 4096, 3)
    q, s, z = IQ.quantize_asym(x, 128)
    err = (x - IQ.dequantize(q, s, z, 128)) / np.repeat(s.astype(np.float64), 128, axis=1)
    assert abs(np.var(err) - 1 / 12) < 0.01 / 12 * 10


def test_cross_term_identity():
    # sum_k x_k * s (q_k - z) == s * (sum x q - z * sum x): the zero-point cross
    # term of 《第 6 课：量化源码走读》 section 3; dropping it changes the result.
    x_act = np.random.default_rng(4).standard_normal(128)
    w = _rand(1, 128, 5)
    q, s, z = IQ.quantize_asym(w, 128)
    s, z = float(s[0, 0]), float(z[0, 0])
    direct = float(np.dot(x_act, IQ.dequantize(q, [[s]], [[z]], 128)[0]))
    split = s * (float(np.dot(x_act, q[0])) - z * float(np.sum(x_act)))
    assert abs(direct - split) < 1e-12 * max(1, abs(direct))
    assert abs(direct - s * float(np.dot(x_act, q[0]))) > 1e-6


def test_pack_nibble_order_by_hand():
    q = np.array([[0, 1, 2, 3, 4, 5, 6, 7, -1, -8, 0, 0, 0, 0, 0, 7]], dtype=np.int32)
    w = IQ.pack_int4(q).view(np.uint32)
    assert w[0, 0] == 0x76543210
    assert w[0, 1] == 0x7000008F
    assert (IQ.unpack_int4(IQ.pack_int4(q), signed=True) == q).all()
    u = np.arange(16, dtype=np.int32).reshape(1, 16)
    assert (IQ.unpack_int4(IQ.pack_int4(u), signed=False) == u).all()


def test_int8_formulas():
    # max 127 -> s = 1 exactly; ties at .5 to even; clip at +-127
    x = np.array([[-127.0, 0.0, 63.5, 64.5, 127.0, -0.5]], dtype=np.float32)
    q, s = IQ.quantize_sym(x, 6, "int8_sym")
    assert float(s[0, 0]) == 1.0
    assert list(q[0]) == [-127, 0, 64, 64, 127, 0]
    # asym: min -1, max 1.55 -> s = 2.55/255 = 0.01, z = round(100) = 100
    x = np.array([[-1.0, 1.55, 0.0, 0.5]], dtype=np.float32)
    q, s, z = IQ.quantize_asym(x, 4, "int8_asym")
    assert float(z[0, 0]) == 100.0
    assert list(q[0]) == [0, 255, 100, 150]


def test_geometry_errors():
    with pytest.raises(ValueError, match="invalid quantization geometry"):
        IQ.quantize_sym(np.zeros((2, 100), np.float32), 128)
    with pytest.raises(ValueError, match="invalid quantization geometry"):
        IQ.quantize_sym(np.zeros((2, 128), np.float32), 0)
    with pytest.raises(ValueError, match="invalid quantization geometry"):
        IQ.pack_int4(np.zeros((1, 12), np.int32))
