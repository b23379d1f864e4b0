"""Pins of the oracle's SmoothQuant smoothing (《第 1 章：推理加速全景》 section
4.3; 《推理优化与量化算子深度技术调研》 section 1.5): brute-force channel maxima,
hand-computed factors that a swapped exponent or a wrong sign breaks, the
special cases alpha = 0 and alpha = 1, the migration balance invariant, the
page's outlier-channel example, the exact equivalence X W^T = X_hat W_hat^T
under power-of-two factors, and the reduction of the smoothed quantizer to
the plain one."""

import numpy as np
import pytest

from oracle import intquant as IQ
from oracle import smooth as SM


def test_channel_absmax_brute_force():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 13)).astype(np.float32)
    ref = [max(abs(float(x[r, j])) for r in range(7)) for j in range(13)]
    assert (SM.channel_absmax(x) == np.array(ref, np.float32)).all()
    # running maximum over two batches = maximum over their concatenation
    y = 3 * rng.standard_normal((5, 13)).astype(np.float32)
    assert (SM.channel_absmax(y, SM.channel_absmax(x)) ==
            SM.channel_absmax(np.concatenate([x, y]))).all()


def test_smooth_scales_hand_values():
    a = np.array([4, 9, 16, 1, 2], np.float32)
    w = np.array([1, 4, 1, 16, 2], np.float32)
    # alpha 0.5: sqrt(a / w) -> 2, 1.5, 4, 0.25, 1
    assert (SM.smooth_scales(a, w, 0.5) == np.array([2, 1.5, 4, 0.25, 1], np.float32)).all()
    # alpha 0.75: 16^0.75 / 1 = 8; alpha 0.25: 1 / 16^0.75 = 1/8 (a swapped
    # alpha / 1 - alpha would give 2 and 1/2)
    assert SM.smooth_scales(np.float32([16]), np.float32([1]), 0.75)[0] == 8.0
    assert SM.smooth_scales(np.float32([1]), np.float32([16]), 0.25)[0] == 0.125


def test_smooth_scales_alpha_limits():
    rng = np.random.default_rng(2)
    a = np.abs(rng.standard_normal(64)).astype(np.float32) + 0.1
    w = np.abs(rng.standard_normal(64)).astype(np.float32) * 0.02 + 1e-3
    # alpha = 0: the factor ignores the activations, s = 1 / w
    assert (SM.smooth_scales(a, w, 0.0) == (1.0 / w.astype(np.float64)).astype(np.float32)).all()
    # alpha = 1: full migration, s = a
    assert (SM.smooth_scales(a, w, 1.0) == a).all()


def test_smooth_scales_degenerate_channels():
    a = np.array([0, 1, 0, 1e30], np.float32)
    w = np.array([1, 0, 0, 1e-30], np.float32)
    s = SM.smooth_scales(a, w, 0.5)
    assert s[0] == 1 and s[1] == 1 and s[2] == 1      # a zero statistic: no migration
    assert s[3] == np.float32(1e30)                    # sqrt(1e60) is representable
    # alpha = 1: s = a, a subnormal a is not a usable factor
    s1 = SM.smooth_scales(np.float32([1e-40, 1e-30]), np.float32([1, 1]), 1.0)
    assert s1[0] == 1 and s1[1] == np.float32(1e-30)
    # alpha = 0: s = 1 / w overflows for a subnormal w
    assert SM.smooth_scales(np.float32([1]), np.float32([1e-39]), 0.0)[0] == 1
    with pytest.raises(ValueError):
        SM.smooth_scales(a, w, 1.5)


def test_migration_balance_invariant():
    # after smoothing, max|X_hat_j| = a / s = (a w)^(1 - alpha) and
    # max|W_hat_j| = w s = (a w)^alpha, so their ratio is (a_j w_j)^(1 - 2
    # alpha); at alpha 0.5 both maxima are sqrt(a_j w_j)
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((64, 32)) * np.exp(rng.standard_normal(32))).astype(np.float32)
    w = (rng.standard_normal((48, 32)) * 0.02).astype(np.float32)
    a, wm = SM.channel_absmax(x), SM.channel_absmax(w)
    for alpha in (0.25, 0.5, 0.8):
        s = SM.smooth_scales(a, wm, alpha)
        xm = SM.channel_absmax(SM.fold(x, s, True)).astype(np.float64)
        ww = SM.channel_absmax(SM.fold(w, s, False)).astype(np.float64)
        ratio = (a.astype(np.float64) * wm) ** (1 - 2 * alpha)
        assert np.allclose(xm / ww, ratio, rtol=1e-5)
        if alpha == 0.5:
            assert np.allclose(xm, np.sqrt(a.astype(np.float64) * wm), rtol=1e-6)


def test_page_outlier_channel_example():
    # 511 channels within [-0.5, 0.5] and one within [-8, 8]; weights with the
    # same column maximum everywhere: alpha 0.5 shrinks the 16x gap to sqrt(16)
    rng = np.random.default_rng(4)
    x = rng.uniform(-0.5, 0.5, (256, 512)).astype(np.float32)
    x[:, 511] = rng.uniform(-8, 8, 256).astype(np.float32)
    x[0, :511] = 0.5
    x[0, 511] = 8.0
    w = rng.uniform(-0.25, 0.25, (64, 512)).astype(np.float32)
    w[0, :] = 0.25
    s = SM.smooth_scales(SM.channel_absmax(x), SM.channel_absmax(w), 0.5)
    xm = SM.channel_absmax(SM.fold(x, s, True)).astype(np.float64)
    assert np.isclose(xm[511] / xm[:511].max(), 4.0, rtol=1e-6)
    assert np.allclose(xm[:511], xm[0], rtol=1e-6)


def test_equivalence_exact_under_power_of_two_factors():
    # Y = (X diag(s)^-1)(diag(s) W): with s_j = 2^e_j every folded value and
    # every product is exact, so the float64 products agree bit for bit
    rng = np.random.default_rng(5)
    x = rng.standard_normal((9, 40)).astype(np.float32)
    w = (rng.standard_normal((11, 40)) * 0.02).astype(np.float32)
    s = np.ldexp(np.float32(1), rng.integers(-6, 7, 40)).astype(np.float32)
    xs, ws = SM.fold(x, s, True), SM.fold(w, s, False)

    def prod(p, q):
        return (p.astype(np.float64)[:, None, :] * q.astype(np.float64)[None, :, :]).sum(-1)
    assert (prod(xs, ws) == prod(x, w)).all()
    # general factors: each term off by at most two float32 roundings
    s2 = SM.smooth_scales(SM.channel_absmax(x), SM.channel_absmax(w), 0.5)
    d = np.abs(prod(SM.fold(x, s2, True), SM.fold(w, s2, False)) - prod(x, w))
    bound = 2.5 * np.finfo(np.float32).eps * prod(np.abs(x), np.abs(w))
    assert (d <= bound).all()


@pytest.mark.parametrize("fmt,group", [("int4_sym", 128), ("int4_asym", 128), ("int8_sym", 256),
                                       ("int8_asym", 256), ("fp8_e4m3", 256)])
def test_unit_factors_reduce_to_plain_quantizer(fmt, group):
    rng = np.random.default_rng(6)
    w = (rng.standard_normal((6, 256)) * 0.02).astype(np.float32)
    one = np.ones(256, np.float32)
    plain = SM.quantize(w, fmt, group)
    for divide in (False, True):
        got = SM.smooth_quantize(w, one, divide, fmt, group)
        for p, g in zip(plain, got):
            assert (p is None and g is None) or (np.asarray(p) == np.asarray(g)).all()
    # the generic quantizer itself against the pinned int8 routine
    q, s = IQ.quantize_sym(w, group if fmt != "int4_sym" else 128, "int8_sym")
    c8, s8, _ = SM.quantize(w, "int8_sym", group if fmt != "int4_sym" else 128)
    assert (c8 == q.astype(np.int8)).all() and (s8 == s).all()


@pytest.mark.parametrize("fmt", ["int8_sym", "fp8_e4m3"])
def test_uniform_power_of_two_factor_scales_only_the_scales(fmt):
    # W_hat = W * 4: same codes, scales x 4 exactly; X_hat = X / 4: scales / 4
    rng = np.random.default_rng(7)
    w = (rng.standard_normal((5, 64)) * 0.02).astype(np.float32)
    c0, s0, _ = SM.quantize(w, fmt, 64)
    four = np.full(64, 4.0, np.float32)
    cm, sm, _ = SM.smooth_quantize(w, four, False, fmt, 64)
    cd, sd, _ = SM.smooth_quantize(w, four, True, fmt, 64)
    assert (cm == c0).all() and (cd == c0).all()
    assert (sm == 4 * s0).all() and (sd == s0 / 4).all()


def test_smoothing_helps_int8_w8a8_with_outlier_channels():
    # the purpose stated on both pages: activations with a few large channels
    # quantize badly per token; after smoothing the INT8 product error drops
    rng = np.random.default_rng(8)
    m, k, n = 64, 512, 64
    x = rng.standard_normal((m, k)).astype(np.float32)
    x[:, rng.choice(k, 5, replace=False)] *= 40
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    ref = x.astype(np.float64) @ w.astype(np.float64).T

    def w8a8(xx, ww):
        qx, sx = IQ.quantize_sym(xx, k, "int8_sym")
        qw, sw = IQ.quantize_sym(ww, k, "int8_sym")
        return (IQ.dequantize(qx, sx, None, k) @ IQ.dequantize(qw, sw, None, k).T)

    def err(y):
        return np.linalg.norm(y - ref) / np.linalg.norm(ref)
    s = SM.smooth_scales(SM.channel_absmax(x), SM.channel_absmax(w), 0.5)
    e_plain = err(w8a8(x, w))
    e_smooth = err(w8a8(SM.fold(x, s, True), SM.fold(w, s, False)))
    assert e_smooth < 0.5 * e_plain


def test_invalid_geometry():
    with pytest.raises(ValueError, match="invalid quantization geometry"):
        SM.channel_absmax(np.zeros((0, 8), np.float32))
    with pytest.raises(ValueError, match="invalid quantization geometry"):
        SM.fold(np.zeros((2, 8), np.float32), np.ones(4, np.float32), True)
    with pytest.raises(ValueError, match="invalid quantization geometry"):
        SM.smooth_scales(np.ones(4, np.float32), np.ones(5, np.float32), 0.5)
