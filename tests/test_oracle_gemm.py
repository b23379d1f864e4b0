"""Pins of the oracle's reference products: pure-Python brute force, closed
forms for constant operands, one-hot activations, and the error metric."""

import numpy as np
import pytest

from oracle import fp8, gemm, intquant as IQ, mx


def test_reference_product_matches_brute_force():
    rng = np.random.default_rng(31)
    a = rng.standard_normal((5, 96))
    w = rng.standard_normal((7, 96))
    assert np.allclose(gemm.reference_product(a, w), gemm.brute_force_product(a, w),
                       rtol=1e-13, atol=1e-13)
    # orientation: Y[m, n] = sum_k A[m, k] W[n, k]
    assert abs(gemm.reference_product(a, w)[2, 3] - sum(a[2] * w[3])) < 1e-12


def test_w4a16_reference_on_tiny_case_brute_force():
    rng = np.random.default_rng(32)
    w = (rng.standard_normal((6, 256)) * 0.02).astype(np.float32)
    x = rng.standard_normal((3, 256)).astype(np.float32)
    for asym in (False, True):
        if asym:
            q, s, z = IQ.quantize_asym(w, 128)
        else:
            (q, s), z = IQ.quantize_sym(w, 128), None
        packed = IQ.pack_int4(q)
        y = gemm.w4a16_reference(x, packed, s, z, 128)
        # brute force from the codes, written per group with the cross term
        yb = np.zeros((3, 6))
        for mi in range(3):
            for n in range(6):
                acc = 0.0
                for g in range(2):
                    sl = slice(128 * g, 128 * (g + 1))
                    sg = float(s[n, g])
                    zg = 0.0 if z is None else float(z[n, g])
                    xq = sum(float(a) * float(b) for a, b in zip(x[mi, sl], q[n, sl]))
                    acc += sg * (xq - zg * float(np.sum(x[mi, sl].astype(np.float64))))
                yb[mi, n] = acc
        assert np.allclose(y, yb, rtol=1e-12, atol=1e-12)


def test_constant_operands_closed_form():
    # all x = a, all w = b (an on-grid value) -> Y = K * a * b exactly
    k = 512
    x = np.full((2, k), 0.75, dtype=np.float32)
    w = np.full((3, k), 0.5, dtype=np.float32)
    q, s = IQ.quantize_sym(w, 128)
    y = gemm.w4a16_reference(x, IQ.pack_int4(q), s, None, 128)
    # scale fp16(0.5/7); q = 7 -> w_hat = 7 * fp16(0.5/7)
    w_hat = 7 * float(s[0, 0])
    assert np.allclose(y, k * 0.75 * w_hat, rtol=0, atol=1e-12)
    # MX: x = 1.5 and w = -3 are on-grid after scaling -> exact
    pa, ea = mx.quantize(np.full((2, 64), 1.5, np.float32))
    pb, eb = mx.quantize(np.full((3, 64), -3.0, np.float32))
    assert (gemm.mx_reference(pa, ea, pb, eb) == 64 * 1.5 * -3.0).all()


def test_one_hot_rows_select_dequantized_columns():
    rng = np.random.default_rng(33)
    w = (rng.standard_normal((9, 256)) * 0.02).astype(np.float32)
    q, s, z = IQ.quantize_asym(w, 128)
    x = np.eye(256, dtype=np.float32)[[0, 5, 130, 255]]
    y = gemm.w4a16_reference(x, IQ.pack_int4(q), s, z, 128)
    w_hat = IQ.dequantize(q, s, z, 128)
    assert (y == w_hat[:, [0, 5, 130, 255]].T).all()


def test_fp8_and_int8_references_use_both_scales():
    rng = np.random.default_rng(34)
    x = rng.standard_normal((4, 64)).astype(np.float32)
    w = (rng.standard_normal((5, 64)) * 0.02).astype(np.float32)
    xq, sx = fp8.quantize_rows(x)
    wq, sw = fp8.quantize_rows(w)
    y = gemm.fp8_reference(xq, sx, wq, sw)
    assert gemm.rel_fro(y, x.astype(np.float64) @ w.T.astype(np.float64)) < 0.05
    qx, sxi, zx = IQ.quantize_asym(x, 64, "int8_asym")
    qw, swi = IQ.quantize_sym(w, 64, "int8_sym")
    y8 = gemm.int8_reference(qx, sxi, zx, qw, swi, None)
    yb = gemm.brute_force_product(IQ.dequantize(qx, sxi, zx, 64), IQ.dequantize(qw, swi, None, 64))
    assert np.allclose(y8, yb, rtol=1e-12, atol=1e-12)
    assert gemm.rel_fro(y8, x.astype(np.float64) @ w.T.astype(np.float64)) < 0.02


def test_rel_fro_metric():
    y = np.array([[3.0, 4.0]])
    assert gemm.rel_fro(y, y) == 0.0
    assert abs(gemm.rel_fro(y * 1.001, y) - 0.001) < 1e-12
    assert abs(gemm.rel_fro(np.array([[3.0, 0.0]]), y) - 0.8) < 1e-12


# ------------------------------------------------------------------ SwiGLU

def test_silu_matches_torch_and_limits():
    import torch
    g = np.linspace(-30.0, 30.0, 601)
    ref = torch.nn.functional.silu(torch.from_numpy(g)).numpy()
    assert np.allclose(gemm.silu(g), ref, rtol=1e-15, atol=1e-300)
    assert gemm.silu(np.array([0.0]))[0] == 0.0
    assert abs(gemm.silu(np.array([40.0]))[0] - 40.0) < 1e-12          # -> g for large g
    assert abs(gemm.silu(np.array([-40.0]))[0]) < 1e-15                 # -> 0 for very negative g


def test_swiglu_reference_is_gate_then_up():
    # tiny brute-force case: [W_gate; W_up] as one quantized [2I][K] matrix;
    # gate rows come first (a swapped split fails the comparison)
    rng = np.random.default_rng(3)
    i, k, m = 3, 128, 2
    w = (rng.standard_normal((2 * i, k)) * 0.05).astype(np.float32)
    x = rng.standard_normal((m, k)).astype(np.float32)
    q, s = IQ.quantize_sym(w, 128)
    packed = IQ.pack_int4(q)
    w_hat = IQ.dequantize(q, s, None, 128)
    y = gemm.brute_force_product(x, w_hat)
    gate, up = y[:, :i], y[:, i:]
    expect = gate / (1.0 + np.exp(-gate)) * up
    h = gemm.swiglu_reference(x, packed, s, None, 128)
    assert np.allclose(h, expect, rtol=1e-12, atol=1e-12)
    swapped = up / (1.0 + np.exp(-up)) * gate
    assert not np.allclose(h, swapped, rtol=1e-3)
    # channel selection picks the same columns
    assert np.allclose(gemm.swiglu_reference(x, packed, s, None, 128, channels=[2, 0]),
                       expect[:, [2, 0]], rtol=1e-12, atol=1e-12)


def test_parity_bound_rejects_a_missing_cross_term():
    # 《第 6 课：量化源码走读》 section 3: an asymmetric product that leaves out the
    # zero-point cross term is wrong.  Planted on the oracle side: at the
    # Llama-3-8B decode distributions (asymmetric INT4 g128, 1 % of the input
    # channels x20) the product without the term, or with every zero point
    # off by one, lies far outside the 2e-3 parity bound, while the exact
    # dequantized product rounded to bf16 stays inside it
    from synthetic import bf16_as_f32, small_case
    c = small_case(4, 1024, 96, seed=31, w_outlier=(0.01, 20.0))
    x = bf16_as_f32(c["x"]).astype(np.float64)
    q, s, z = IQ.quantize_asym(c["w"], 128)
    ref = x @ IQ.dequantize(q, s, z, 128).T
    no_cross = x @ IQ.dequantize(q, s, np.zeros_like(z), 128).T
    off_by_one = x @ IQ.dequantize(q, s, z + 1, 128).T
    import torch
    rounded = torch.from_numpy(ref).to(torch.bfloat16).double().numpy()
    assert gemm.rel_fro(rounded, ref) <= 2e-3
    assert gemm.rel_fro(no_cross, ref) > 100 * 2e-3
    assert gemm.rel_fro(off_by_one, ref) > 2e-3


def test_fp8_swiglu_reference_brute_force():
    # tiny case against a pure-Python evaluation of the definition: decode
    # every E4M3 code from its bit fields, rescale by s_x s_w, sum, then
    # SiLU(gate) * up with the gate rows first (a swapped split, or the
    # scales left out, fails the comparison)
    import math
    from oracle import fp8 as F8
    rng = np.random.default_rng(12)
    m, k, i = 2, 64, 3
    x = rng.standard_normal((m, k)).astype(np.float32)
    w = (rng.standard_normal((2 * i, k)) * 0.05).astype(np.float32)
    xq, sx = F8.quantize_rows(x)
    wq, sw = F8.quantize_rows(w)

    def dec(c):
        c = int(c)
        e, f = (c >> 3) & 15, c & 7
        mag = (8 + f) * 2.0 ** (e - 10) if e else f * 2.0 ** -9
        return -mag if c & 0x80 else mag

    sxv, swv = np.asarray(sx).reshape(-1), np.asarray(sw).reshape(-1)
    y = [[sum(dec(xq[a, t]) * dec(wq[b, t]) for t in range(k)) * float(sxv[a]) * float(swv[b])
          for b in range(2 * i)] for a in range(m)]
    expect = np.array([[y[a][c] / (1.0 + math.exp(-y[a][c])) * y[a][c + i] for c in range(i)]
                       for a in range(m)])
    h = gemm.fp8_swiglu_reference(xq, sx, wq, sw)
    assert np.allclose(h, expect, rtol=1e-12, atol=1e-14)
    swapped = np.array([[y[a][c + i] / (1.0 + math.exp(-y[a][c + i])) * y[a][c] for c in range(i)]
                        for a in range(m)])
    assert not np.allclose(h, swapped, rtol=1e-3)
    unscaled = gemm.fp8_swiglu_reference(xq, np.ones_like(sxv), wq, np.ones_like(swv))
    assert not np.allclose(h, unscaled, rtol=1e-3)
    assert np.allclose(gemm.fp8_swiglu_reference(xq, sx, wq, sw, channels=[1]), expect[:, [1]],
                       rtol=1e-12, atol=1e-14)
    with pytest.raises(ValueError):
        gemm.fp8_swiglu_reference(xq, sx, wq[:5], sw[:5])
