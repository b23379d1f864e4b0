"""GPU parity of the quantized GEMMs against the oracle's fp64 product of the
dequantized operands (relative Frobenius error <= 2e-3, no NaN/Inf), with
bit-exact operand codes: FP8 W8A8 with dynamic per-token activation scales,
MXFP4 W4A4, INT8 W8A8 (symmetric/asymmetric pairs) and the W4A16 prefill
GEMM.  Small cases span several tiles with ragged M/N/K tails; the full-size
workloads are checked on sampled rows (the oracle quantizes those rows of the
seeded inputs itself)."""

import numpy as np
import pytest
import torch

import quantized_gemm_group_amd as qg
from oracle import formats as of, fp8 as of8, gemm as og, intquant as oi, mx as omx
from synthetic import (bf16_as_f32, rng_for, small_case, to_bf16, workload_case,
                       normal_activations, normal_weights, scale_input_channels,
                       scale_random_entries)
from tests.gpu_util import cosine, device, finite_checks, host, to_dev

pytestmark = pytest.mark.gpu

TOL = 2e-3


def check(y, ref, what):
    """rel. Frobenius <= 2e-3 (the bar, statistical: dominated by the bf16
    output rounding, rms ~1.7e-3 of a value); outputs too few for that
    average to settle (< 1024) get the stronger per-element bound instead:
    within one bf16 step (2^-8 relative) of the exact value, plus a small
    absolute floor for fp32 accumulation on near-cancelling sums."""
    finite_checks(y)
    if y.size < 1024:
        floor = 1e-3 * np.sqrt(np.mean(ref.astype(np.float64) ** 2))
        bad = np.abs(y - ref) > 2.0 ** -8 * np.abs(ref) + floor
        assert not bad.any(), f"{what}: {bad.sum()} outputs beyond one bf16 step"
        return 0.0
    err = og.rel_fro(y, ref)
    assert err <= TOL, f"{what}: rel_fro {err}"
    assert cosine(y, ref) > 0.99
    return err


# ----------------------------------------------------------------------- FP8

def fp8_case(m, k, n, seed):
    c = small_case(m, k, n, seed, x_outlier=(0.001, 100.0))
    return c["w"], c["x"]


# K a multiple of 64 (whole k-steps; 1, 3 and 5 of them leave the last pair
# of k-steps half empty) and K = 48, 176, 1040 (a last k-step of 3, 3 and 1
# of its four 16-byte chunks)
@pytest.mark.parametrize("m,k,n", [(64, 256, 80), (130, 512, 200), (257, 1040, 129), (1, 128, 16),
                                   (300, 2048, 384), (40, 48, 72), (100, 176, 96), (5, 64, 24),
                                   (70, 192, 136), (300, 320, 264)])
def test_fp8_gemm_small(m, k, n):
    dev = device()
    w, x = fp8_case(m, k, n, seed=m + n + k)
    print(f"fp8 gemm m={m} k={k} n={n}", flush=True)
    xq, sx, _ = qg.quantize_pack(to_dev(x, dev), "fp8_e4m3")
    wq, sw, _ = qg.quantize_pack(to_dev(w, dev), "fp8_e4m3")
    oxq, osx = of8.quantize_rows(bf16_as_f32(x))
    owq, osw = of8.quantize_rows(w)
    assert (host(xq) == oxq).all() and (host(wq) == owq).all()
    y = host(qg.qgemm(xq, wq, sw, None, "fp8_e4m3", "fp8_e4m3", a_scales=sx))
    check(y, og.fp8_reference(oxq, osx, owq, osw), "fp8")


def _sample_rows(n, count, seed, tile=256):
    """Sampled output rows (or columns) of a full-size product: the first and
    last 8, one at random inside every `tile`-wide block (so every 256 x 256
    workgroup tile of the output, and with it every XCD and tile-order slot,
    is looked at), and `count` more at random."""
    rng = np.random.default_rng(seed)
    per_tile = np.array([t + rng.integers(0, min(tile, n - t)) for t in range(0, n, tile)])
    return np.unique(np.concatenate([np.arange(8), np.arange(n - 8, n), per_tile,
                                     rng.choice(n, count, replace=False)]))


def test_fp8_gemm_8192_sampled():
    dev = device()
    c = workload_case("fp8_8192")
    print("fp8 gemm M=N=K=8192", flush=True)
    xq, sx, _ = qg.quantize_pack(to_dev(c["x"], dev), "fp8_e4m3")
    wq, sw, _ = qg.quantize_pack(to_dev(c["w"], dev), "fp8_e4m3")
    y = host(qg.qgemm(xq, wq, sw, None, "fp8_e4m3", "fp8_e4m3", a_scales=sx))
    rm, rn = _sample_rows(8192, 24, 1), _sample_rows(8192, 24, 2)
    oxq, osx = of8.quantize_rows(bf16_as_f32(c["x"][rm]))
    owq, osw = of8.quantize_rows(c["w"][rn])
    assert (host(xq)[rm] == oxq).all() and (host(sx)[rm, 0] == osx).all()
    assert (host(wq)[rn] == owq).all() and (host(sw)[rn, 0] == osw).all()
    check(y[np.ix_(rm, rn)], og.fp8_reference(oxq, osx, owq, osw), "fp8 8192")


# ---------------------------------------------------------------------- MXFP4

# K a multiple of 128 (one aligned exponent dword per row and k-step of 128
# codes) with 1 to 6, 11 and 32 k-steps, odd and even step counts included;
# K = 32 and 1056 load each k-step's exponents byte by byte
@pytest.mark.parametrize("m,k,n", [(64, 256, 64), (130, 512, 200), (33, 1056, 129), (1, 32, 16),
                                   (256, 4096, 260), (96, 128, 72), (70, 384, 300),
                                   (257, 640, 64), (128, 768, 520), (40, 1408, 96)])
def test_mx_gemm_small(m, k, n):
    dev = device()
    c = small_case(m, k, n, seed=3 * m + n, w_outlier=(0.01, 50.0))
    print(f"mx gemm m={m} k={k} n={n}", flush=True)
    ac, ae = qg.mx_quant(to_dev(c["x"], dev))
    bc, be = qg.mx_quant(to_dev(c["w"], dev))
    oac, oae = omx.quantize(bf16_as_f32(c["x"]))
    obc, obe = omx.quantize(c["w"])
    assert (host(ac) == oac).all() and (host(ae) == oae).all()
    assert (host(bc) == obc).all() and (host(be) == obe).all()
    y = host(qg.mx_gemm(ac, ae, bc, be))
    check(y, og.mx_reference(oac, oae, obc, obe), "mx")


def test_mx_gemm_4096x8192_sampled():
    dev = device()
    c = workload_case("mxfp4_4096x8192")
    print("mx gemm M=4096 N=K=8192", flush=True)
    ac, ae = qg.mx_quant(to_dev(c["x"], dev))
    bc, be = qg.mx_quant(to_dev(c["w"], dev))
    y = host(qg.mx_gemm(ac, ae, bc, be))
    rm, rn = _sample_rows(4096, 24, 3), _sample_rows(8192, 24, 4)
    oac, oae = omx.quantize(bf16_as_f32(c["x"][rm]))
    obc, obe = omx.quantize(c["w"][rn])
    assert (host(ac)[rm] == oac).all() and (host(ae)[rm] == oae).all()
    assert (host(bc)[rn] == obc).all() and (host(be)[rn] == obe).all()
    check(y[np.ix_(rm, rn)], og.mx_reference(oac, oae, obc, obe), "mx 4096x8192")


# ----------------------------------------------------------------------- INT8

def _int8_oracle(v, fmt):
    k = v.shape[1]
    if fmt == "int8_sym":
        q, s = oi.quantize_sym(v, k, "int8_sym")
        return q.astype(np.int8), s, None
    q, s, z = oi.quantize_asym(v, k, "int8_asym")
    return q.astype(np.uint8), s, z


@pytest.mark.parametrize("afmt", ["int8_sym", "int8_asym"])
@pytest.mark.parametrize("wfmt", ["int8_sym", "int8_asym"])
@pytest.mark.parametrize("m,k,n", [(64, 256, 80), (130, 1040, 200)])
def test_int8_gemm(m, k, n, afmt, wfmt):
    dev = device()
    c = small_case(m, k, n, seed=m * 7 + n, x_outlier=(0.001, 100.0))
    x = bf16_as_f32(c["x"])
    if afmt == "int8_asym":
        x = x + np.float32(0.75)              # a shifted activation distribution
        x = bf16_as_f32(to_bf16(x))
    print(f"int8 gemm m={m} k={k} n={n} a={afmt} w={wfmt}", flush=True)
    aq, as_, az = qg.quantize_pack(to_dev(to_bf16(x), dev), afmt)
    wq, ws, wz = qg.quantize_pack(to_dev(c["w"], dev), wfmt)
    oaq, oas, oaz = _int8_oracle(x, afmt)
    owq, ows, owz = _int8_oracle(c["w"], wfmt)
    assert (host(aq) == oaq).all() and (host(wq) == owq).all()
    y = host(qg.qgemm(aq, wq, ws, wz, wfmt, afmt, a_scales=as_, a_zeros=az))
    ref = og.int8_reference(oaq.astype(np.int64), oas, oaz, owq.astype(np.int64), ows, owz)
    check(y, ref, f"int8 {afmt}/{wfmt}")


def test_int8_gemm_4096_sampled():
    dev = device()
    rng = rng_for(44)
    w = normal_weights(rng, 4096, 4096)
    x = normal_activations(rng, 4096, 4096)
    scale_random_entries(rng, x, 0.001, 100.0)
    xb = to_bf16(x)
    print("int8 gemm M=N=K=4096 asym activations, sym weights", flush=True)
    aq, as_, az = qg.quantize_pack(to_dev(xb, dev), "int8_asym")
    wq, ws, _ = qg.quantize_pack(to_dev(w, dev), "int8_sym")
    y = host(qg.qgemm(aq, wq, ws, None, "int8_sym", "int8_asym", a_scales=as_, a_zeros=az))
    rm, rn = _sample_rows(4096, 24, 5), _sample_rows(4096, 24, 6)
    oaq, oas, oaz = _int8_oracle(bf16_as_f32(xb[rm]), "int8_asym")
    owq, ows, _ = _int8_oracle(w[rn], "int8_sym")
    assert (host(aq)[rm] == oaq).all() and (host(wq)[rn] == owq).all()
    ref = og.int8_reference(oaq.astype(np.int64), oas, oaz, owq.astype(np.int64), ows, None)
    check(y[np.ix_(rm, rn)], ref, "int8 4096")


@pytest.mark.parametrize("fmt", ["int8_sym", "int8_asym"])
def test_int8_gemm_long_k_stays_exact(fmt):
    # K = 262144 with constant extreme codes: the product sums reach 2^32,
    # past int32 (one int32 run may hold 512 k-blocks of 128; the kernel
    # folds longer sums into fp64)
    dev = device()
    k = 262144
    rng = rng_for(45)
    if fmt == "int8_sym":
        lo, hi, dt = -127, 127, np.int8
        a = np.stack([np.full(k, lo), rng.integers(lo, hi + 1, k), np.full(k, hi)]).astype(dt)
        w = np.stack([np.full(k, lo), np.full(k, hi), rng.integers(lo, hi + 1, k),
                      np.where(np.arange(k) % 2 == 0, lo, hi)]).astype(dt)
        az = wz = None
    else:
        lo, hi, dt = 0, 255, np.uint8
        a = np.stack([np.full(k, lo), rng.integers(lo, hi + 1, k), np.full(k, hi)]).astype(dt)
        w = np.stack([np.full(k, lo), np.full(k, hi), rng.integers(lo, hi + 1, k),
                      np.where(np.arange(k) % 2 == 0, lo, hi)]).astype(dt)
        az = np.array([255.0, 128.0, 0.0], dtype=np.float32)
        wz = np.array([255.0, 0.0, 100.0, 7.0], dtype=np.float32)
    a_s = np.array([1.0 / 127, 2.0 ** -10, 3.0e-3], dtype=np.float32)
    w_s = np.array([2.0 ** -12, 1.0 / 255, 5.0e-4, 2.0 ** -9], dtype=np.float32)
    print(f"int8 gemm long K={k} {fmt}", flush=True)
    t = lambda v: to_dev(v, dev)
    y = host(qg.qgemm(t(a), t(w), t(w_s), None if wz is None else t(wz), fmt, fmt,
                      a_scales=t(a_s), a_zeros=None if az is None else t(az)))
    ref = og.int8_reference(a.astype(np.int64), a_s, az, w.astype(np.int64), w_s, wz)
    # the constant rows' exact products (e.g. 262144 * 127^2 > 2^31) are
    # what a wrapped int32 sum would get wrong
    assert abs(ref[0, 0]) > 1.0
    check(y, ref, f"int8 long K {fmt}")


# --------------------------------------------------------------- W4A16 prefill

# groups of 128 per row G = 1, 2, 3, 5, 7, 8, 11, 12, 16: the k-loop runs in
# unrolled blocks of 6 groups, then pairs, then a single group
@pytest.mark.parametrize("asym", [False, True])
@pytest.mark.parametrize("m,k,n", [(64, 256, 80), (200, 1024, 136), (1, 128, 16), (300, 2048, 520),
                                   (130, 384, 300), (70, 640, 260), (96, 896, 72),
                                   (33, 1408, 264), (140, 1536, 128)])
def test_w4a16_gemm_small(m, k, n, asym):
    dev = device()
    c = small_case(m, k, n, seed=m + 11 * n, w_outlier=(0.01, 20.0))
    fmt = "int4_asym" if asym else "int4_sym"
    print(f"w4a16 gemm m={m} k={k} n={n} {fmt}", flush=True)
    codes, scales, zeros = qg.quantize_pack(to_dev(c["w"], dev), fmt, 128)
    if asym:
        q, s, z = oi.quantize_asym(c["w"], 128)
    else:
        (q, s), z = oi.quantize_sym(c["w"], 128), None
    packed = oi.pack_int4(q)
    assert (host(codes) == packed).all()
    y = host(qg.qgemm(to_dev(c["x"], dev), codes, scales, zeros, fmt, "bf16"))
    check(y, og.w4a16_reference(bf16_as_f32(c["x"]), packed, s, z, 128), f"w4a16 {fmt}")


@pytest.mark.parametrize("asym", [False, True])
@pytest.mark.parametrize("k", [512, 640])      # 4 groups (paired scale loads), 5 groups (single)
def test_w4a16_gemm_last_wave_quarters(asym, k):
    # 3 x 90 = 270 tiles of 128 x 256: on a 256-CU GPU 256 whole tiles run
    # first and the last 14 as 32-token quarters (the last row tile is ragged,
    # 44 rows: one full and one partial quarter, two empty).  Against the
    # oracle, and bit for bit against each 128-row slice computed alone (one
    # partly filled wave, whole tiles): every output is the same arithmetic.
    dev = device()
    m, n = 300, 23040
    fmt = "int4_asym" if asym else "int4_sym"
    print(f"w4a16 gemm last-wave quarters m={m} k={k} n={n} {fmt}", flush=True)
    c = small_case(m, k, n, seed=5 + asym + k, w_outlier=(0.01, 20.0))
    codes, scales, zeros = qg.quantize_pack(to_dev(c["w"], dev), fmt, 128)
    if asym:
        q, s, z = oi.quantize_asym(c["w"], 128)
    else:
        (q, s), z = oi.quantize_sym(c["w"], 128), None
    packed = oi.pack_int4(q)
    x = to_dev(c["x"], dev)
    y = qg.qgemm(x, codes, scales, zeros, fmt, "bf16")
    check(host(y), og.w4a16_reference(bf16_as_f32(c["x"]), packed, s, z, 128), f"w4a16 {fmt}")
    for r0 in (0, 128, 256):
        part = qg.qgemm(x[r0:r0 + 128].contiguous(), codes, scales, zeros, fmt, "bf16")
        assert torch.equal(part.view(torch.int16), y[r0:r0 + 128].view(torch.int16)), r0


@pytest.mark.parametrize("asym", [False, True])
@pytest.mark.parametrize("group", [32, 64, 256])
@pytest.mark.parametrize("m,k,n", [(130, 1024, 200), (33, 2048, 72)])
def test_w4a16_gemm_other_group_sizes(m, k, n, group, asym):
    # groups other than 128 (《第 1 章：推理加速全景》 section 4.1 granularity)
    dev = device()
    fmt = "int4_asym" if asym else "int4_sym"
    print(f"w4a16 gemm group={group} m={m} k={k} n={n} {fmt}", flush=True)
    c = small_case(m, k, n, seed=group + 3 * m + n, w_outlier=(0.01, 20.0))
    codes, scales, zeros = qg.quantize_pack(to_dev(c["w"], dev), fmt, group)
    if asym:
        q, s, z = oi.quantize_asym(c["w"], group)
    else:
        (q, s), z = oi.quantize_sym(c["w"], group), None
    packed = oi.pack_int4(q)
    assert (host(codes) == packed).all()
    y = host(qg.qgemm(to_dev(c["x"], dev), codes, scales, zeros, fmt, "bf16", group=group))
    check(y, og.w4a16_reference(bf16_as_f32(c["x"]), packed, s, z, group), f"w4a16 g{group}")


@pytest.mark.parametrize("proj", [0, 1])
def test_w4a16_prefill_qwen72b_sampled(proj):
    dev = device()
    c = workload_case("qwen72b_prefill", proj)
    print(f"w4a16 prefill {c['name']} M=2048 K={c['k']} N={c['n']}", flush=True)
    codes, scales, _ = qg.quantize_pack(to_dev(c["w"], dev), "int4_sym", 128)
    y = host(qg.qgemm(to_dev(c["x"], dev), codes, scales, None, "int4_sym", "bf16"))
    rm, rn = _sample_rows(2048, 24, 7 + proj), _sample_rows(c["n"], 24, 9 + proj)
    q, s = oi.quantize_sym(c["w"][rn], 128)
    packed = oi.pack_int4(q)
    assert (host(codes)[rn] == packed).all()
    assert (host(scales)[rn].view(np.uint16) == s.view(np.uint16)).all()
    ref = og.w4a16_reference(bf16_as_f32(c["x"][rm]), packed, s, None, 128)
    check(y[np.ix_(rm, rn)], ref, "w4a16 prefill")


def test_qgemm_format_pair_errors():
    dev = device()
    a = torch.zeros((4, 128), dtype=torch.uint8, device=dev)
    with pytest.raises(qg.QGError):
        qg.qgemm(a, a, torch.ones((4, 1), device=dev), None, "fp8_e4m3", "int8_sym",
                 a_scales=torch.ones((4, 1), device=dev))



# ------------------------------------------------------- layout pins (one-hot)
# Rows of A that are unit vectors e_k select one dequantized weight each:
# y[m][n] = bf16(w_hat[n][k_m]) exactly (the products are exact and the sum
# has one nonzero term), so any slip in the operand layout, the nibble or
# byte order, the k mapping or the output placement shows up bit for bit.

_ONE_HOT_K = 1024


def _one_hot_positions(m, k, seed):
    # group and block edges, every nibble position of a word, and random ones
    fixed = [0, 1, 7, 8, 15, 16, 31, 32, 63, 64, 127, 128, 129, 255, 256, 511, 512, 1000, 1023]
    rng = np.random.default_rng(seed)
    return np.concatenate([fixed, rng.integers(0, k, m - len(fixed))]).astype(np.int64)


@pytest.mark.parametrize("asym", [False, True])
def test_w4a16_gemm_one_hot_is_bit_exact(asym):
    dev = device()
    m, k, n = 256, _ONE_HOT_K, 300
    w = (rng_for(21).standard_normal((n, k), dtype=np.float32) * np.float32(0.02))
    fmt = "int4_asym" if asym else "int4_sym"
    codes, scales, zeros = qg.quantize_pack(to_dev(w, dev), fmt, 128)
    if asym:
        q, s, z = oi.quantize_asym(w, 128)
    else:
        (q, s), z = oi.quantize_sym(w, 128), None
    ks = _one_hot_positions(m, k, 22)
    x = np.zeros((m, k), np.float32)
    x[np.arange(m), ks] = 1.0
    y = host(qg.qgemm(to_dev(to_bf16(x), dev), codes, scales, zeros, fmt, "bf16"))
    w_hat = oi.dequantize(oi.unpack_int4(oi.pack_int4(q), signed=not asym), s, z, 128, out="f32")
    expect = of.round_to_bf16(w_hat[:, ks].T)
    assert (y.view(np.uint32) == expect.view(np.uint32)).all()


def test_fp8_gemm_one_hot_is_bit_exact():
    # activation codes 0x38 (E4M3 1.0) at k_m with unit scales: the epilogue
    # forms dec(w) * s_w in fp32 and rounds it once to bf16
    dev = device()
    m, k, n = 256, _ONE_HOT_K, 300
    w = (rng_for(23).standard_normal((n, k), dtype=np.float32) * np.float32(0.02))
    wq, sw = of8.quantize_rows(w)
    ks = _one_hot_positions(m, k, 24)
    xq = np.zeros((m, k), np.uint8)
    xq[np.arange(m), ks] = 0x38
    sx = np.ones(m, np.float32)
    y = host(qg.qgemm(to_dev(xq, dev), to_dev(wq, dev), to_dev(np.asarray(sw, np.float32), dev),
                      None, "fp8_e4m3", "fp8_e4m3", a_scales=to_dev(sx, dev)))
    dec = of.decode(wq[:, ks].T, "e4m3").astype(np.float32)
    expect = of.round_to_bf16(dec * np.asarray(sw, np.float32)[None, :])
    # equal values (code 0x80 is -0; the matrix core's sum gives +0)
    assert np.isfinite(y).all() and (y == expect).all()


def test_mx_gemm_one_hot_is_bit_exact():
    # A holds one E2M1 1.0 (code 2) at k_m with exponent byte 127 in every
    # block: y[m][n] = bf16(e2m1(b[n][k_m]) * 2^(eb - 127)), exact
    dev = device()
    m, k, n = 256, _ONE_HOT_K, 300
    w = rng_for(25).standard_normal((n, k), dtype=np.float32) * np.float32(0.02)
    w[:, 5] *= np.float32(50)
    bc, be = omx.quantize(w)
    ks = _one_hot_positions(m, k, 26)
    nib = np.zeros((m, k), np.uint8)
    nib[np.arange(m), ks] = 2
    ac = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    ae = np.full((m, k // 32), 127, np.uint8)
    y = host(qg.mx_gemm(to_dev(ac, dev), to_dev(ae, dev), to_dev(bc, dev), to_dev(be, dev)))
    expect = of.round_to_bf16(omx.dequantize(bc, be)[:, ks].T.astype(np.float32))
    # equal values: E2M1 code 8 is -0, and the matrix core's sum 0 + 1 * (-0)
    # is +0; every nonzero output is compared bit for bit
    assert np.isfinite(y).all() and (y == expect).all()


def test_mx_gemm_on_edge_blocks():
    # MX operands with zero, fp32-subnormal, 6 * 2^k-edge and tie blocks (the
    # quantizer's edge matrix, with the huge block scaled to keep the
    # products finite) through the GEMM; zero rows give exact zeros
    from tests.test_gpu_quant import mx_edge_matrix
    dev = device()
    a = mx_edge_matrix(45, 2048, 5)
    a[5, :32] = np.float32(3e30) * np.sign(a[5, :32] + 0.5)
    w = mx_edge_matrix(70, 2048, 6)
    w[5, :32] = np.float32(1e-20)
    ac, ae = qg.mx_quant(to_dev(a, dev))
    bc, be = qg.mx_quant(to_dev(w, dev))
    oac, oae = omx.quantize(a)
    obc, obe = omx.quantize(w)
    assert (host(ac) == oac).all() and (host(ae) == oae).all()
    assert (host(bc) == obc).all() and (host(be) == obe).all()
    y = host(qg.mx_gemm(ac, ae, bc, be))
    ref = og.mx_reference(oac, oae, obc, obe)
    zero_rows = ~oac.any(axis=1)
    assert (y[zero_rows] == 0).all()
    check(y, ref, "mx edge blocks")


def test_fp8_gemm_with_zero_rows():
    # all-zero activation rows and weight rows take scale 1 (the zero-block
    # rule) and all-zero codes; their outputs are exactly zero
    dev = device()
    w, x = fp8_case(130, 512, 200, seed=77)
    x = bf16_as_f32(x)
    x[[0, 17, 129]] = 0.0
    w[[3, 199]] = 0.0
    xq, sx, _ = qg.quantize_pack(to_dev(to_bf16(x), dev), "fp8_e4m3")
    wq, sw, _ = qg.quantize_pack(to_dev(w, dev), "fp8_e4m3")
    oxq, osx = of8.quantize_rows(x)
    owq, osw = of8.quantize_rows(w)
    assert (host(xq) == oxq).all() and (host(wq) == owq).all()
    assert (host(sx).reshape(-1) == np.asarray(osx).reshape(-1)).all()
    assert host(sx).reshape(-1)[0] == 1.0 and host(sw).reshape(-1)[3] == 1.0
    y = host(qg.qgemm(xq, wq, sw, None, "fp8_e4m3", "fp8_e4m3", a_scales=sx))
    assert (y[[0, 17, 129]] == 0).all() and (y[:, [3, 199]] == 0).all()
    check(y, og.fp8_reference(oxq, osx, owq, osw), "fp8 zero rows")
