"""GPU parity of the W4A16 decode GEMV against the oracle's fp64 product of
the dequantized operands: relative Frobenius error <= 2e-3, no NaN/Inf,
bit-exact codes, and a one-hot layout pin (each output equals the bf16
rounding of one dequantized weight)."""

import numpy as np
import pytest
import torch

import quantized_gemm_group_amd as qg
from oracle import formats as of, gemm as og, intquant as oi
from synthetic import WORKLOADS, bf16_as_f32, rng_for, small_case, to_bf16, workload_case
from tests.gpu_util import cosine, device, finite_checks, host, to_dev

pytestmark = pytest.mark.gpu

TOL = 2e-3


def oracle_weights(w, asym):
    if asym:
        q, s, z = oi.quantize_asym(w, 128, "int4_asym")
    else:
        (q, s), z = oi.quantize_sym(w, 128, "int4_sym"), None
    return oi.pack_int4(q), s, z


def run_case(m, k, n, asym, seed, outliers=(0.01, 20.0)):
    dev = device()
    c = small_case(m, k, n, seed, w_outlier=outliers)
    fmt = "int4_asym" if asym else "int4_sym"
    print(f"qgemv m={m} k={k} n={n} fmt={fmt} seed={seed}", flush=True)
    codes, scales, zeros = qg.quantize_pack(to_dev(c["w"], dev), fmt, 128)
    packed, s, z = oracle_weights(c["w"], asym)
    assert (host(codes) == packed).all()
    y = host(qg.qgemv(to_dev(c["x"], dev), codes, scales, zeros, fmt))
    # the tiled-code kernels run the same arithmetic in the same order
    yt = host(qg.qgemv_tiled(to_dev(c["x"], dev), qg.tile_gemv_weights(codes), scales, zeros, fmt))
    assert (yt.view(np.uint32) == y.view(np.uint32)).all(), "tiled GEMV differs from canonical"
    ref = og.w4a16_reference(bf16_as_f32(c["x"]), packed, s, z, 128)
    finite_checks(y)
    if y.size < 1024:      # too few outputs for the statistical bar: per-element bound
        floor = 1e-3 * np.sqrt(np.mean(ref ** 2))
        assert (np.abs(y - ref) <= 2.0 ** -8 * np.abs(ref) + floor).all()
        return 0.0
    err = og.rel_fro(y, ref)
    assert err <= TOL, f"rel_fro {err}"
    assert cosine(y, ref) > 0.99
    return err


@pytest.mark.parametrize("asym", [False, True])
@pytest.mark.parametrize("m,k,n", [(1, 128, 64), (1, 1024, 200), (3, 1024, 200), (4, 4096, 1000),
                                   (16, 2048, 333), (7, 14336, 96), (16, 640, 48),
                                   # per-wave kernel: 16 groups per wave (K = 18432), 14 K-slices,
                                   # 4 groups per wave (G = 4, 12), M = 2 in the 4-row layout
                                   (1, 18432, 40), (2, 14336, 70), (4, 512, 33), (1, 1536, 17),
                                   # 5..16 rows: 16 groups per wave (G = 144), two channel tiles
                                   # per wave with a ragged last tile, 4 groups per wave (G = 12)
                                   (9, 18432, 50), (12, 1024, 16400), (5, 1536, 77),
                                   # 5..16 rows, x staged in LDS: 2 tiles per workgroup with a
                                   # one-tile last workgroup, 3 tiles on 4 tile-lanes, one
                                   # K-slice, 3 units per wave
                                   (5, 4096, 4100), (13, 512, 8200), (8, 256, 40),
                                   (6, 1024, 40000),
                                   # 3 and 4 rows, x staged in LDS (4 or more tiles per
                                   # workgroup, ragged last tile); 4 rows with 2 tiles per
                                   # workgroup stay on the per-wave kernel
                                   (4, 1024, 16400), (3, 512, 20008), (4, 2048, 6150)])
def test_qgemv_small(m, k, n, asym):
    run_case(m, k, n, asym, seed=m * 1000 + n)


def test_qgemv_ragged_single_row():
    run_case(1, 256, 1, True, seed=3)
    run_case(2, 256, 17, False, seed=4)


@pytest.mark.parametrize("asym", [False, True])
def test_qgemv_one_hot_is_bit_exact(asym):
    # x rows are unit vectors e_k: y[m][n] = bf16(w_hat[n][k_m]) exactly
    dev = device()
    k, n = 1024, 80
    w = (rng_for(9).standard_normal((n, k), dtype=np.float32) * np.float32(0.02))
    fmt = "int4_asym" if asym else "int4_sym"
    codes, scales, zeros = qg.quantize_pack(to_dev(w, dev), fmt, 128)
    packed, s, z = oracle_weights(w, asym)
    ks = [0, 1, 7, 8, 127, 128, 300, 1023, 513, 64, 65, 1000, 5, 6, 900, 777]
    x = np.zeros((16, k), np.float32)
    x[np.arange(16), ks] = 1.0
    y = host(qg.qgemv(to_dev(to_bf16(x), dev), codes, scales, zeros, fmt))
    yt = host(qg.qgemv_tiled(to_dev(to_bf16(x), dev), qg.tile_gemv_weights(codes), scales, zeros,
                             fmt))
    q = oi.unpack_int4(packed, signed=not asym)
    w_hat = oi.dequantize(q, s, z, 128, out="f32")
    expect = of.round_to_bf16(w_hat[:, ks].T)
    assert (y.view(np.uint32) == expect.view(np.uint32)).all()
    assert (yt.view(np.uint32) == expect.view(np.uint32)).all()


@pytest.mark.parametrize("n,k", [(16, 128), (37, 384), (5, 1024), (1000, 4096)])
def test_tile_gemv_weights_layout(n, k):
    # the tiled layout of the header, written out with numpy: block (t, g) of
    # 1 KiB holds rows 16t .. 16t+15, bytes 64g .. 64g+63 of each, quarter by
    # quarter (16 bytes of each of the 16 rows, then the next 16), zero rows
    # past N
    dev = device()
    codes = rng_for(n + k).integers(-2 ** 31, 2 ** 31, size=(n, k // 8), dtype=np.int64)
    codes = codes.astype(np.int32)
    got = host(qg.tile_gemv_weights(to_dev(codes, dev)).data)
    tiles, g = (n + 15) // 16, k // 128
    rows = np.zeros((tiles * 16, k // 2), np.uint8)
    rows[:n] = codes.view(np.uint8).reshape(n, k // 2)
    want = rows.reshape(tiles, 16, g, 4, 16).transpose(0, 2, 3, 1, 4).reshape(-1)
    assert got.shape == want.shape and (got == want).all()


def test_qgemv_gemv_4096_full():
    dev = device()
    c = workload_case("gemv_4096")
    print("qgemv gemv_4096 M=1 K=N=4096 int4_sym", flush=True)
    codes, scales, _ = qg.quantize_pack(to_dev(c["w"], dev), "int4_sym", 128)
    packed, s, _ = oracle_weights(c["w"], False)
    assert (host(codes) == packed).all()
    assert (host(scales).view(np.uint16) == s.view(np.uint16)).all()
    x = c["x"][:1]
    y = host(qg.qgemv(to_dev(x, dev), codes, scales, None, "int4_sym"))
    yt = host(qg.qgemv_tiled(to_dev(x, dev), qg.tile_gemv_weights(codes), scales, None,
                             "int4_sym"))
    assert (yt.view(np.uint32) == y.view(np.uint32)).all()
    ref = og.w4a16_reference(bf16_as_f32(x), packed, s, None, 128)
    finite_checks(y)
    assert og.rel_fro(y, ref) <= TOL


@pytest.mark.parametrize("proj", range(4))
def test_qgemv_llama3_8b_decode_sampled(proj):
    # full-size shapes, all three batch sizes; codes and outputs checked on
    # sampled output channels (the oracle quantizes those rows itself)
    dev = device()
    c = workload_case("llama3_8b_decode", proj)
    n, k = c["n"], c["k"]
    print(f"qgemv llama3_8b_decode {c['name']} K={k} N={n}", flush=True)
    codes, scales, zeros = qg.quantize_pack(to_dev(c["w"], dev), "int4_asym", 128)
    rng = np.random.default_rng(proj)
    rows = np.unique(np.concatenate([np.arange(16), np.arange(n - 16, n),
                                     rng.choice(n, 160, replace=False)]))
    packed, s, z = oracle_weights(c["w"][rows], True)
    assert (host(codes)[rows] == packed).all()
    assert (host(scales)[rows].view(np.uint16) == s.view(np.uint16)).all()
    assert (host(zeros)[rows].view(np.uint16) == z.view(np.uint16)).all()
    xs = bf16_as_f32(c["x"])
    tiled = qg.tile_gemv_weights(codes)
    for m in WORKLOADS["llama3_8b_decode"].ms:
        y = host(qg.qgemv(to_dev(c["x"][:m], dev), codes, scales, zeros, "int4_asym"))
        yt = host(qg.qgemv_tiled(to_dev(c["x"][:m], dev), tiled, scales, zeros, "int4_asym"))
        assert (yt.view(np.uint32) == y.view(np.uint32)).all(), f"M={m} tiled differs"
        finite_checks(y)
        ref = og.w4a16_reference(xs[:m], packed, s, z, 128)
        err = og.rel_fro(y[:, rows], ref)
        assert err <= TOL, f"M={m} rel_fro {err}"



# ------------------------------------------------ group sizes other than 128

@pytest.mark.parametrize("asym", [False, True])
@pytest.mark.parametrize("group", [32, 64, 256, 1024])
@pytest.mark.parametrize("m,k,n", [(1, 1024, 100), (4, 2048, 37), (16, 4096, 64), (7, 1024, 300)])
def test_qgemv_other_group_sizes(m, k, n, group, asym):
    # 《第 1 章：推理加速全景》 section 4.1: per-group granularity from 32 to 128
    # (and coarser); the codes, scales and zero points of quantize_pack with
    # the group, the GEMV on canonical and tiled codes against the oracle
    dev = device()
    fmt = "int4_asym" if asym else "int4_sym"
    print(f"qgemv group={group} m={m} k={k} n={n} {fmt}", flush=True)
    c = small_case(m, k, n, seed=group + m + n, w_outlier=(0.01, 20.0))
    codes, scales, zeros = qg.quantize_pack(to_dev(c["w"], dev), fmt, group)
    if asym:
        q, s, z = oi.quantize_asym(c["w"], group, "int4_asym")
    else:
        (q, s), z = oi.quantize_sym(c["w"], group, "int4_sym"), None
    packed = oi.pack_int4(q)
    assert (host(codes) == packed).all()
    assert (host(scales).view(np.uint16) == s.view(np.uint16)).all()
    x = to_dev(c["x"], dev)
    y = host(qg.qgemv(x, codes, scales, zeros, fmt, group=group))
    yt = host(qg.qgemv_tiled(x, qg.tile_gemv_weights(codes), scales, zeros, fmt, group=group))
    assert (yt.view(np.uint32) == y.view(np.uint32)).all()
    ref = og.w4a16_reference(bf16_as_f32(c["x"]), packed, s, z, group)
    finite_checks(y)
    if y.size < 1024:
        floor = 1e-3 * np.sqrt(np.mean(ref ** 2))
        assert (np.abs(y - ref) <= 2.0 ** -8 * np.abs(ref) + floor).all()
    else:
        assert og.rel_fro(y, ref) <= TOL


def test_group_32_one_hot_is_bit_exact():
    # the natural-order unpack of the other-group kernel: x rows e_k select
    # one dequantized weight (groups of 32, asymmetric)
    dev = device()
    k, n = 512, 48
    w = (rng_for(19).standard_normal((n, k), dtype=np.float32) * np.float32(0.02))
    codes, scales, zeros = qg.quantize_pack(to_dev(w, dev), "int4_asym", 32)
    q, s, z = oi.quantize_asym(w, 32, "int4_asym")
    ks = [0, 1, 7, 8, 31, 32, 33, 63, 64, 100, 127, 128, 200, 300, 450, 511]
    x = np.zeros((16, k), np.float32)
    x[np.arange(16), ks] = 1.0
    y = host(qg.qgemv(to_dev(to_bf16(x), dev), codes, scales, zeros, "int4_asym", group=32))
    w_hat = oi.dequantize(oi.unpack_int4(oi.pack_int4(q), signed=False), s, z, 32, out="f32")
    expect = of.round_to_bf16(w_hat[:, ks].T)
    assert (y == expect).all()
