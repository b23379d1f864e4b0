"""GPU parity of the fused SwiGLU projection (qg_qgemm_swiglu): one W4A16
GEMM over the quantized concatenation [W_gate; W_up] with SiLU(gate) * up in
the epilogue, against the oracle's float64 reference (relative Frobenius
error <= 2e-3), on ragged shapes and on the Qwen2.5-72B FFN gate+up shape
(the 29568 weight rows are gate and up of 14784 channels) on sampled
channels; and against the unfused path (the plain GEMM, then SiLU * up)."""

import numpy as np
import pytest
import torch

import quantized_gemm_group_amd as qg
from oracle import gemm as og, intquant as oi
from synthetic import bf16_as_f32, rng_for, small_case, workload_case
from tests.gpu_util import cosine, device, finite_checks, host, to_dev

pytestmark = pytest.mark.gpu

TOL = 2e-3


def check(h, ref, what):
    finite_checks(h)
    err = og.rel_fro(h, ref)
    assert err <= TOL, f"{what}: rel_fro {err}"
    assert cosine(h, ref) > 0.999
    return err


@pytest.mark.parametrize("asym", [False, True])
@pytest.mark.parametrize("m,k,i", [(64, 256, 40), (200, 1024, 136), (1, 128, 8), (130, 384, 300),
                                   (300, 2048, 520), (96, 896, 72), (40, 1408, 136)])
def test_swiglu_small(m, k, i, asym):
    dev = device()
    fmt = "int4_asym" if asym else "int4_sym"
    print(f"swiglu m={m} k={k} I={i} {fmt}", flush=True)
    c = small_case(m, k, 2 * i, seed=m + 13 * i, w_outlier=(0.01, 20.0))
    codes, scales, zeros = qg.quantize_pack(to_dev(c["w"], dev), fmt, 128)
    if asym:
        q, s, z = oi.quantize_asym(c["w"], 128)
    else:
        (q, s), z = oi.quantize_sym(c["w"], 128), None
    packed = oi.pack_int4(q)
    assert (host(codes) == packed).all()
    h = host(qg.qgemm_swiglu(to_dev(c["x"], dev), codes, scales, zeros, fmt))
    assert h.shape == (m, i)
    check(h, og.swiglu_reference(bf16_as_f32(c["x"]), packed, s, z, 128), f"swiglu {fmt}")


@pytest.mark.parametrize("asym", [False, True])
@pytest.mark.parametrize("k", [512, 640])      # paired / single scale loads
def test_swiglu_last_wave_quarters(asym, k):
    # 3 x 90 = 270 tiles of 128 tokens x 128 channels of h: the last 14 run as
    # 32-token quarters on a 256-CU GPU; against the oracle, and bit for bit
    # against each 128-row slice computed alone
    dev = device()
    m, i = 300, 11520
    fmt = "int4_asym" if asym else "int4_sym"
    print(f"swiglu last-wave quarters m={m} k={k} I={i} {fmt}", flush=True)
    c = small_case(m, k, 2 * i, seed=17 + asym + k, w_outlier=(0.01, 20.0))
    codes, scales, zeros = qg.quantize_pack(to_dev(c["w"], dev), fmt, 128)
    if asym:
        q, s, z = oi.quantize_asym(c["w"], 128)
    else:
        (q, s), z = oi.quantize_sym(c["w"], 128), None
    x = to_dev(c["x"], dev)
    h = qg.qgemm_swiglu(x, codes, scales, zeros, fmt)
    check(host(h), og.swiglu_reference(bf16_as_f32(c["x"]), oi.pack_int4(q), s, z, 128),
          f"swiglu {fmt}")
    for r0 in (0, 128, 256):
        part = qg.qgemm_swiglu(x[r0:r0 + 128].contiguous(), codes, scales, zeros, fmt)
        assert torch.equal(part.view(torch.int16), h[r0:r0 + 128].view(torch.int16)), r0


def test_swiglu_qwen72b_gate_up_sampled():
    dev = device()
    c = workload_case("qwen72b_prefill", 0)          # K = 8192, 29568 rows = 2 x 14784
    n2, k = c["n"], c["k"]
    i = n2 // 2
    print(f"swiglu qwen72b gate+up M=2048 K={k} I={i}", flush=True)
    codes, scales, _ = qg.quantize_pack(torch.from_numpy(c["w"]).to(dev), "int4_sym", 128)
    h = host(qg.qgemm_swiglu(c["x"].to(dev), codes, scales, None, "int4_sym"))
    ch = np.unique(np.concatenate([np.arange(8), np.arange(i - 8, i),
                                   rng_for(72).choice(i, 48, replace=False)]))
    rows = np.concatenate([ch, ch + i])
    q, s = oi.quantize_sym(c["w"][rows], 128)
    assert (host(codes)[rows] == oi.pack_int4(q)).all()
    packed_all = np.zeros((n2, k // 8), np.int32)
    scales_all = np.ones((n2, k // 128), np.float16)
    packed_all[rows] = oi.pack_int4(q)
    scales_all[rows] = s
    ref = og.swiglu_reference(bf16_as_f32(c["x"]), packed_all, scales_all, None, 128, channels=ch)
    check(h[:, ch], ref, "swiglu qwen72b")


def test_swiglu_equals_unfused():
    # the fused epilogue against the plain GEMM followed by SiLU * up on the
    # host (fp32 GEMM outputs are rounded to bf16 in the unfused path, so the
    # two agree to the bf16 rounding of gate and up)
    dev = device()
    c = small_case(256, 1024, 2 * 384, seed=9)
    codes, scales, _ = qg.quantize_pack(to_dev(c["w"], dev), "int4_sym", 128)
    x = to_dev(c["x"], dev)
    h = host(qg.qgemm_swiglu(x, codes, scales, None, "int4_sym"))
    y = host(qg.qgemm(x, codes, scales, None, "int4_sym", "bf16")).astype(np.float64)
    g, u = y[:, :384], y[:, 384:]
    assert og.rel_fro(h, og.silu(g) * u) <= 4e-3


# ------------------------------------------------------------ decode GEMV

def _check_small(h, ref, what):
    """rel. Frobenius <= 2e-3, or for fewer than 1024 outputs the
    per-element bound of one bf16 step plus a small absolute floor."""
    finite_checks(h)
    if h.size < 1024:
        floor = 1e-3 * np.sqrt(np.mean(ref ** 2))
        bad = np.abs(h - ref) > 2.0 ** -8 * np.abs(ref) + floor
        assert not bad.any(), f"{what}: {bad.sum()} outputs beyond one bf16 step"
        return
    check(h, ref, what)


# M = 1 (one x row, group sums by shuffles), 2..4 (the 4-row layout), 5..16
# (the 16-row kernel with the gate / up tile pair); K from one 512 slice to
# 16 slices; I ragged (not a multiple of 16) and I = 14336 / 2 shapes
@pytest.mark.parametrize("asym", [False, True])
@pytest.mark.parametrize("m,k,i", [(1, 512, 40), (1, 4096, 1000), (1, 16384, 24), (3, 1024, 33),
                                   (4, 2048, 200), (2, 8192, 17), (5, 512, 48), (9, 4096, 300),
                                   (16, 8192, 64), (16, 1536, 1),
                                   # x staged in LDS: 2 channel tiles per workgroup with a ragged
                                   # last tile; 2 units per wave with an empty last one; 3 and 4
                                   # rows with 4 tiles per workgroup (ragged last workgroup)
                                   (16, 2048, 5000), (7, 1024, 9000), (3, 512, 12400),
                                   (4, 1024, 12600)])
def test_qgemv_swiglu_small(m, k, i, asym):
    dev = device()
    fmt = "int4_asym" if asym else "int4_sym"
    print(f"qgemv_swiglu m={m} k={k} I={i} {fmt}", flush=True)
    c = small_case(m, k, 2 * i, seed=7 * m + i + k, w_outlier=(0.01, 20.0))
    codes, scales, zeros = qg.quantize_pack(to_dev(c["w"], dev), fmt, 128)
    if asym:
        q, s, z = oi.quantize_asym(c["w"], 128)
    else:
        (q, s), z = oi.quantize_sym(c["w"], 128), None
    packed = oi.pack_int4(q)
    assert (host(codes) == packed).all()
    x = to_dev(c["x"], dev)
    h = host(qg.qgemv_swiglu(x, codes, scales, zeros, fmt))
    ht = host(qg.qgemv_swiglu(x, qg.tile_gemv_weights(codes), scales, zeros, fmt))
    assert h.shape == (m, i)
    # same arithmetic in the same order on either code layout
    assert (ht.view(np.uint32) == h.view(np.uint32)).all(), "tiled differs from canonical"
    _check_small(h, og.swiglu_reference(bf16_as_f32(c["x"]), packed, s, z, 128),
                 f"qgemv_swiglu {fmt}")


@pytest.mark.parametrize("m", [1, 4, 16])
def test_qgemv_swiglu_llama3_8b_gate_up_sampled(m):
    # the decode workload's gate+up projection (K = 4096, 28672 rows =
    # gate and up of 14336 channels), asymmetric INT4 with outlier input
    # channels; the oracle quantizes sampled channels' gate and up rows
    dev = device()
    c = workload_case("llama3_8b_decode", 2)
    n2, k = c["n"], c["k"]
    i = n2 // 2
    print(f"qgemv_swiglu llama3_8b gate+up M={m} K={k} I={i}", flush=True)
    codes, scales, zeros = qg.quantize_pack(torch.from_numpy(c["w"]).to(dev), "int4_asym", 128)
    tiled = qg.tile_gemv_weights(codes)
    h = host(qg.qgemv_swiglu(c["x"][:m].to(dev), tiled, scales, zeros, "int4_asym"))
    ch = np.unique(np.concatenate([np.arange(16), np.arange(i - 16, i),
                                   rng_for(88 + m).choice(i, 160, replace=False)]))
    rows = np.concatenate([ch, ch + i])
    q, s, z = oi.quantize_asym(c["w"][rows], 128)
    assert (host(codes)[rows] == oi.pack_int4(q)).all()
    packed_all = np.zeros((n2, k // 8), np.int32)
    scales_all = np.ones((n2, k // 128), np.float16)
    zeros_all = np.zeros((n2, k // 128), np.float16)
    packed_all[rows], scales_all[rows], zeros_all[rows] = oi.pack_int4(q), s, z
    ref = og.swiglu_reference(bf16_as_f32(c["x"][:m]), packed_all, scales_all, zeros_all, 128,
                              channels=ch)
    check(h[:, ch], ref, f"qgemv_swiglu llama3 M={m}")
    # and against the unfused decode path: the GEMV, then SiLU(g) * u
    y = host(qg.qgemv_tiled(c["x"][:m].to(dev), tiled, scales, zeros, "int4_asym"))
    y = y.astype(np.float64)
    assert og.rel_fro(h, og.silu(y[:, :i]) * y[:, i:]) <= 4e-3


# ------------------------------------------------------------ FP8 W8A8

from oracle import fp8 as of8  # noqa: E402


# ragged M, I (not a multiple of 4 or 8, a partial last 128-channel tile),
# K with a partial last k-step (48, 176, 1040) or an odd number of whole
# k-steps (64, 192)
@pytest.mark.parametrize("m,k,i", [(64, 256, 40), (130, 512, 200), (257, 1040, 129), (1, 128, 16),
                                   (300, 2048, 384), (40, 48, 72), (100, 176, 97), (8, 64, 2),
                                   (70, 192, 136)])
def test_fp8_swiglu_small(m, k, i):
    dev = device()
    print(f"fp8 swiglu m={m} k={k} I={i}", flush=True)
    c = small_case(m, k, 2 * i, seed=5 * m + i + k, x_outlier=(0.001, 100.0))
    xq, sx, _ = qg.quantize_pack(to_dev(c["x"], dev), "fp8_e4m3")
    wq, sw, _ = qg.quantize_pack(to_dev(c["w"], dev), "fp8_e4m3")
    oxq, osx = of8.quantize_rows(bf16_as_f32(c["x"]))
    owq, osw = of8.quantize_rows(c["w"])
    assert (host(xq) == oxq).all() and (host(wq) == owq).all()
    h = host(qg.qgemm_swiglu_fp8(xq, sx, wq, sw))
    assert h.shape == (m, i)
    _check_small(h, og.fp8_swiglu_reference(oxq, osx, owq, osw), "fp8 swiglu")


def test_fp8_swiglu_8192_sampled():
    # the FP8 workload's operands (M = K = 8192) read as [W_gate; W_up] of
    # 4096 channels each; sampled channels against the oracle, and the whole
    # output against the unfused path (the FP8 GEMM, then SiLU(g) * u)
    dev = device()
    c = workload_case("fp8_8192")
    print("fp8 swiglu M=K=8192 I=4096", flush=True)
    xq, sx, _ = qg.quantize_pack(to_dev(c["x"], dev), "fp8_e4m3")
    wq, sw, _ = qg.quantize_pack(to_dev(c["w"], dev), "fp8_e4m3")
    h = host(qg.qgemm_swiglu_fp8(xq, sx, wq, sw))
    i = 4096
    rm = np.unique(np.concatenate([np.arange(4), np.arange(8188, 8192),
                                   rng_for(61).choice(8192, 40, replace=False)]))
    ch = np.unique(np.concatenate([np.arange(8), np.arange(i - 8, i),
                                   rng_for(62).choice(i, 56, replace=False)]))
    rows = np.concatenate([ch, ch + i])
    oxq, osx = of8.quantize_rows(bf16_as_f32(c["x"][rm]))
    owq, osw = of8.quantize_rows(c["w"][rows])
    assert (host(xq)[rm] == oxq).all() and (host(wq)[rows] == owq).all()
    ref = og.fp8_swiglu_reference(oxq, osx, owq, osw)
    check(h[np.ix_(rm, ch)], ref, "fp8 swiglu 8192")
    y = host(qg.qgemm(xq, wq, sw, None, "fp8_e4m3", "fp8_e4m3", a_scales=sx)).astype(np.float64)
    assert og.rel_fro(h, og.silu(y[:, :i]) * y[:, i:]) <= 4e-3
