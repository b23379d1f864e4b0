"""GPU parity of the SmoothQuant path against the CPU oracle: channel maxima
(bit-exact, with accumulation over batches, ragged K and many row chunks),
the smoothing factors (bit-exact, including the degenerate channels and the
alpha limits), the smoothed quantization (codes, scales and zeros bit-exact
for every format, both fold directions, bf16 and fp32 sources), the static
channel scales, the full 8192 x 8192 activations with outlier channels, and
the end-to-end INT8 W8A8 product of smoothed operands (within 2e-3 of the
oracle's fp64 product, and closer to X W^T than without smoothing)."""

import numpy as np
import pytest
import torch

import quantized_gemm_group_amd as qg
from oracle import gemm as og, intquant as oi, kvcache as okv, smooth as osm
from synthetic import bf16_as_f32, rng_for, smoothquant_case, to_bf16
from tests.gpu_util import bits16, bits32, device, host, to_dev

pytestmark = pytest.mark.gpu

FMTS = ["int4_sym", "int4_asym", "int8_sym", "int8_asym", "fp8_e4m3"]


def same_bits(a, b):
    a, b = np.ascontiguousarray(a), np.ascontiguousarray(b)
    assert a.shape == b.shape, (a.shape, b.shape)
    if a.dtype.itemsize == 2:
        return (bits16(a) == bits16(b)).all()
    if a.dtype.itemsize == 4:
        return (bits32(a) == bits32(b)).all()
    return (a.view(np.uint8) == b.view(np.uint8)).all()


def source(x32, src, dev):
    """Device tensor of x in the source dtype, and the values the oracle sees."""
    if src == "bf16":
        t = to_bf16(x32)
        return to_dev(t, dev), bf16_as_f32(t)
    return to_dev(x32, dev), x32


@pytest.mark.parametrize("src", ["bf16", "f32"])
@pytest.mark.parametrize("rows,k", [(1, 8), (37, 520), (300, 4104), (1000, 1024), (5, 16392)])
def test_channel_absmax_bit_exact(rows, k, src):
    dev = device()
    print(f"channel_absmax rows={rows} K={k} {src}", flush=True)
    rng = rng_for(rows + k)
    x = rng.standard_normal((rows, k), dtype=np.float32)
    x[:, rng.choice(k, max(1, k // 100), replace=False)] *= 30
    x[0, : min(k, 5)] = -0.0
    xd, xo = source(x, src, dev)
    got = host(qg.channel_absmax(xd))
    assert same_bits(got, osm.channel_absmax(xo))


def test_channel_absmax_accumulates_over_batches():
    dev = device()
    rng = rng_for(7)
    a = rng.standard_normal((200, 2048), dtype=np.float32)
    b = 2 * rng.standard_normal((333, 2048), dtype=np.float32)
    run = qg.channel_absmax(to_dev(a, dev))
    qg.channel_absmax(to_dev(b, dev), out=run)
    assert same_bits(host(run), osm.channel_absmax(b, osm.channel_absmax(a)))
    # a running maximum already larger everywhere stays as it is
    big = torch.full((2048,), 1e6, dtype=torch.float32, device=dev)
    qg.channel_absmax(to_dev(a, dev), out=big)
    assert (host(big) == np.float32(1e6)).all()


@pytest.mark.parametrize("alpha", [0.0, 0.5, 0.85, 1.0])
def test_smooth_scales_bit_exact(alpha):
    dev = device()
    rng = rng_for(11)
    k = 4099
    a = np.abs(rng.standard_normal(k, dtype=np.float32)) * np.exp(rng.standard_normal(k)).astype(np.float32)
    w = np.abs(rng.standard_normal(k, dtype=np.float32)) * np.float32(0.05)
    a[:4] = [0, 1, 0, 1e-40]
    w[:4] = [1, 0, 0, 1]
    a[4], w[4] = 1e30, 1e-30
    s = host(qg.smooth_scales(to_dev(a.astype(np.float32), dev), to_dev(w.astype(np.float32), dev),
                              alpha))
    ref = osm.smooth_scales(a, w, alpha)
    bad = np.flatnonzero(bits32(s) != bits32(ref))
    assert len(bad) == 0, f"{len(bad)} factors differ, first {bad[:4]}: {s[bad[:4]]} {ref[bad[:4]]}"


@pytest.mark.parametrize("alpha", [0.3, 0.5, 0.85])
def test_smooth_scales_bulk_agreement(alpha):
    # 2^20 factor pairs over twelve decades.  The GPU takes the fp64 power
    # from its math library, the oracle from the host's; each is within an
    # ulp of the exact fp64 value, so the fp32 factors may only differ where
    # that value sits within a few fp64 units of the midpoint between two
    # fp32 numbers.  Every other factor must match bit for bit, and any
    # difference must be one fp32 step at such a midpoint.
    dev = device()
    rng = rng_for(int(alpha * 100) + 17)
    n = 1 << 20
    a = (10.0 ** rng.uniform(-6, 6, n)).astype(np.float32)
    w = (10.0 ** rng.uniform(-6, 6, n)).astype(np.float32)
    s = host(qg.smooth_scales(to_dev(a, dev), to_dev(w, dev), alpha))
    ref = osm.smooth_scales(a, w, alpha)
    diff = np.flatnonzero(bits32(s) != bits32(ref))
    print(f"alpha={alpha}: {len(diff)} of {n} factors split at a midpoint", flush=True)
    if len(diff):
        gs, rs = s[diff], ref[diff]
        assert (np.abs(bits32(gs).astype(np.int64) - bits32(rs).astype(np.int64)) == 1).all()
        v = (np.power(a[diff].astype(np.float64), alpha)
             / np.power(w[diff].astype(np.float64), 1.0 - alpha))
        mid = (gs.astype(np.float64) + rs.astype(np.float64)) / 2
        assert (np.abs(v - mid) <= 8 * np.spacing(v)).all(), "a split away from a midpoint"


@pytest.mark.parametrize("divide", [False, True])
@pytest.mark.parametrize("src", ["bf16", "f32"])
@pytest.mark.parametrize("fmt,group", [(f, 128) for f in FMTS] + [("int8_sym", 1024),
                                                                  ("fp8_e4m3", 3072),
                                                                  ("int8_asym", 32),
                                                                  ("fp8_e4m3", 1536)])
def test_quantize_pack_smooth_bit_exact(fmt, group, src, divide):
    dev = device()
    rows, k = 24, 3072
    print(f"quantize_pack_smooth {fmt} g{group} {src} divide={divide}", flush=True)
    c = smoothquant_case(rows, k, 16, seed=group + (7 if divide else 3))
    x = bf16_as_f32(c["x"]) if divide else c["w"]
    stat_x = osm.channel_absmax(bf16_as_f32(c["x"]))
    s = osm.smooth_scales(stat_x, osm.channel_absmax(c["w"]), 0.5)
    xd, xo = source(x, src, dev)
    codes, scales, zeros = qg.quantize_pack_smooth(xd, to_dev(s, dev), fmt, group, divide=divide)
    rc, rs, rz = osm.smooth_quantize(xo, s, divide, fmt, group)
    assert same_bits(host(codes), rc)
    assert same_bits(host(scales), rs)
    if rz is not None:
        assert same_bits(host(zeros), rz)


def test_unit_factors_match_plain_quantizer():
    dev = device()
    w = rng_for(5).standard_normal((64, 1024), dtype=np.float32) * np.float32(0.02)
    one = torch.ones(1024, dtype=torch.float32, device=dev)
    for fmt in FMTS:
        a = qg.quantize_pack(to_dev(w, dev), fmt)
        b = qg.quantize_pack_smooth(to_dev(w, dev), one, fmt)
        for p, q in zip(a, b):
            assert (p is None and q is None) or same_bits(host(p), host(q))


def test_channel_scales_bit_exact():
    dev = device()
    a = np.abs(rng_for(3).standard_normal(1000, dtype=np.float32)) * np.float32(7)
    a[:3] = [0, 1e-44, 448]
    got = host(qg.channel_scales(to_dev(a, dev), 448.0))
    assert same_bits(got, okv.channel_scales(a, 448.0))


def test_smoothquant_activations_8192_full_size():
    # the 8192 x 8192 activations with 1 % outlier channels: statistics over
    # all rows, factors, and the smoothed per-token INT8 / FP8 codes of
    # sampled rows against the oracle
    dev = device()
    print("smoothquant 8192 x 8192 activations", flush=True)
    c = smoothquant_case(8192, 8192, 64, seed=6)
    x_dev = to_dev(c["x"], dev)
    xo = bf16_as_f32(c["x"])
    stat = qg.channel_absmax(x_dev)
    ref_stat = osm.channel_absmax(xo)
    assert same_bits(host(stat), ref_stat)
    wstat = osm.channel_absmax(c["w"])
    s = qg.smooth_scales(stat, to_dev(wstat, dev), 0.5)
    ref_s = osm.smooth_scales(ref_stat, wstat, 0.5)
    assert same_bits(host(s), ref_s)
    rows = np.unique(np.concatenate([np.arange(4), np.arange(8188, 8192),
                                     rng_for(60).choice(8192, 24, replace=False)]))
    for fmt in ("int8_sym", "fp8_e4m3"):
        codes, scales, _ = qg.quantize_pack_smooth(x_dev, s, fmt, divide=True)
        rc, rs, _ = osm.smooth_quantize(xo[rows], ref_s, True, fmt, 8192)
        assert same_bits(host(codes)[rows], rc)
        assert same_bits(host(scales)[rows], rs)
    # the outlier channels' range shrinks: smoothed maxima are sqrt(a w)
    xs_max = osm.channel_absmax(osm.fold(xo[:512], ref_s, True))
    assert xs_max[c["outlier_channels"]].max() < 0.5 * ref_stat[c["outlier_channels"]].min()


def test_smoothquant_int8_w8a8_end_to_end():
    # calibrate, smooth and quantize both operands on the GPU, then the INT8
    # GEMM: within 2e-3 of the oracle's product of the dequantized smoothed
    # operands, and closer to X W^T than the same path without smoothing
    dev = device()
    m, k, n = 256, 2048, 384
    c = smoothquant_case(m, k, n, seed=9)
    x_dev, w_dev = to_dev(c["x"], dev), to_dev(c["w"], dev)
    s = qg.smooth_scales(qg.channel_absmax(x_dev), qg.channel_absmax(w_dev), 0.5)
    wc, ws, _ = qg.quantize_pack_smooth(w_dev, s, "int8_sym")
    xc, xs, _ = qg.quantize_pack_smooth(x_dev, s, "int8_sym", divide=True)
    y = host(qg.qgemm(xc, wc, ws, None, "int8_sym", "int8_sym", a_scales=xs)).astype(np.float64)
    xo = bf16_as_f32(c["x"])
    so = osm.smooth_scales(osm.channel_absmax(xo), osm.channel_absmax(c["w"]), 0.5)
    assert same_bits(host(s), so)
    qx, sx, _ = osm.smooth_quantize(xo, so, True, "int8_sym", k)
    qw, sw, _ = osm.smooth_quantize(c["w"], so, False, "int8_sym", k)
    ref = oi.dequantize(qx, sx, None, k) @ oi.dequantize(qw, sw, None, k).T
    assert og.rel_fro(y, ref) <= 2e-3
    exact = xo.astype(np.float64) @ c["w"].astype(np.float64).T
    pc, ps, _ = qg.quantize_pack(w_dev, "int8_sym")
    ac, as_, _ = qg.quantize_pack(x_dev, "int8_sym")
    y_plain = host(qg.qgemm(ac, pc, ps, None, "int8_sym", "int8_sym", a_scales=as_))
    assert og.rel_fro(y, exact) < 0.7 * og.rel_fro(y_plain.astype(np.float64), exact)
