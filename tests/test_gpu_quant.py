"""GPU parity of quantize_pack, dequant and mx_quant against the CPU oracle:
codes, packed words, scales, zero points and E8M0 bytes must match bit for
bit, on seeded inputs with outliers plus hand-placed edge groups (all zero,
all negative, fp16-subnormal scales, exact ties, a single huge value)."""

import numpy as np
import pytest
import torch

import quantized_gemm_group_amd as qg
from oracle import fp8 as of8, intquant as oi, mx as omx
from synthetic import rng_for, to_bf16, bf16_as_f32
from tests.gpu_util import bits16, bits32, device, host, to_dev

pytestmark = pytest.mark.gpu

FMTS = ["int4_sym", "int4_asym", "int8_sym", "int8_asym", "fp8_e4m3"]


def edge_matrix(rows, k, group, seed):
    """N(0, 0.02) weights with 1 % outlier columns x20 and edge groups."""
    rng = rng_for(seed)
    w = (rng.standard_normal((rows, k), dtype=np.float32) * np.float32(0.02))
    cols = rng.choice(k, size=max(1, k // 100), replace=False)
    w[:, cols] *= np.float32(20)
    g = min(group, k)
    if rows >= 6 and k >= 2 * g:
        w[0, :g] = 0.0                                        # all-zero group
        w[1, g:2 * g] = -np.abs(w[1, g:2 * g]) - 0.001        # all negative
        w[2, :g] *= np.float32(1e-4)                          # fp16-subnormal scale
        w[3, :g] = 0.0
        w[3, 5] = 3.0e4                                       # one huge value
        # exact ties for the symmetric INT4 rule: max 7 -> scale 1, values k+0.5
        w[4, :g] = np.float32(0.5) * (np.arange(g) % 13 - 6).astype(np.float32)
        w[4, 0] = 7.0
        w[5, :g] = -1e-30                                     # tiny negatives
    return w


def oracle_quant(fmt, x, group):
    rows, k = x.shape
    if fmt == "int4_sym":
        q, s = oi.quantize_sym(x, group, "int4_sym")
        return oi.pack_int4(q), s, None
    if fmt == "int4_asym":
        q, s, z = oi.quantize_asym(x, group, "int4_asym")
        return oi.pack_int4(q), s, z
    if fmt == "int8_sym":
        q, s = oi.quantize_sym(x, group, "int8_sym")
        return q.astype(np.int8), s, None
    if fmt == "int8_asym":
        q, s, z = oi.quantize_asym(x, group, "int8_asym")
        return q.astype(np.uint8), s, z
    codes, s = of8.quantize_rows(x.reshape(rows * (k // group), group))
    return codes.reshape(rows, k), s.reshape(rows, k // group), None


def _same_bits(a, b):
    a, b = np.ascontiguousarray(a), np.ascontiguousarray(b)
    assert a.shape == b.shape and a.dtype.itemsize == b.dtype.itemsize
    if a.dtype.itemsize == 2:
        return (bits16(a) == bits16(b)).all()
    if a.dtype.itemsize == 4:
        return (bits32(a) == bits32(b)).all()
    return (a.view(np.uint8) == b.view(np.uint8)).all()


@pytest.mark.parametrize("src", ["f32", "bf16"])
@pytest.mark.parametrize("group", [8, 32, 128, 512, 1024, 1536, 3072])
@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_pack_bit_exact(fmt, group, src):
    dev = device()
    rows, k = 37, 3072
    w = edge_matrix(rows, k, group, seed=100 + group)
    if src == "bf16":
        wt = to_bf16(w)
        w_or = bf16_as_f32(wt)
    else:
        wt = torch.from_numpy(w)
        w_or = w
    print(f"quantize_pack fmt={fmt} group={group} src={src} rows={rows} K={k}", flush=True)
    codes, scales, zeros = qg.quantize_pack(to_dev(wt, dev), fmt, group)
    c_o, s_o, z_o = oracle_quant(fmt, w_or, group)
    assert _same_bits(host(codes), c_o), "codes differ"
    assert _same_bits(host(scales), s_o), "scales differ"
    if z_o is not None:
        assert _same_bits(host(zeros), z_o), "zero points differ"


@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_pack_single_row_and_single_group(fmt):
    dev = device()
    for rows, k, group in [(1, 128, 128), (1, 8, 8), (3, 64, 64), (5, 24, 8)]:
        if fmt.startswith("int4") and k % 8:
            continue
        w = (rng_for(rows * k).standard_normal((rows, k), dtype=np.float32))
        codes, scales, zeros = qg.quantize_pack(to_dev(w, dev), fmt, group)
        c_o, s_o, z_o = oracle_quant(fmt, w, group)
        assert _same_bits(host(codes), c_o) and _same_bits(host(scales), s_o)
        if z_o is not None:
            assert _same_bits(host(zeros), z_o)


@pytest.mark.parametrize("k", [2048, 4096, 8192])
@pytest.mark.parametrize("fmt", ["fp8_e4m3", "int8_sym", "int8_asym"])
def test_per_row_quant_one_wave_per_row(fmt, k):
    # per-row scales (group == K) of rows of 2048..8192 elements: one wave per
    # row holds it in registers; 13 rows leave a partly filled workgroup
    dev = device()
    x = rng_for(k + 7).standard_normal((13, k), dtype=np.float32)
    x[3] = 0.0                     # all-zero row: scale 1
    x[5, ::97] *= np.float32(300)  # outliers
    xt = to_bf16(x)
    print(f"per-row quant fmt={fmt} K={k}", flush=True)
    codes, scales, zeros = qg.quantize_pack(to_dev(xt, dev), fmt, k)
    c_o, s_o, z_o = oracle_quant(fmt, bf16_as_f32(xt), k)
    assert _same_bits(host(codes), c_o) and _same_bits(host(scales), s_o)
    if z_o is not None:
        assert _same_bits(host(zeros), z_o)


def test_fp8_dynamic_activation_quant_with_outliers():
    # per-token scales of bf16 activations with 0.1 % entries x100 (the FP8
    # workload's distribution), rows spanning several workgroups
    dev = device()
    rng = rng_for(4242)
    x = rng.standard_normal((300, 8192), dtype=np.float32)
    x.reshape(-1)[rng.choice(x.size, size=x.size // 1000, replace=False)] *= np.float32(100)
    xb = to_bf16(x)
    codes, scales, _ = qg.quantize_pack(to_dev(xb, dev), "fp8_e4m3")
    c_o, s_o = of8.quantize_rows(bf16_as_f32(xb))
    assert (host(codes) == c_o).all()
    assert (bits32(host(scales)[:, 0]) == bits32(s_o)).all()


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("fmt", FMTS + ["mxfp4"])
def test_dequant_bit_exact(fmt, out):
    dev = device()
    from oracle import formats as of
    rows, k = 29, 1024
    group = 32 if fmt == "mxfp4" else (128 if fmt.startswith("int4") else 256)
    w = edge_matrix(rows, k, group, seed=7)
    if fmt == "mxfp4":
        c_o, e_o = omx.quantize(w)
        ref = omx.dequantize(c_o, e_o).astype(np.float32)
        codes, scales, zeros = to_dev(c_o, dev), to_dev(e_o, dev), None
    else:
        c_o, s_o, z_o = oracle_quant(fmt, w, group)
        if fmt.startswith("int4"):
            q = oi.unpack_int4(c_o, signed=(fmt == "int4_sym"))
            ref = oi.dequantize(q, s_o, z_o, group, out="f32")
        elif fmt == "fp8_e4m3":
            ref = of8.dequantize_rows(c_o.reshape(-1, group), s_o.reshape(-1)).reshape(
                rows, k).astype(np.float32)
        else:
            ref = oi.dequantize(c_o.astype(np.int64), s_o, z_o, group, out="f32")
        codes = to_dev(c_o, dev)
        scales = to_dev(s_o, dev)
        zeros = None if z_o is None else to_dev(z_o, dev)
    odt = torch.float32 if out == "f32" else torch.bfloat16
    got = host(qg.dequant(codes, scales, zeros, fmt, k, group, out_dtype=odt))
    if out == "bf16":
        ref = of.round_to_bf16(ref)
    assert (bits32(got.astype(np.float32)) == bits32(ref)).all()


def mx_edge_matrix(rows, k, seed):
    rng = rng_for(seed)
    x = rng.standard_normal((rows, k), dtype=np.float32)
    x[:, 3] *= np.float32(50)
    x[0, :32] = 0.0                                       # zero block
    x[1, :32] = np.float32(1e-40)                         # fp32-subnormal block
    x[1, 32:64] = np.float32(3e-39) * rng.standard_normal(32).astype(np.float32)
    x[2, :32] = np.float32(6.0 * 2.0 ** 5)                # max exactly 6*2^k
    x[2, 32] = np.nextafter(np.float32(6.0 * 2.0 ** -3), np.float32(1))   # just above
    x[2, 33:64] = 0.1
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], np.float32)
    x[3, :32] = np.tile(np.concatenate([mids, -mids]), 2)  # ties, max 6 -> e = 0
    x[4, :32] = -0.0
    x[5, :32] = np.float32(3.0e38) * np.sign(rng.standard_normal(32)).astype(np.float32)
    return x


@pytest.mark.parametrize("src", ["f32", "bf16"])
def test_mx_quant_bit_exact(src):
    dev = device()
    x = mx_edge_matrix(45, 2048, 5)
    if src == "bf16":
        xt = to_bf16(x)
        x_or = bf16_as_f32(xt)
    else:
        xt = torch.from_numpy(x)
        x_or = x
    codes, e8 = qg.mx_quant(to_dev(xt, dev))
    c_o, e_o = omx.quantize(x_or)
    assert (host(e8) == e_o).all(), "E8M0 bytes differ"
    assert (host(codes) == c_o).all(), "E2M1 codes differ"


def test_geometry_errors_raise_value_error():
    dev = device()
    x = torch.zeros((4, 96), device=dev)
    with pytest.raises(ValueError, match="invalid quantization geometry"):
        qg.mx_quant(x[:, :48].contiguous())
    with pytest.raises(ValueError, match="invalid quantization geometry"):
        qg.quantize_pack(x, "int4_sym", 64)


def _bf16_patterns_up_to(limit_bits):
    """Every finite bf16 value with magnitude bits <= limit_bits, both signs."""
    mags = np.arange(0, limit_bits + 1, dtype=np.uint32)
    pats = np.concatenate([mags, mags | 0x8000]).astype(np.uint32)
    return (pats << 16).view(np.float32)


@pytest.mark.parametrize("group", [128, 8192])
def test_fp8_codes_of_every_bf16_value(group):
    # each group holds 448 so its scale is exactly 1: the codes are the E4M3
    # encoding of every bf16 value in [-448, 448] (0x43E0 = 448)
    dev = device()
    vals = _bf16_patterns_up_to(0x43E0)
    per = group - 1
    groups = -(-vals.size // per)
    groups = -(-groups // (8192 // group)) * (8192 // group)    # whole rows of 8192
    body = np.zeros(groups * per, np.float32)
    body[:vals.size] = vals
    x = np.concatenate([np.full((groups, 1), 448.0, np.float32), body.reshape(groups, per)], axis=1)
    x = x.reshape(-1, 8192)
    print(f"fp8 encoding of {vals.size} bf16 values, group {group}", flush=True)
    codes, scales, _ = qg.quantize_pack(to_dev(to_bf16(x), dev), "fp8_e4m3", group)
    c_o, s_o, _ = oracle_quant("fp8_e4m3", x, group)
    assert (host(scales) == 1.0).all()
    assert _same_bits(host(codes), c_o)


def test_mx_codes_at_e2m1_ties():
    # blocks with max 6 (exponent 0) holding every E2M1 midpoint, its bf16
    # neighbours and the grid values themselves
    dev = device()
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)
    mids = (grid[1:] + grid[:-1]) / 2
    pts = np.concatenate([grid, mids])
    b = to_bf16(pts.astype(np.float32)).view(torch.int16).numpy().astype(np.int32)
    near = np.concatenate([b - 1, b + 1, b])
    near = near[(near >= 0) & (near <= 0x40C0)].astype(np.uint32)     # 0x40C0 = 6.0
    vals = (near << 16).view(np.float32)
    vals = np.concatenate([vals, -vals])
    per = 31
    n = -(-vals.size // per) * per
    body = np.zeros(n, np.float32)
    body[:vals.size] = vals
    x = np.concatenate([np.full((n // per, 1), 6.0, np.float32), body.reshape(-1, per)], axis=1)
    x = x.reshape(1, -1)
    print(f"mx encoding at {vals.size} tie points", flush=True)
    c, e = qg.mx_quant(to_dev(to_bf16(x), dev))
    c_o, e_o = omx.quantize(bf16_as_f32(to_bf16(x)))
    assert (host(e) == 127).all() and (e_o == 127).all()
    assert (host(c) == c_o).all()
