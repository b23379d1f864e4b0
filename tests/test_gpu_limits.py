"""GPU parity at the largest operands the library accepts: every kernel
addresses its operands with 32-bit byte offsets inside buffers of at most
2 GiB - 4 KiB (including the up to 256 rows a tile may run past the end), so
the decode GEMV and the W4A16, FP8 and MXFP4 GEMMs are run with weight
codes just under that limit (ragged row counts), and checked against the
oracle on sampled output channels, including the last rows.  The codes and
scales are drawn directly on the GPU (random packed words, fp16 scales and
integer zero points; FP8 codes without the two NaN patterns; E8M0 exponents
near 127); the oracle dequantizes the sampled rows from the same codes."""

import numpy as np
import pytest
import torch

import quantized_gemm_group_amd as qg
from oracle import gemm as og
from synthetic import bf16_as_f32, rng_for, to_bf16
from tests.gpu_util import device, finite_checks, host, to_dev

pytestmark = pytest.mark.gpu

LIMIT = 0x7ffff000
TOL = 2e-3


def max_rows(row_bytes):
    return LIMIT // row_bytes - 256


def int4_operand(n, k, dev, seed):
    g = torch.Generator(device=dev).manual_seed(seed)
    codes = torch.randint(0, 256, (n, k // 2), dtype=torch.uint8, device=dev,
                          generator=g).view(torch.int32)
    scales = (torch.rand((n, k // 128), device=dev, generator=g) * 0.009 + 0.001).half()
    zeros = torch.randint(0, 16, (n, k // 128), device=dev, generator=g).half()
    return codes, scales, zeros


def sample_rows(n, seed):
    rng = rng_for(seed)
    return np.unique(np.concatenate([np.arange(16), np.arange(n - 40, n),
                                     rng.choice(n, 100, replace=False)]))


def host_rows(t, rows, dev):
    return host(t[torch.from_numpy(rows).to(dev)])


def test_qgemv_at_the_offset_limit():
    dev = device()
    k = 16384
    n = max_rows(k // 2)                       # 261887: 2,145,378,304 bytes of codes
    assert (n + 256) * (k // 2) <= LIMIT < (n + 257) * (k // 2)
    print(f"qgemv at the offset limit: N={n} K={k}", flush=True)
    codes, scales, zeros = int4_operand(n, k, dev, 1)
    rows = sample_rows(n, 2)
    packed, s, z = (host_rows(t, rows, dev) for t in (codes, scales, zeros))
    x = to_bf16(rng_for(3).standard_normal((16, k), dtype=np.float32))
    xs = bf16_as_f32(x)
    for m in (1, 4, 16):
        y = host(qg.qgemv(to_dev(x[:m], dev), codes, scales, zeros, "int4_asym"))
        assert y.shape == (m, n)
        finite_checks(y)
        ref = og.w4a16_reference(xs[:m], packed, s, z, 128)
        err = og.rel_fro(y[:, rows], ref)
        assert err <= TOL, f"M={m} rel_fro {err}"
    del codes, scales, zeros
    torch.cuda.empty_cache()


def test_w4a16_gemm_at_the_offset_limit():
    dev = device()
    k = 16384
    n = max_rows(k // 2)
    m = 130
    print(f"W4A16 GEMM at the offset limit: M={m} N={n} K={k}", flush=True)
    codes, scales, _ = int4_operand(n, k, dev, 4)
    rows = sample_rows(n, 5)
    packed, s = (host_rows(t, rows, dev) for t in (codes, scales))
    x = to_bf16(rng_for(6).standard_normal((m, k), dtype=np.float32))
    y = host(qg.qgemm(to_dev(x, dev), codes, scales, None, "int4_sym", "bf16"))
    assert y.shape == (m, n)
    finite_checks(y)
    ref = og.w4a16_reference(bf16_as_f32(x), packed, s, None, 128)
    err = og.rel_fro(y[:, rows], ref)
    assert err <= TOL, f"rel_fro {err}"
    del codes, scales
    torch.cuda.empty_cache()


def test_fp8_gemm_at_the_offset_limit():
    dev = device()
    k = 16384
    n = max_rows(k)                            # 130815 rows of 16 KiB
    m = 260
    print(f"FP8 GEMM at the offset limit: M={m} N={n} K={k}", flush=True)
    g = torch.Generator(device=dev).manual_seed(7)
    # E4M3 codes without 0x7F / 0xFF (NaN): magnitude bits 0..0x7E, any sign
    mag = torch.randint(0, 0x7F, (n, k), dtype=torch.uint8, device=dev, generator=g)
    sign = torch.randint(0, 2, (n, k), dtype=torch.uint8, device=dev, generator=g) << 7
    wq = mag | sign
    del mag, sign
    sw = torch.rand(n, device=dev, generator=g) * 0.01 + 0.001
    x = torch.from_numpy(rng_for(8).standard_normal((m, k), dtype=np.float32)).to(dev)
    xq, sx, _ = qg.quantize_pack(x, "fp8_e4m3")
    from oracle import fp8 as of8
    oxq, osx = of8.quantize_rows(host(x))
    assert (host(xq) == oxq).all() and (host(sx).reshape(-1) == np.asarray(osx).reshape(-1)).all()
    y = host(qg.qgemm(xq, wq, sw, None, "fp8_e4m3", "fp8_e4m3", a_scales=sx))
    assert y.shape == (m, n)
    finite_checks(y)
    rows = sample_rows(n, 9)
    w_rows = host_rows(wq, rows, dev)
    from oracle import fp8 as of8
    xa = of8.dequantize_rows(host(xq), host(sx).reshape(-1))
    wa = of8.dequantize_rows(w_rows, host(sw)[rows])
    ref = xa @ wa.T
    err = og.rel_fro(y[:, rows], ref)
    assert err <= TOL, f"rel_fro {err}"
    del wq, sw, xq, sx
    torch.cuda.empty_cache()


def test_mx_gemm_at_the_offset_limit():
    dev = device()
    k = 32768
    n = max_rows(k // 2)                       # 130815 rows of 16 KiB of E2M1 codes
    m = 260
    print(f"MXFP4 GEMM at the offset limit: M={m} N={n} K={k}", flush=True)
    g = torch.Generator(device=dev).manual_seed(10)
    bc = torch.randint(0, 256, (n, k // 2), dtype=torch.uint8, device=dev, generator=g)
    be = torch.randint(120, 131, (n, k // 32), dtype=torch.uint8, device=dev, generator=g)
    x = torch.from_numpy(rng_for(11).standard_normal((m, k), dtype=np.float32)).to(dev)
    ac, ae = qg.mx_quant(x)
    from oracle import mx as omx
    oac, oae = omx.quantize(host(x))
    assert (host(ac) == oac).all() and (host(ae) == oae).all()
    y = host(qg.mx_gemm(ac, ae, bc, be))
    assert y.shape == (m, n)
    finite_checks(y)
    rows = sample_rows(n, 12)
    ref = og.mx_reference(host(ac), host(ae), host_rows(bc, rows, dev), host_rows(be, rows, dev))
    err = og.rel_fro(y[:, rows], ref)
    assert err <= TOL, f"rel_fro {err}"
    del bc, be, ac, ae
    torch.cuda.empty_cache()
