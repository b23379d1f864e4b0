"""The debug library (libqgemm_debug.so, QG_DEBUG_FP32): every product entry
point also records the fp32 value that it rounds to bf16.  Two pins per
kernel: the bf16 output is that fp32 value rounded once to nearest even (bit
for bit), and the fp32 value is the oracle's float64 product within fp32
accumulation error (relative Frobenius <= 1e-5), which localises a parity
failure below the bf16 rounding.  SwiGLU outputs multiply two such sums and
go through the hardware exponential, so their bound is 3e-5.  The scaled
FP8 / FP4 matrix instructions do not accumulate as a sequence of IEEE fp32
additions (measured: 5e-5 at K = 512 with outlier activations), so FP8 and
MXFP4 products are held to 2e-4 (still a tenth of the bf16 rounding)."""

import ctypes

import numpy as np
import pytest
import torch

import quantized_gemm_group_amd as qg
from quantized_gemm_group_amd import _lib
from oracle import formats as of, fp8 as of8, gemm as og, intquant as oi, mx as omx
from synthetic import bf16_as_f32, small_case
from tests.gpu_util import device, host, to_dev

pytestmark = pytest.mark.gpu

P = lambda t: ctypes.c_void_p(0 if t is None else t.data_ptr())  # noqa: E731


def _run(dlib, fn, shape, dev):
    """Call fn(dbg) with a fresh fp32 debug buffer set, then clear it."""
    dbg = torch.full(shape, float("nan"), dtype=torch.float32, device=dev)
    assert dlib.qg_debug_fp32_output(P(dbg), None) == _lib.OK
    try:
        st = fn()
        torch.cuda.synchronize()
    finally:
        assert dlib.qg_debug_fp32_output(None, None) == _lib.OK
    assert st == _lib.OK
    return host(dbg)


def _pins(y, dbg, ref, what, tol=1e-5):
    assert np.isfinite(dbg).all(), f"{what}: outputs not recorded"
    assert (y.view(np.uint32) == of.round_to_bf16(dbg).view(np.uint32)).all(), \
        f"{what}: bf16 output is not the recorded fp32 value rounded once"
    err = og.rel_fro(dbg, ref)
    assert err <= tol, f"{what}: fp32 pre-rounding rel_fro {err}"


@pytest.fixture(scope="module")
def dlib():
    lib = _lib.load_debug()
    assert lib.qg_debug_build() == 1
    return lib


def test_product_library_has_no_recorder():
    lib = _lib.load()
    assert lib.qg_debug_build() == 0
    assert lib.qg_debug_fp32_output(None, None) == _lib.ERR_UNSUPPORTED


@pytest.mark.parametrize("m,group", [(1, 128), (4, 128), (16, 128), (3, 64)])
def test_debug_qgemv(dlib, m, group):
    dev = device()
    k, n = 1024, 300
    c = small_case(m, k, n, seed=m + group, w_outlier=(0.01, 20.0))
    codes, s, z = qg.quantize_pack(to_dev(c["w"], dev), "int4_asym", group)
    q, so, zo = oi.quantize_asym(c["w"], group)
    x = to_dev(c["x"], dev)
    y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    dbg = _run(dlib, lambda: dlib.qg_qgemv(_lib.INT4_ASYM, P(x), m, P(codes), P(s), P(z), n, k,
                                           group, P(y), None), (m, n), dev)
    ref = og.w4a16_reference(bf16_as_f32(c["x"]), oi.pack_int4(q), so, zo, group)
    _pins(host(y), dbg, ref, f"qgemv m={m} g={group}")


def test_debug_w4a16_gemm_and_swiglu(dlib):
    dev = device()
    m, k, n = 130, 1024, 264
    c = small_case(m, k, n, seed=5, w_outlier=(0.01, 20.0))
    codes, s, _ = qg.quantize_pack(to_dev(c["w"], dev), "int4_sym", 128)
    q, so = oi.quantize_sym(c["w"], 128)
    packed = oi.pack_int4(q)
    x = to_dev(c["x"], dev)
    xf = bf16_as_f32(c["x"])
    y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    dbg = _run(dlib, lambda: dlib.qg_qgemm(_lib.INT4_SYM, _lib.BF16_ACT, P(x), None, None, m,
                                           P(codes), P(s), None, n, k, 128, P(y), None),
               (m, n), dev)
    _pins(host(y), dbg, og.w4a16_reference(xf, packed, so, None, 128), "w4a16 gemm")
    h = torch.empty((m, n // 2), dtype=torch.bfloat16, device=dev)
    dbg = _run(dlib, lambda: dlib.qg_qgemm_swiglu(_lib.INT4_SYM, _lib.BF16_ACT, P(x), m, P(codes),
                                                  P(s), None, n, k, 128, P(h), None),
               (m, n // 2), dev)
    _pins(host(h), dbg, og.swiglu_reference(xf, packed, so, None, 128), "w4a16 swiglu", 3e-5)
    h4 = torch.empty((4, n // 2), dtype=torch.bfloat16, device=dev)
    dbg = _run(dlib, lambda: dlib.qg_qgemv_swiglu(_lib.INT4_SYM, P(x), 4, P(codes), P(s), None,
                                                  n, k, 128, 0, P(h4), None), (4, n // 2), dev)
    _pins(host(h4), dbg, og.swiglu_reference(xf[:4], packed, so, None, 128), "qgemv swiglu",
          3e-5)


def test_debug_fp8_int8_mx(dlib):
    dev = device()
    m, k, n = 130, 512, 200
    c = small_case(m, k, n, seed=9, x_outlier=(0.001, 100.0))
    xf = bf16_as_f32(c["x"])
    xq, sx, _ = qg.quantize_pack(to_dev(c["x"], dev), "fp8_e4m3")
    wq, sw, _ = qg.quantize_pack(to_dev(c["w"], dev), "fp8_e4m3")
    oxq, osx = of8.quantize_rows(xf)
    owq, osw = of8.quantize_rows(c["w"])
    y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    dbg = _run(dlib, lambda: dlib.qg_qgemm(_lib.FP8_E4M3, _lib.FP8_E4M3, P(xq), P(sx), None, m,
                                           P(wq), P(sw), None, n, k, k, P(y), None), (m, n), dev)
    _pins(host(y), dbg, og.fp8_reference(oxq, osx, owq, osw), "fp8 gemm", 2e-4)
    h = torch.empty((m, n // 2), dtype=torch.bfloat16, device=dev)
    dbg = _run(dlib, lambda: dlib.qg_qgemm_swiglu_fp8(P(xq), P(sx), m, P(wq), P(sw), n, k, P(h),
                                                      None), (m, n // 2), dev)
    _pins(host(h), dbg, og.fp8_swiglu_reference(oxq, osx, owq, osw), "fp8 swiglu", 2e-4)
    aq, as_, _ = qg.quantize_pack(to_dev(c["x"], dev), "int8_sym")
    iq, is_, _ = qg.quantize_pack(to_dev(c["w"], dev), "int8_sym")
    oaq, oas = oi.quantize_sym(xf, k, "int8_sym")
    oiq, ois = oi.quantize_sym(c["w"], k, "int8_sym")
    dbg = _run(dlib, lambda: dlib.qg_qgemm(_lib.INT8_SYM, _lib.INT8_SYM, P(aq), P(as_), None, m,
                                           P(iq), P(is_), None, n, k, k, P(y), None), (m, n), dev)
    _pins(host(y), dbg, og.int8_reference(oaq.astype(np.int64), oas, None, oiq.astype(np.int64),
                                          ois, None), "int8 gemm")
    ac, ae = qg.mx_quant(to_dev(c["x"], dev))
    bc, be = qg.mx_quant(to_dev(c["w"], dev))
    oac, oae = omx.quantize(xf)
    obc, obe = omx.quantize(c["w"])
    dbg = _run(dlib, lambda: dlib.qg_mx_gemm(P(ac), P(ae), m, P(bc), P(be), n, k, P(y), None),
               (m, n), dev)
    _pins(host(y), dbg, og.mx_reference(oac, oae, obc, obe), "mx gemm", 2e-4)
