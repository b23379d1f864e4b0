"""The C ABI library: it loads without a GPU, exports every entry point the
header declares, and rejects invalid arguments before any HIP call (so these
tests never launch a kernel)."""

import ctypes
import os
import re

import pytest

from quantized_gemm_group_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qgemm.h")

vp = ctypes.c_void_p
A16 = vp(0x1000)      # fake, aligned: never dereferenced (validation fails first)
A16b = vp(0x2000)
A16c = vp(0x3000)
A16d = vp(0x4000)
A16e = vp(0x5000)
MIS = vp(0x1008)      # misaligned


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_header_declarations_are_exported(lib):
    text = open(HEADER).read()
    declared = set(re.findall(r"^\s*(?:qg_status|const char\*|int)\s+(qg_\w+)\s*\(", text, re.M))
    assert declared == set(_lib.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.qg_abi_version() == 1
    assert lib.qg_status_str(_lib.ERR_GEOMETRY) == b"invalid quantization geometry"
    assert lib.qg_status_str(_lib.OK) == b"ok"
    assert lib.qg_status_str(99) == b"unknown status"


def test_quantize_pack_validation(lib):
    q = lib.qg_quantize_pack
    assert q(_lib.INT4_SYM, A16, _lib.F32, 4, 256, 100, A16b, A16c, None, None) == _lib.ERR_GEOMETRY
    assert q(_lib.INT4_SYM, A16, _lib.F32, 4, 256, 0, A16b, A16c, None, None) == _lib.ERR_GEOMETRY
    assert q(_lib.INT4_SYM, A16, _lib.F32, 0, 256, 128, A16b, A16c, None, None) == _lib.ERR_GEOMETRY
    assert q(_lib.INT4_SYM, A16, _lib.F32, 4, 12, 12, A16b, A16c, None, None) == _lib.ERR_GEOMETRY
    assert q(_lib.INT4_ASYM, A16, _lib.F32, 4, 256, 128, A16b, A16c, None, None) == _lib.ERR_NULL
    assert q(_lib.INT4_SYM, A16, _lib.F32, 4, 256, 128, A16b, A16c, A16d, None) == _lib.ERR_NULL
    assert q(_lib.INT4_SYM, None, _lib.F32, 4, 256, 128, A16b, A16c, None, None) == _lib.ERR_NULL
    assert q(_lib.INT4_SYM, MIS, _lib.F32, 4, 256, 128, A16b, A16c, None, None) == _lib.ERR_ALIGN
    assert q(_lib.BF16_ACT, A16, _lib.F32, 4, 256, 128, A16b, A16c, None, None) == _lib.ERR_FORMAT
    assert q(_lib.INT8_SYM, A16, 7, 4, 256, 256, A16b, A16c, None, None) == _lib.ERR_FORMAT


def test_dequant_validation(lib):
    d = lib.qg_dequant
    assert d(_lib.MXFP4, A16, A16b, None, 4, 256, 64, A16c, _lib.F32, None) == _lib.ERR_GEOMETRY
    assert d(_lib.INT4_SYM, A16, A16b, None, 4, 256, 128, None, _lib.F32, None) == _lib.ERR_NULL
    assert d(_lib.INT4_SYM, A16, A16b, None, 4, 256, 128, MIS, _lib.F32, None) == _lib.ERR_ALIGN
    assert d(_lib.INT4_SYM, A16, A16b, None, 4, 256, 128, A16c, 5, None) == _lib.ERR_FORMAT
    assert d(_lib.BF16_ACT, A16, A16b, None, 4, 256, 128, A16c, _lib.F32, None) == _lib.ERR_FORMAT


def test_qgemv_validation(lib):
    g = lib.qg_qgemv
    assert g(_lib.INT4_SYM, A16, 0, A16b, A16c, None, 16, 256, 128, A16e, None) == _lib.ERR_GEOMETRY
    assert g(_lib.INT4_SYM, A16, 17, A16b, A16c, None, 16, 256, 128, A16e, None) == _lib.ERR_GEOMETRY
    assert g(_lib.INT4_SYM, A16, 1, A16b, A16c, None, 0, 256, 128, A16e, None) == _lib.ERR_GEOMETRY
    assert g(_lib.INT4_SYM, A16, 1, A16b, A16c, None, 16, 200, 128, A16e, None) == _lib.ERR_GEOMETRY
    # groups of 32, 64 and multiples of 128 are implemented; 96 is not
    assert g(_lib.INT4_SYM, A16, 1, A16b, A16c, None, 16, 384, 96, A16e, None) == _lib.ERR_UNSUPPORTED
    assert g(_lib.INT4_SYM, A16, 1, A16b, A16c, None, 16, 96, 32, A16e, None) == _lib.ERR_UNSUPPORTED
    assert g(_lib.INT8_SYM, A16, 1, A16b, A16c, None, 16, 256, 128, A16e, None) == _lib.ERR_FORMAT
    assert g(_lib.INT4_ASYM, A16, 1, A16b, A16c, None, 16, 256, 128, A16e, None) == _lib.ERR_NULL
    assert g(_lib.INT4_SYM, MIS, 1, A16b, A16c, None, 16, 256, 128, A16e, None) == _lib.ERR_ALIGN
    assert g(_lib.INT4_SYM, A16, 1, A16b, A16c, None, 16, 256, 128, None, None) == _lib.ERR_NULL


def test_qgemm_validation(lib):
    g = lib.qg_qgemm
    i4, bf, f8, i8 = _lib.INT4_SYM, _lib.BF16_ACT, _lib.FP8_E4M3, _lib.INT8_SYM
    assert g(i4, f8, A16, None, None, 8, A16b, A16c, None, 8, 256, 128, A16e, None) == _lib.ERR_FORMAT
    assert g(i4, bf, A16, None, None, 0, A16b, A16c, None, 8, 256, 128, A16e, None) == _lib.ERR_GEOMETRY
    assert g(i4, bf, A16, None, None, 8, A16b, A16c, None, 8, 384, 96, A16e, None) == _lib.ERR_UNSUPPORTED
    assert g(f8, f8, A16, A16d, None, 8, A16b, A16c, None, 8, 256, 128, A16e, None) == _lib.ERR_UNSUPPORTED
    assert g(f8, f8, A16, None, None, 8, A16b, A16c, None, 8, 256, 256, A16e, None) == _lib.ERR_NULL
    assert g(i8, _lib.INT8_ASYM, A16, A16d, None, 8, A16b, A16c, None, 8, 256, 256, A16e,
             None) == _lib.ERR_NULL
    assert g(f8, f8, A16, A16d, None, 8, A16b, A16c, None, 8, 8, 8, A16e, None) == _lib.ERR_GEOMETRY


def test_mx_validation(lib):
    assert lib.qg_mx_quant(A16, _lib.BF16, 4, 48, A16b, A16c, None) == _lib.ERR_GEOMETRY
    assert lib.qg_mx_quant(A16, _lib.BF16, 4, 0, A16b, A16c, None) == _lib.ERR_GEOMETRY
    assert lib.qg_mx_quant(A16, _lib.BF16, 4, 64, None, A16c, None) == _lib.ERR_NULL
    assert lib.qg_mx_quant(MIS, _lib.BF16, 4, 64, A16b, A16c, None) == _lib.ERR_ALIGN
    assert lib.qg_mx_gemm(A16, A16b, 4, A16c, A16d, 4, 40, A16e, None) == _lib.ERR_GEOMETRY
    assert lib.qg_mx_gemm(A16, A16b, 4, A16c, A16d, 0, 64, A16e, None) == _lib.ERR_GEOMETRY
    assert lib.qg_mx_gemm(A16, None, 4, A16c, A16d, 4, 64, A16e, None) == _lib.ERR_NULL
    assert lib.qg_mx_gemm(A16, A16b, 4, A16c, A16d, 4, 64, MIS, None) == _lib.ERR_ALIGN


def test_norm_quant_validation(lib):
    n = lib.qg_norm_quant
    L, R = _lib.NORM_LAYER, _lib.NORM_RMS
    f8, s8, a8 = _lib.FP8_E4M3, _lib.INT8_SYM, _lib.INT8_ASYM
    e = ctypes.c_float(1e-5)
    ok = (A16, _lib.BF16, A16b, A16c, e, 4, 256, A16d, A16e, None, None)
    assert n(7, f8, *ok) == _lib.ERR_FORMAT
    assert n(L, _lib.INT4_SYM, *ok) == _lib.ERR_FORMAT
    assert n(L, f8, A16, 9, A16b, A16c, e, 4, 256, A16d, A16e, None, None) == _lib.ERR_FORMAT
    assert n(L, f8, A16, _lib.BF16, A16b, A16c, e, 4, 260, A16d, A16e, None, None) == _lib.ERR_GEOMETRY
    assert n(L, f8, A16, _lib.BF16, A16b, A16c, e, 0, 256, A16d, A16e, None, None) == _lib.ERR_GEOMETRY
    assert n(L, f8, A16, _lib.BF16, A16b, A16c, ctypes.c_float(-1.0), 4, 256, A16d, A16e, None,
             None) == _lib.ERR_GEOMETRY
    assert n(L, f8, A16, _lib.BF16, A16b, None, e, 4, 256, A16d, A16e, None, None) == _lib.ERR_NULL
    assert n(R, f8, *ok) == _lib.ERR_NULL                  # RMSNorm takes no beta
    assert n(L, a8, *ok) == _lib.ERR_NULL                  # asymmetric needs zeros
    assert n(L, s8, A16, _lib.BF16, MIS, A16c, e, 4, 256, A16d, A16e, None, None) == _lib.ERR_ALIGN
    assert n(L, f8, A16, _lib.BF16, A16b, A16c, e, 4, 16392, A16d, A16e, None,
             None) == _lib.ERR_UNSUPPORTED
    mx = _lib.MXFP4
    assert n(L, mx, A16, _lib.BF16, A16b, A16c, e, 4, 264, A16d, A16e, None,
             None) == _lib.ERR_GEOMETRY                       # K % 32
    assert n(L, mx, A16, _lib.BF16, A16b, A16c, e, 4, 256, A16d, A16e, A16, None) == _lib.ERR_NULL
    assert n(L, mx, A16, _lib.BF16, A16b, A16c, e, 4, 256, A16d, None, None, None) == _lib.ERR_NULL


def test_qgemm_swiglu_validation(lib):
    f = lib.qg_qgemm_swiglu
    i4, bf = _lib.INT4_SYM, _lib.BF16_ACT
    assert f(_lib.FP8_E4M3, bf, A16, 4, A16b, A16c, None, 64, 256, 128, A16e, None) == _lib.ERR_FORMAT
    assert f(i4, _lib.INT8_SYM, A16, 4, A16b, A16c, None, 64, 256, 128, A16e, None) == _lib.ERR_FORMAT
    assert f(i4, bf, A16, 4, A16b, A16c, None, 63, 256, 128, A16e, None) == _lib.ERR_GEOMETRY
    assert f(i4, bf, A16, 0, A16b, A16c, None, 64, 256, 128, A16e, None) == _lib.ERR_GEOMETRY
    assert f(i4, bf, A16, 4, A16b, A16c, None, 64, 256, 100, A16e, None) == _lib.ERR_GEOMETRY
    assert f(i4, bf, None, 4, A16b, A16c, None, 64, 256, 128, A16e, None) == _lib.ERR_NULL
    assert f(_lib.INT4_ASYM, bf, A16, 4, A16b, A16c, None, 64, 256, 128, A16e, None) == _lib.ERR_NULL
    assert f(i4, bf, A16, 4, A16b, A16c, None, 64, 256, 128, MIS, None) == _lib.ERR_ALIGN
    assert f(i4, bf, A16, 4, A16b, A16c, None, 64, 512, 256, A16e, None) == _lib.ERR_UNSUPPORTED


def test_python_raises_value_error_for_geometry(lib):
    assert lib.qg_qgemv(_lib.INT4_SYM, A16, 17, A16b, A16c, None, 16, 256, 128, A16e,
                        None) == _lib.ERR_GEOMETRY
    with pytest.raises(ValueError, match="invalid quantization geometry"):
        _lib.check(_lib.ERR_GEOMETRY)
    with pytest.raises(_lib.QGError):
        _lib.check(_lib.ERR_ALIGN)


def test_operands_past_32_bit_offsets_are_rejected(lib):
    # the kernels address each operand with 32-bit byte offsets (plus up to
    # 256 rows of tile overhang): larger operands are refused before any launch
    i4, bf, f8 = _lib.INT4_SYM, _lib.BF16_ACT, _lib.FP8_E4M3
    big = 1 << 19
    assert lib.qg_qgemm(f8, f8, A16, A16d, None, big, A16b, A16c, None, 8, 8192, 8192, A16e,
                        None) == _lib.ERR_UNSUPPORTED
    assert lib.qg_qgemm(i4, bf, A16, None, None, big, A16b, A16c, None, 8, 8192, 128, A16e,
                        None) == _lib.ERR_UNSUPPORTED
    assert lib.qg_mx_gemm(A16, A16b, 8, A16c, A16d, big * 2, 8192, A16e, None) == _lib.ERR_UNSUPPORTED
    assert lib.qg_qgemv(i4, A16, 1, A16b, A16c, None, 1 << 20, 8192, 128, A16e,
                        None) == _lib.ERR_UNSUPPORTED


def test_quantize_pack_smooth_validation(lib):
    q = lib.qg_quantize_pack_smooth
    ok = (_lib.INT4_SYM, A16, _lib.F32, 4, 256, 128, A16e, 0, A16b, A16c, None, None)
    assert q(*ok[:6], None, *ok[7:]) == _lib.ERR_NULL                   # no factors
    assert q(*ok[:6], MIS, *ok[7:]) == _lib.ERR_ALIGN                   # misaligned factors
    assert q(*ok[:7], 2, *ok[8:]) == _lib.ERR_GEOMETRY                  # divide not 0/1
    assert q(_lib.INT4_SYM, A16, _lib.F32, 4, 256, 100, A16e, 0, A16b, A16c, None,
             None) == _lib.ERR_GEOMETRY
    assert q(_lib.MXFP4, *ok[1:]) == _lib.ERR_FORMAT
    assert q(_lib.INT8_ASYM, *ok[1:]) == _lib.ERR_NULL                  # asym needs zeros


def test_channel_statistics_validation(lib):
    a = lib.qg_channel_absmax
    assert a(A16, _lib.BF16, 0, 256, 0, A16b, None) == _lib.ERR_GEOMETRY
    assert a(A16, _lib.BF16, 4, 12, 0, A16b, None) == _lib.ERR_GEOMETRY
    assert a(A16, _lib.BF16, 4, 256, 2, A16b, None) == _lib.ERR_GEOMETRY
    assert a(A16, 5, 4, 256, 0, A16b, None) == _lib.ERR_FORMAT
    assert a(None, _lib.BF16, 4, 256, 0, A16b, None) == _lib.ERR_NULL
    assert a(A16, _lib.BF16, 4, 256, 0, MIS, None) == _lib.ERR_ALIGN
    s = lib.qg_smooth_scales
    assert s(A16, A16b, ctypes.c_float(1.5), 64, A16c, None) == _lib.ERR_GEOMETRY
    assert s(A16, A16b, ctypes.c_float(-0.1), 64, A16c, None) == _lib.ERR_GEOMETRY
    assert s(A16, A16b, ctypes.c_float(float("nan")), 64, A16c, None) == _lib.ERR_GEOMETRY
    assert s(A16, A16b, ctypes.c_float(0.5), 0, A16c, None) == _lib.ERR_GEOMETRY
    assert s(A16, None, ctypes.c_float(0.5), 64, A16c, None) == _lib.ERR_NULL
    c = lib.qg_channel_scales
    assert c(A16, 64, ctypes.c_float(0.0), A16b, None) == _lib.ERR_GEOMETRY
    assert c(A16, 64, ctypes.c_float(float("inf")), A16b, None) == _lib.ERR_GEOMETRY
    assert c(A16, 0, ctypes.c_float(448.0), A16b, None) == _lib.ERR_GEOMETRY
    assert c(MIS, 64, ctypes.c_float(448.0), A16b, None) == _lib.ERR_ALIGN


def test_kv_cache_store_validation(lib):
    k = lib.qg_kv_cache_store
    # x, dtype, tokens, heads, head_dim, slots, num_slots, channel_scales, codes, scales
    tok = (A16, _lib.BF16, 4, 8, 128, A16b, 64, None, A16c, A16d, None)
    ch = (A16, _lib.BF16, 4, 8, 128, A16b, 64, A16e, A16c, None, None)
    assert k(*tok[:4], 100, *tok[5:]) == _lib.ERR_GEOMETRY             # head_dim % 8
    assert k(*tok[:4], 1024, *tok[5:]) == _lib.ERR_GEOMETRY            # head_dim > 512
    assert k(*tok[:3], 0, *tok[4:]) == _lib.ERR_GEOMETRY               # heads
    assert k(*tok[:6], 0, *tok[7:]) == _lib.ERR_GEOMETRY               # num_slots
    assert k(*tok[:2], -1, *tok[3:]) == _lib.ERR_GEOMETRY              # tokens
    assert k(*tok[:9], None, None) == _lib.ERR_NULL                     # per token needs scales
    assert k(*ch[:9], A16d, None) == _lib.ERR_NULL                      # both scale kinds
    assert k(*tok[:5], None, *tok[6:]) == _lib.ERR_NULL                 # no slot mapping
    assert k(*tok[:2], 1 << 28, 16, *tok[4:]) == _lib.ERR_UNSUPPORTED   # tokens * heads >= 2^31
    assert k(*tok[:5], vp(0x2004), *tok[6:]) == _lib.ERR_ALIGN          # slots 8-byte
    assert k(*tok[:8], vp(0x3004), *tok[9:]) == _lib.ERR_ALIGN          # codes 8-byte
    assert k(*tok[:9], vp(0x4002), None) == _lib.ERR_ALIGN              # scales 4-byte
    assert k(*ch[:7], vp(0x5008), *ch[8:]) == _lib.ERR_ALIGN            # channel scales 16
    assert k(A16, 9, *tok[2:]) == _lib.ERR_FORMAT
    # no tokens: valid, nothing is enqueued (no HIP call is made)
    assert k(None, _lib.BF16, 0, 8, 128, A16b, 64, None, A16c, A16d, None) == _lib.OK
    assert k(None, _lib.BF16, 0, 8, 128, None, 64, None, A16c, A16d, None) == _lib.OK


def test_binding_rejects_mismatched_operands_before_any_call():
    # the binding checks shapes, dtypes and outputs before it touches the
    # library (the C ABI cannot see tensor extents); CPU tensors suffice
    # because the device check comes after the shapes
    import torch
    import quantized_gemm_group_amd as qg
    m, k, n = 2, 256, 16
    x = torch.zeros((m, k), dtype=torch.bfloat16)
    codes = torch.zeros((n, k // 8), dtype=torch.int32)
    s = torch.zeros((n, k // 128), dtype=torch.float16)
    z = torch.zeros((n, k // 128), dtype=torch.float16)
    y = torch.zeros((m, n), dtype=torch.bfloat16)

    def bad(match, fn, *a, **kw):
        with pytest.raises(ValueError, match=match):
            fn(*a, **kw)

    # well formed: only the device check is left
    bad("must live on the GPU", qg.qgemv, x, codes, s, z, "int4_asym", out=y)
    bad("out must be", qg.qgemv, x, codes, s, z, "int4_asym", out=y[:, :8])
    bad("out must be", qg.qgemv, x, codes, s, z, "int4_asym", out=y.float())
    bad("weight codes", qg.qgemv, x, codes[:, :16], s, z, "int4_asym")
    bad("weight codes", qg.qgemv, torch.zeros((m, 2 * k), dtype=torch.bfloat16), codes, s, z,
        "int4_asym")
    bad("weight scales", qg.qgemv, x, codes, s[:, :1], z, "int4_asym")
    bad("weight scales", qg.qgemv, x, codes, s.float(), z, "int4_asym")
    bad("weight zeros", qg.qgemv, x, codes, s, None, "int4_asym")
    bad("weight zeros must be None", qg.qgemv, x, codes, s, z, "int4_sym")
    bad("x must be bf16", qg.qgemv, x.float(), codes, s, z, "int4_asym")
    bad("weight scales", qg.qgemm, x, codes[:8], s, z, "int4_asym", "bf16")
    bad("a_scales must be None", qg.qgemm, x, codes, s, z, "int4_asym", "bf16",
        a_scales=torch.ones(m))
    bad("must live on the GPU", qg.qgemm, x, codes, s, z, "int4_asym", "bf16", out=y)
    # FP8 W8A8: per-row scales of both operands
    a8 = torch.zeros((m, k), dtype=torch.uint8)
    w8 = torch.zeros((n, k), dtype=torch.uint8)
    ws, as_ = torch.ones((n, 1)), torch.ones((m, 1))
    bad("must live on the GPU", qg.qgemm, a8, w8, ws, None, "fp8_e4m3", "fp8_e4m3", a_scales=as_)
    bad("a_scales", qg.qgemm, a8, w8, ws, None, "fp8_e4m3", "fp8_e4m3", a_scales=as_[:1])
    bad("a_scales", qg.qgemm, a8, w8, ws, None, "fp8_e4m3", "fp8_e4m3", a_scales=None)
    bad("weight scales", qg.qgemm, a8, w8, ws[:4], None, "fp8_e4m3", "fp8_e4m3", a_scales=as_)
    bad("weight codes", qg.qgemm, a8, w8[:, :128], ws, None, "fp8_e4m3", "fp8_e4m3", a_scales=as_)
    bad("activation codes", qg.qgemm, a8.to(torch.int8), w8, ws, None, "fp8_e4m3", "fp8_e4m3",
        a_scales=as_)
    bad("a_zeros", qg.qgemm, a8, w8.to(torch.int8), ws, None, "int8_sym", "int8_asym",
        a_scales=as_)
    # SwiGLU and MXFP4
    bad("out must be", qg.qgemm_swiglu, x, codes, s, None, "int4_sym", out=y)
    bad("even row count", qg.qgemm_swiglu, x, codes[:15], s[:15], None, "int4_sym")
    mc, me = torch.zeros((m, k // 2), dtype=torch.uint8), torch.zeros((m, k // 32), dtype=torch.uint8)
    bc, be = torch.zeros((n, k // 2), dtype=torch.uint8), torch.zeros((n, k // 32), dtype=torch.uint8)
    bad("must live on the GPU", qg.mx_gemm, mc, me, bc, be, out=y)
    bad("b_e8m0", qg.mx_gemm, mc, me, bc, be[:, :4])
    bad("a_e8m0", qg.mx_gemm, mc, me[:1], bc, be)
    bad("out must be", qg.mx_gemm, mc, me, bc, be, out=y.t())
    bad("codes", qg.dequant, codes[:, :4], s, z, "int4_asym", k)


def test_tiled_gemv_validation(lib):
    t = lib.qg_tile_gemv_weights
    assert t(A16, 0, 256, A16b, None) == _lib.ERR_GEOMETRY
    assert t(A16, 16, 200, A16b, None) == _lib.ERR_GEOMETRY
    assert t(A16, 16, 65536 * 2, A16b, None) == _lib.ERR_UNSUPPORTED
    assert t(A16, 16, 256, A16, None) == _lib.ERR_UNSUPPORTED           # in place
    assert t(None, 16, 256, A16b, None) == _lib.ERR_NULL
    assert t(MIS, 16, 256, A16b, None) == _lib.ERR_ALIGN
    g = lib.qg_qgemv_tiled
    assert g(_lib.INT4_SYM, A16, 17, A16b, A16c, None, 16, 256, 128, A16e, None) == _lib.ERR_GEOMETRY
    assert g(_lib.INT8_SYM, A16, 1, A16b, A16c, None, 16, 256, 128, A16e, None) == _lib.ERR_FORMAT
    assert g(_lib.INT4_ASYM, A16, 1, A16b, A16c, None, 16, 256, 128, A16e, None) == _lib.ERR_NULL


def test_qgemv_swiglu_validation(lib):
    f = lib.qg_qgemv_swiglu
    i4 = _lib.INT4_SYM
    ok = (A16, 1, A16b, A16c, None, 64, 4096, 128, 0, A16e, None)
    assert f(_lib.INT8_SYM, *ok) == _lib.ERR_FORMAT
    assert f(i4, A16, 17, *ok[2:]) == _lib.ERR_GEOMETRY
    assert f(i4, *ok[:5], 63, *ok[6:]) == _lib.ERR_GEOMETRY             # odd N2
    assert f(i4, *ok[:8], 2, *ok[9:]) == _lib.ERR_GEOMETRY              # tiled flag
    assert f(i4, *ok[:6], 4096, 64, *ok[8:]) == _lib.ERR_UNSUPPORTED    # group
    assert f(i4, *ok[:6], 640, *ok[7:]) == _lib.ERR_UNSUPPORTED         # K % 512
    assert f(i4, A16, 8, *ok[2:6], 16384, *ok[7:]) == _lib.ERR_UNSUPPORTED   # M > 4, K > 8192
    assert f(_lib.INT4_ASYM, *ok) == _lib.ERR_NULL
    assert f(i4, *ok[:9], MIS, None) == _lib.ERR_ALIGN


def test_qgemm_swiglu_fp8_validation(lib):
    f = lib.qg_qgemm_swiglu_fp8
    ok = (A16, A16b, 8, A16c, A16d, 64, 256, A16e, None)
    assert f(*ok[:5], 63, *ok[6:]) == _lib.ERR_GEOMETRY                 # odd N2
    assert f(*ok[:6], 200, *ok[7:]) == _lib.ERR_GEOMETRY                # K % 16
    assert f(A16, A16b, 0, *ok[3:]) == _lib.ERR_GEOMETRY
    assert f(A16, None, *ok[2:]) == _lib.ERR_NULL
    assert f(*ok[:7], None, None) == _lib.ERR_NULL
    assert f(*ok[:7], MIS, None) == _lib.ERR_ALIGN
    assert f(A16, A16b, 1 << 20, *ok[3:6], 8192, A16e, None) == _lib.ERR_UNSUPPORTED


def test_debug_library_loads_and_product_library_refuses_recording(lib):
    assert lib.qg_debug_build() == 0
    assert lib.qg_debug_fp32_output(None, None) == _lib.ERR_UNSUPPORTED
    dlib = _lib.load_debug()
    assert dlib.qg_debug_build() == 1
    for name in _lib.EXPORTS:
        assert hasattr(dlib, name), name
    assert dlib.qg_debug_fp32_output(vp(0x1002), None) == _lib.ERR_ALIGN
