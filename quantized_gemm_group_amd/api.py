"""Python binding of the C ABI: the same operations, torch tensors in and out.

Marshalling only: every function checks tensor placement, dtypes and
shapes (the C ABI takes raw pointers and sizes, so a mis-shaped operand or
output cannot be detected past this layer), allocates its outputs with torch
on the input's device, and makes ONE call into libqgemm.so on the current
HIP stream.  No arithmetic of the method
happens here.
"""

from __future__ import annotations

import ctypes

import torch

from . import _lib

FORMATS = {
    "int4_sym": _lib.INT4_SYM,
    "int4_asym": _lib.INT4_ASYM,
    "int8_sym": _lib.INT8_SYM,
    "int8_asym": _lib.INT8_ASYM,
    "fp8_e4m3": _lib.FP8_E4M3,
    "bf16": _lib.BF16_ACT,
    "mxfp4": _lib.MXFP4,
}
_ASYM = {"int4_asym", "int8_asym"}


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _dev(t: torch.Tensor) -> torch.device:
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.device


def _src_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return _lib.BF16
    if t.dtype == torch.float32:
        return _lib.F32
    raise ValueError("source must be bf16 or fp32")


def _expect(t, shape, dtype, what: str, dev=None):
    """Raise ValueError unless t is a contiguous tensor of exactly this shape
    and dtype (on dev when given).  The C ABI takes raw pointers and sizes,
    so a mis-shaped operand cannot be detected past this point."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{what} must be a tensor")
    if t.dtype != dtype or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what} must be {dtype} of shape {tuple(shape)}, got {t.dtype} "
                         f"{tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if dev is not None and t.device != dev:
        raise ValueError(f"{what} must be on {dev}, got {t.device}")


def _expect_rows(t, rows: int, what: str, dev=None):
    """A per-row fp32 vector of `rows` values: shape [rows] or [rows][1]."""
    if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or \
            tuple(t.shape) not in ((rows,), (rows, 1)):
        raise ValueError(f"{what} must be fp32 of shape [{rows}] or [{rows}][1]")
    _expect(t, t.shape, torch.float32, what, dev)


def _expect_none(t, what: str):
    if t is not None:
        raise ValueError(f"{what} must be None for this format")


def _weights(fmt: str, codes, scales, zeros, n: int, k: int, group: int, dev):
    """The stored operand of quantize_pack: codes, scales (+ zeros)."""
    if fmt not in FORMATS or fmt in ("bf16", "mxfp4"):
        raise ValueError(f"unknown weight format {fmt}")
    if group <= 0 or k % group:
        raise ValueError("invalid quantization geometry: group must divide K")
    cshape, cdt, sdt = _code_shapes(fmt, n, k, group)
    _expect(codes, cshape, cdt, "weight codes", dev)
    # one scale per row (group == K) may also come as a flat [rows] vector
    sshape = (n, k // group)
    if group == k and isinstance(scales, torch.Tensor) and scales.dim() == 1:
        sshape = (n,)
    _expect(scales, sshape, sdt, "weight scales", dev)
    if fmt in _ASYM:
        _expect(zeros, sshape, sdt, "weight zeros", dev)
    else:
        _expect_none(zeros, "weight zeros")


def _code_shapes(fmt: str, rows: int, k: int, group: int):
    """(codes shape, codes dtype, scale dtype) of the storage format."""
    if fmt.startswith("int4"):
        return (rows, k // 8), torch.int32, torch.float16
    if fmt == "int8_sym":
        return (rows, k), torch.int8, torch.float32
    if fmt in ("int8_asym", "fp8_e4m3"):
        return (rows, k), torch.uint8, torch.float32
    raise ValueError(f"unknown format {fmt}")


def default_group(fmt: str, k: int) -> int:
    return 128 if fmt.startswith("int4") else k


def quantize_pack(x: torch.Tensor, fmt: str, group: int | None = None):
    """Quantize x [rows][K] (bf16 or fp32) along K.  Returns
    (codes, scales, zeros or None) in the storage format of include/qgemm.h."""
    lib = _lib.load()
    dev = _dev(x)
    rows, k = x.shape
    group = default_group(fmt, k) if group is None else group
    if group <= 0 or k % group:
        raise ValueError("invalid quantization geometry: group must divide K")
    cshape, cdt, sdt = _code_shapes(fmt, rows, k, group)
    codes = torch.empty(cshape, dtype=cdt, device=dev)
    scales = torch.empty((rows, k // group), dtype=sdt, device=dev)
    zeros = torch.empty_like(scales) if fmt in _ASYM else None
    _lib.check(lib.qg_quantize_pack(FORMATS[fmt], _ptr(x), _src_dtype(x), rows, k, group,
                                    _ptr(codes), _ptr(scales), _ptr(zeros), _stream(dev)))
    return codes, scales, zeros


NORMS = {"layer": _lib.NORM_LAYER, "rms": _lib.NORM_RMS}


def norm_quant(x: torch.Tensor, gamma: torch.Tensor, beta: torch.Tensor | None = None,
               fmt: str = "fp8_e4m3", norm: str = "layer", eps: float = 1e-5):
    """Fused LayerNorm ("layer", needs beta) or RMSNorm ("rms", beta None) of
    each row of x [rows][K] (bf16 or fp32) followed by its per-row dynamic
    quantization ("fp8_e4m3", "int8_sym", "int8_asym"), or its MXFP4
    quantization ("mxfp4").  gamma, beta: fp32 [K].  Returns (codes
    [rows][K], scales fp32 [rows][1], zeros or None); for "mxfp4" (codes
    uint8 [rows][K/2], E8M0 exponents uint8 [rows][K/32], None)."""
    lib = _lib.load()
    dev = _dev(x)
    if norm not in NORMS:
        raise ValueError(f"unknown normalization {norm}")
    if fmt not in ("fp8_e4m3", "int8_sym", "int8_asym", "mxfp4"):
        raise ValueError(f"norm_quant: unsupported format {fmt}")
    rows, k = x.shape
    for t, what in ((gamma, "gamma"), (beta, "beta")):
        if t is not None:
            _f32_vec(t, dev, k, what)
    if fmt == "mxfp4":
        if k % 32:
            raise ValueError("invalid quantization geometry: K must be a multiple of 32")
        codes = torch.empty((rows, k // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((rows, k // 32), dtype=torch.uint8, device=dev)
        zeros = None
    else:
        cshape, cdt, sdt = _code_shapes(fmt, rows, k, k)
        codes = torch.empty(cshape, dtype=cdt, device=dev)
        scales = torch.empty((rows, 1), dtype=sdt, device=dev)
        zeros = torch.empty_like(scales) if fmt in _ASYM else None
    _lib.check(lib.qg_norm_quant(NORMS[norm], FORMATS[fmt], _ptr(x), _src_dtype(x), _ptr(gamma),
                                 _ptr(beta), ctypes.c_float(eps), rows, k, _ptr(codes),
                                 _ptr(scales), _ptr(zeros), _stream(dev)))
    return codes, scales, zeros


def dequant(codes: torch.Tensor, scales: torch.Tensor, zeros, fmt: str, k: int,
            group: int | None = None, out_dtype=torch.float32) -> torch.Tensor:
    """x_hat = s * (q - z) (or 2^e * e2m1 for "mxfp4") as [rows][K]."""
    dev = codes.device        # checked for the GPU below, after the shapes
    rows = codes.shape[0]
    group = (32 if fmt == "mxfp4" else default_group(fmt, k)) if group is None else group
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("out_dtype must be bf16 or fp32")
    if fmt == "mxfp4":
        if group != 32 or k % 32:
            raise ValueError("invalid quantization geometry: MX blocks are 32 elements")
        _expect(codes, (rows, k // 2), torch.uint8, "codes", dev)
        _expect(scales, (rows, k // 32), torch.uint8, "e8m0 scales", dev)
        _expect_none(zeros, "zeros")
    else:
        _weights(fmt, codes, scales, zeros, rows, k, group, dev)
    _dev(codes)
    lib = _lib.load()
    out = torch.empty((rows, k), dtype=out_dtype, device=dev)
    dt = _lib.BF16 if out_dtype == torch.bfloat16 else _lib.F32
    _lib.check(lib.qg_dequant(FORMATS[fmt], _ptr(codes), _ptr(scales), _ptr(zeros), rows, k,
                              group, _ptr(out), dt, _stream(dev)))
    return out


def qgemv(x: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, zeros, fmt: str,
          group: int = 128, out: torch.Tensor | None = None) -> torch.Tensor:
    """W4A16 decode product y = x * dequant(W)^T for 1 <= M <= 16; x bf16 [M][K]."""
    dev = x.device        # checked for the GPU below, after the shapes
    if x.dtype != torch.bfloat16 or x.dim() != 2:
        raise ValueError("x must be bf16 [M][K]")
    if not fmt.startswith("int4"):
        raise ValueError("qgemv: weights must be int4_sym or int4_asym")
    m, k = x.shape
    n = codes.shape[0]
    _weights(fmt, codes, scales, zeros, n, k, group, dev)
    if out is not None:
        _expect(out, (m, n), torch.bfloat16, "out", dev)
    _dev(x)
    lib = _lib.load()
    y = torch.empty((m, n), dtype=torch.bfloat16, device=dev) if out is None else out
    _lib.check(lib.qg_qgemv(FORMATS[fmt], _ptr(x), m, _ptr(codes), _ptr(scales), _ptr(zeros),
                            n, k, group, _ptr(y), _stream(dev)))
    return y


class TiledCodes:
    """INT4 codes of an [N][K] weight in the decode GEMV's tile layout (the
    one-time relayout of tile_gemv_weights): `data` holds ceil(N/16)*16*K/2
    bytes; n and k are the weight's sizes."""

    def __init__(self, data: torch.Tensor, n: int, k: int):
        self.data, self.n, self.k = data, n, k

    @property
    def device(self):
        return self.data.device


def tile_gemv_weights(codes: torch.Tensor, k: int | None = None) -> TiledCodes:
    """Relayout of canonical INT4 codes (int32 [N][K/8]) into the decode GEMV's
    tile layout (1 KiB per 16 rows x one group of 128)."""
    dev = codes.device
    if codes.dim() != 2 or codes.dtype != torch.int32:
        raise ValueError("codes must be int32 [N][K/8]")
    n = codes.shape[0]
    k = codes.shape[1] * 8 if k is None else k
    _expect(codes, (n, k // 8), torch.int32, "codes", dev)
    if k % 128:
        raise ValueError("invalid quantization geometry: K must be a multiple of 128")
    _dev(codes)
    lib = _lib.load()
    out = torch.empty(((n + 15) // 16 * 16 * k // 2,), dtype=torch.uint8, device=dev)
    _lib.check(lib.qg_tile_gemv_weights(_ptr(codes), n, k, _ptr(out), _stream(dev)))
    return TiledCodes(out, n, k)


def qgemv_tiled(x: torch.Tensor, codes: TiledCodes, scales: torch.Tensor, zeros, fmt: str,
                group: int = 128, out: torch.Tensor | None = None) -> torch.Tensor:
    """qgemv on tiled codes (tile_gemv_weights); same results as qgemv."""
    dev = x.device        # checked for the GPU below, after the shapes
    if not isinstance(codes, TiledCodes):
        raise ValueError("codes must come from tile_gemv_weights")
    if x.dtype != torch.bfloat16 or x.dim() != 2:
        raise ValueError("x must be bf16 [M][K]")
    if not fmt.startswith("int4"):
        raise ValueError("qgemv: weights must be int4_sym or int4_asym")
    m, k = x.shape
    n = codes.n
    if codes.k != k:
        raise ValueError(f"tiled codes are for K={codes.k}, x has K={k}")
    _expect(codes.data, ((n + 15) // 16 * 16 * k // 2,), torch.uint8, "tiled codes", dev)
    if group <= 0 or k % group:
        raise ValueError("invalid quantization geometry: group must divide K")
    _expect(scales, (n, k // group), torch.float16, "weight scales", dev)
    if fmt in _ASYM:
        _expect(zeros, (n, k // group), torch.float16, "weight zeros", dev)
    else:
        _expect_none(zeros, "weight zeros")
    if out is not None:
        _expect(out, (m, n), torch.bfloat16, "out", dev)
    _dev(x)
    lib = _lib.load()
    y = torch.empty((m, n), dtype=torch.bfloat16, device=dev) if out is None else out
    _lib.check(lib.qg_qgemv_tiled(FORMATS[fmt], _ptr(x), m, _ptr(codes.data), _ptr(scales),
                                  _ptr(zeros), n, k, group, _ptr(y), _stream(dev)))
    return y


def qgemv_swiglu(x: torch.Tensor, codes, scales: torch.Tensor, zeros, fmt: str,
                 group: int = 128, out: torch.Tensor | None = None) -> torch.Tensor:
    """Fused SwiGLU decode projection h = SiLU(x W_gate^T) * (x W_up^T) for
    1 <= M <= 16 rows of bf16 x [M][K] and INT4 weights quantized as the
    [2I][K] concatenation [W_gate; W_up]; codes canonical (int32 [2I][K/8])
    or TiledCodes of that concatenation.  Returns h bf16 [M][I]."""
    dev = x.device        # checked for the GPU below, after the shapes
    if x.dtype != torch.bfloat16 or x.dim() != 2:
        raise ValueError("x must be bf16 [M][K]")
    if not fmt.startswith("int4"):
        raise ValueError("qgemv_swiglu: weights must be int4_sym or int4_asym")
    m, k = x.shape
    tiled = isinstance(codes, TiledCodes)
    if tiled:
        n2 = codes.n
        if codes.k != k:
            raise ValueError(f"tiled codes are for K={codes.k}, x has K={k}")
        _expect(codes.data, ((n2 + 15) // 16 * 16 * k // 2,), torch.uint8, "tiled codes", dev)
        data = codes.data
    else:
        n2 = codes.shape[0]
        _expect(codes, (n2, k // 8), torch.int32, "weight codes", dev)
        data = codes
    if n2 % 2:
        raise ValueError("invalid quantization geometry: [W_gate; W_up] needs an even row count")
    if group <= 0 or k % group:
        raise ValueError("invalid quantization geometry: group must divide K")
    _expect(scales, (n2, k // group), torch.float16, "weight scales", dev)
    if fmt in _ASYM:
        _expect(zeros, (n2, k // group), torch.float16, "weight zeros", dev)
    else:
        _expect_none(zeros, "weight zeros")
    if out is not None:
        _expect(out, (m, n2 // 2), torch.bfloat16, "out", dev)
    _dev(x)
    lib = _lib.load()
    h = torch.empty((m, n2 // 2), dtype=torch.bfloat16, device=dev) if out is None else out
    _lib.check(lib.qg_qgemv_swiglu(FORMATS[fmt], _ptr(x), m, _ptr(data), _ptr(scales),
                                   _ptr(zeros), n2, k, group, 1 if tiled else 0, _ptr(h),
                                   _stream(dev)))
    return h


def qgemm(a: torch.Tensor, w_codes: torch.Tensor, w_scales: torch.Tensor, w_zeros, wfmt: str,
          afmt: str, a_scales=None, a_zeros=None, k: int | None = None,
          group: int | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """Quantized GEMM y = dequant(a) * dequant(W)^T with bf16 output.
    Pairs: (int4_*, "bf16"), ("fp8_e4m3", "fp8_e4m3"), (int8_*, int8_*)."""
    dev = a.device        # checked for the GPU below, after the shapes
    if a.dim() != 2:
        raise ValueError("a must be [M][K]")
    m = a.shape[0]
    if k is not None and k != a.shape[1]:
        raise ValueError("k must equal a.shape[1]")
    k = a.shape[1]
    n = w_codes.shape[0]
    group = default_group(wfmt, k) if group is None else group
    pair = ((wfmt in ("int4_sym", "int4_asym") and afmt == "bf16")
            or (wfmt == "fp8_e4m3" and afmt == "fp8_e4m3")
            or (wfmt in ("int8_sym", "int8_asym") and afmt in ("int8_sym", "int8_asym")))
    if not pair:
        pass                      # the library reports the unsupported pair (QG_ERR_FORMAT)
    elif afmt == "bf16":
        _weights(wfmt, w_codes, w_scales, w_zeros, n, k, group, dev)
        if a.dtype != torch.bfloat16:
            raise ValueError("a must be bf16 for bf16 activations")
        _expect_none(a_scales, "a_scales")
        _expect_none(a_zeros, "a_zeros")
    else:
        _weights(wfmt, w_codes, w_scales, w_zeros, n, k, group, dev)
        _expect(a, (m, k), _code_shapes(afmt, m, k, k)[1], "a (activation codes)", dev)
        _expect_rows(a_scales, m, "a_scales", dev)
        if afmt in _ASYM:
            _expect_rows(a_zeros, m, "a_zeros", dev)
        else:
            _expect_none(a_zeros, "a_zeros")
    if out is not None:
        _expect(out, (m, n), torch.bfloat16, "out", dev)
    _dev(a)
    lib = _lib.load()
    y = torch.empty((m, n), dtype=torch.bfloat16, device=dev) if out is None else out
    _lib.check(lib.qg_qgemm(FORMATS[wfmt], FORMATS[afmt], _ptr(a), _ptr(a_scales), _ptr(a_zeros),
                            m, _ptr(w_codes), _ptr(w_scales), _ptr(w_zeros), n, k, group,
                            _ptr(y), _stream(dev)))
    return y


def qgemm_swiglu(a: torch.Tensor, w_codes: torch.Tensor, w_scales: torch.Tensor, w_zeros,
                 wfmt: str, group: int = 128, out: torch.Tensor | None = None) -> torch.Tensor:
    """Fused SwiGLU projection h = SiLU(a W_gate^T) * (a W_up^T) with bf16 a
    [M][K] and INT4 weights quantized as the [2I][K] concatenation
    [W_gate; W_up].  Returns h bf16 [M][I]."""
    dev = a.device        # checked for the GPU below, after the shapes
    if a.dtype != torch.bfloat16 or a.dim() != 2:
        raise ValueError("a must be bf16 [M][K]")
    if not wfmt.startswith("int4"):
        raise ValueError("qgemm_swiglu: weights must be int4_sym or int4_asym")
    m, k = a.shape
    n2 = w_codes.shape[0]
    if n2 % 2:
        raise ValueError("invalid quantization geometry: [W_gate; W_up] needs an even row count")
    _weights(wfmt, w_codes, w_scales, w_zeros, n2, k, group, dev)
    if out is not None:
        _expect(out, (m, n2 // 2), torch.bfloat16, "out", dev)
    _dev(a)
    lib = _lib.load()
    h = torch.empty((m, n2 // 2), dtype=torch.bfloat16, device=dev) if out is None else out
    _lib.check(lib.qg_qgemm_swiglu(FORMATS[wfmt], FORMATS["bf16"], _ptr(a), m, _ptr(w_codes),
                                   _ptr(w_scales), _ptr(w_zeros), n2, k, group, _ptr(h),
                                   _stream(dev)))
    return h


def qgemm_swiglu_fp8(a_codes: torch.Tensor, a_scales: torch.Tensor, w_codes: torch.Tensor,
                     w_scales: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Fused SwiGLU projection of FP8 W8A8: h = SiLU(g) * u with g, u the
    rescaled code products over the gate and up rows of the per-row FP8
    quantized [2I][K] concatenation [W_gate; W_up]; a_codes uint8 [M][K]
    with per-token scales.  Returns h bf16 [M][I]."""
    dev = a_codes.device        # checked for the GPU below, after the shapes
    if a_codes.dim() != 2 or w_codes.dim() != 2:
        raise ValueError("codes must be [rows][K]")
    m, k = a_codes.shape
    n2 = w_codes.shape[0]
    if n2 % 2:
        raise ValueError("invalid quantization geometry: [W_gate; W_up] needs an even row count")
    _expect(a_codes, (m, k), torch.uint8, "a_codes", dev)
    _expect_rows(a_scales, m, "a_scales", dev)
    _expect(w_codes, (n2, k), torch.uint8, "w_codes", dev)
    _expect_rows(w_scales, n2, "w_scales", dev)
    if out is not None:
        _expect(out, (m, n2 // 2), torch.bfloat16, "out", dev)
    _dev(a_codes)
    lib = _lib.load()
    h = torch.empty((m, n2 // 2), dtype=torch.bfloat16, device=dev) if out is None else out
    _lib.check(lib.qg_qgemm_swiglu_fp8(_ptr(a_codes), _ptr(a_scales), m, _ptr(w_codes),
                                       _ptr(w_scales), n2, k, _ptr(h), _stream(dev)))
    return h


def mx_quant(x: torch.Tensor):
    """OCP MXFP4 quantization of x [rows][K] along K.  Returns (codes uint8
    [rows][K/2], e8m0 uint8 [rows][K/32])."""
    lib = _lib.load()
    dev = _dev(x)
    rows, k = x.shape
    if k % 32 or k == 0:
        raise ValueError("invalid quantization geometry: K must be a multiple of 32")
    codes = torch.empty((rows, k // 2), dtype=torch.uint8, device=dev)
    e8m0 = torch.empty((rows, k // 32), dtype=torch.uint8, device=dev)
    _lib.check(lib.qg_mx_quant(_ptr(x), _src_dtype(x), rows, k, _ptr(codes), _ptr(e8m0),
                               _stream(dev)))
    return codes, e8m0


def mx_gemm(a_codes: torch.Tensor, a_e8m0: torch.Tensor, b_codes: torch.Tensor,
            b_e8m0: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Block-scaled MXFP4 product y = A * B^T (both [rows][K] in MX form), bf16."""
    dev = a_codes.device        # checked for the GPU below, after the shapes
    if a_codes.dim() != 2 or b_codes.dim() != 2:
        raise ValueError("MX codes must be [rows][K/2]")
    m, kh = a_codes.shape
    n = b_codes.shape[0]
    if (2 * kh) % 32:
        raise ValueError("invalid quantization geometry: K must be a multiple of 32")
    _expect(a_codes, (m, kh), torch.uint8, "a_codes", dev)
    _expect(a_e8m0, (m, 2 * kh // 32), torch.uint8, "a_e8m0", dev)
    _expect(b_codes, (n, kh), torch.uint8, "b_codes", dev)
    _expect(b_e8m0, (n, 2 * kh // 32), torch.uint8, "b_e8m0", dev)
    if out is not None:
        _expect(out, (m, n), torch.bfloat16, "out", dev)
    _dev(a_codes)
    lib = _lib.load()
    y = torch.empty((m, n), dtype=torch.bfloat16, device=dev) if out is None else out
    _lib.check(lib.qg_mx_gemm(_ptr(a_codes), _ptr(a_e8m0), m, _ptr(b_codes), _ptr(b_e8m0), n,
                              2 * kh, _ptr(y), _stream(dev)))
    return y


def _f32_vec(t: torch.Tensor, dev: torch.device, n: int, what: str):
    if t.dtype != torch.float32 or _dev(t) != dev or t.numel() != n:
        raise ValueError(f"{what} must be an fp32 tensor of {n} values on the input's device")


def quantize_pack_smooth(x: torch.Tensor, smooth: torch.Tensor, fmt: str,
                         group: int | None = None, divide: bool = False):
    """quantize_pack of x [rows][K] with column k multiplied by smooth[k]
    (divide False: weights, W diag(s)) or divided by it (divide True:
    activations, X diag(s)^-1) first; smooth fp32 [K].  Same outputs as
    quantize_pack."""
    lib = _lib.load()
    dev = _dev(x)
    rows, k = x.shape
    _f32_vec(smooth, dev, k, "smooth")
    group = default_group(fmt, k) if group is None else group
    if group <= 0 or k % group:
        raise ValueError("invalid quantization geometry: group must divide K")
    cshape, cdt, sdt = _code_shapes(fmt, rows, k, group)
    codes = torch.empty(cshape, dtype=cdt, device=dev)
    scales = torch.empty((rows, k // group), dtype=sdt, device=dev)
    zeros = torch.empty_like(scales) if fmt in _ASYM else None
    _lib.check(lib.qg_quantize_pack_smooth(FORMATS[fmt], _ptr(x), _src_dtype(x), rows, k, group,
                                           _ptr(smooth), 1 if divide else 0, _ptr(codes),
                                           _ptr(scales), _ptr(zeros), _stream(dev)))
    return codes, scales, zeros


def channel_absmax(x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Per-column max |x| over the rows of x [rows][K] (bf16 or fp32), fp32
    [K].  With ``out`` given it holds a running maximum (earlier calibration
    batches) that is raised in place."""
    lib = _lib.load()
    dev = _dev(x)
    rows, k = x.shape
    acc = out is not None
    if acc:
        _f32_vec(out, dev, k, "out")
    else:
        out = torch.empty((k,), dtype=torch.float32, device=dev)
    _lib.check(lib.qg_channel_absmax(_ptr(x), _src_dtype(x), rows, k, 1 if acc else 0, _ptr(out),
                                     _stream(dev)))
    return out


def smooth_scales(act_absmax: torch.Tensor, w_absmax: torch.Tensor, alpha: float = 0.5):
    """SmoothQuant factors s = act_absmax^alpha / w_absmax^(1 - alpha), fp32 [K]."""
    lib = _lib.load()
    dev = _dev(act_absmax)
    k = act_absmax.numel()
    _f32_vec(act_absmax, dev, k, "act_absmax")
    _f32_vec(w_absmax, dev, k, "w_absmax")
    s = torch.empty((k,), dtype=torch.float32, device=dev)
    _lib.check(lib.qg_smooth_scales(_ptr(act_absmax), _ptr(w_absmax), ctypes.c_float(alpha), k,
                                    _ptr(s), _stream(dev)))
    return s


def channel_scales(absmax: torch.Tensor, qmax: float = 448.0) -> torch.Tensor:
    """Static per-channel scales absmax / qmax (1 where zero), same shape."""
    lib = _lib.load()
    dev = _dev(absmax)
    if absmax.dtype != torch.float32:
        raise ValueError("absmax must be fp32")
    s = torch.empty_like(absmax)
    _lib.check(lib.qg_channel_scales(_ptr(absmax), absmax.numel(), ctypes.c_float(qmax), _ptr(s),
                                     _stream(dev)))
    return s


def kv_cache_store(x: torch.Tensor, slot_mapping: torch.Tensor, cache_codes: torch.Tensor,
                   cache_scales: torch.Tensor | None = None,
                   channel_scales: torch.Tensor | None = None) -> None:
    """FP8 E4M3 quantization of x [tokens][heads][head_dim] (bf16 or fp32)
    into the paged cache in place: token t goes to slot slot_mapping[t]
    (int64; slots outside the cache are skipped).  Per token and head with
    cache_scales fp32 [slots][heads], or with static channel_scales fp32
    [heads][head_dim]; cache_codes uint8 [slots][heads][head_dim]."""
    lib = _lib.load()
    dev = _dev(x)
    t, h, d = x.shape
    if slot_mapping.dtype != torch.int64 or _dev(slot_mapping) != dev or slot_mapping.numel() != t:
        raise ValueError("slot_mapping must be an int64 tensor of one slot per token")
    if (cache_codes.dtype != torch.uint8 or _dev(cache_codes) != dev or cache_codes.dim() != 3
            or tuple(cache_codes.shape[1:]) != (h, d)):
        raise ValueError("cache_codes must be uint8 [slots][heads][head_dim] on the device")
    slots = cache_codes.shape[0]
    if cache_scales is not None:
        _f32_vec(cache_scales, dev, slots * h, "cache_scales")
    if channel_scales is not None:
        _f32_vec(channel_scales, dev, h * d, "channel_scales")
    _lib.check(lib.qg_kv_cache_store(_ptr(x), _src_dtype(x), t, h, d, _ptr(slot_mapping), slots,
                                     _ptr(channel_scales), _ptr(cache_codes), _ptr(cache_scales),
                                     _stream(dev)))


# ------------------------------------------------ roofline calibration

CALIB_KINDS = {"bf16": _lib.CALIB_BF16, "fp8": _lib.CALIB_FP8, "fp4": _lib.CALIB_FP4,
               "int8": _lib.CALIB_INT8}
CALIB_K = {"bf16": 16, "fp8": 64, "fp4": 64, "int8": 32}


def calib_stream_read(src: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Read-only stream over src (bytes a multiple of 64 KiB): returns the XOR
    of each 64 KiB chunk's 32-bit words, uint32 as int32 [bytes / 65536]."""
    dev = _dev(src)
    nbytes = src.numel() * src.element_size()
    if nbytes < 65536 or nbytes % 65536:
        raise ValueError("calib_stream_read: the tensor must hold a multiple of 64 KiB")
    if out is None:
        out = torch.empty(nbytes // 65536, dtype=torch.int32, device=dev)
    else:
        _expect(out, (nbytes // 65536,), torch.int32, "out", dev)
    lib = _lib.load()
    _lib.check(lib.qg_calib_stream_read(_ptr(src), nbytes, _ptr(out), _stream(dev)))
    return out


def calib_mfma(kind: str, waves: int, iters: int, out: torch.Tensor, ) -> torch.Tensor:
    """MFMA-only loop of `kind` ("bf16", "fp8", "fp4", "int8"); out fp32
    [waves * 64] on the GPU receives one checksum per lane.  Operations per
    launch: waves * iters * 8 * 2 * 32 * 32 * CALIB_K[kind]."""
    dev = _dev(out)
    if kind not in CALIB_KINDS:
        raise ValueError(f"unknown calibration kind {kind}")
    _expect(out, (waves * 64,), torch.float32, "out", dev)
    lib = _lib.load()
    _lib.check(lib.qg_calib_mfma(CALIB_KINDS[kind], waves, iters, _ptr(out), _stream(dev)))
    return out
