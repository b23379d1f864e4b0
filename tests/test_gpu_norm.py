"""GPU parity of the fused normalization + per-row quantization (qg_norm_quant)
against the CPU oracle: codes, scales and zero points bit for bit, for
LayerNorm and RMSNorm, FP8 E4M3, INT8 sym/asym and MXFP4 (codes and E8M0
exponents), bf16 and fp32 sources,
ragged K (not a multiple of the workgroup's 2048-element stride), rows with
outliers, constant rows and all-zero rows; and at the FP8 GEMM's activation
shape (8192 x 8192, 0.1 % of the entries x100) and the MXFP4 GEMM's
(4096 x 8192) on sampled rows."""

import numpy as np
import pytest
import torch

import quantized_gemm_group_amd as qg
from oracle import norm as onq
from synthetic import bf16_as_f32, norm_weights, rng_for, to_bf16, workload_case
from tests.gpu_util import bits32, device, host, to_dev

pytestmark = pytest.mark.gpu

FMTS = ["fp8_e4m3", "int8_sym", "int8_asym"]
EPS = {"layer": 1e-5, "rms": 1e-6}


def activations(rows, k, seed):
    rng = rng_for(seed)
    x = (rng.standard_normal((rows, k), dtype=np.float32) * np.float32(1.5) + np.float32(0.3))
    idx = rng.choice(rows * k, size=max(1, rows * k // 500), replace=False)
    x.reshape(-1)[idx] *= np.float32(50)
    if rows >= 3:
        x[1, :] = np.float32(0.75)        # constant row: LayerNorm gives beta
        x[2, :] = 0.0                     # all-zero row
    return x


def check_against_oracle(x_dev, x_f32, gamma, beta, kind, fmt, rows_idx=None):
    dev = x_dev.device
    g = to_dev(gamma, dev)
    b = to_dev(beta, dev) if kind == "layer" else None
    codes, scales, zeros = qg.norm_quant(x_dev, g, b, fmt, kind, EPS[kind])
    c, s = host(codes), host(scales).reshape(-1)
    if fmt == "mxfp4":
        s = None
    z = None if zeros is None else host(zeros).reshape(-1)
    if rows_idx is not None:
        c = c[rows_idx]
        s = None if s is None else s[rows_idx]
        z = None if z is None else z[rows_idx]
    oc, os_, oz = onq.norm_quant(x_f32, gamma, beta if kind == "layer" else None, kind, fmt,
                                 EPS[kind])
    assert c.dtype == oc.dtype
    bad = np.argwhere(c != oc)
    assert len(bad) == 0, f"{len(bad)} code mismatches, first {bad[:4].tolist()}"
    if fmt == "mxfp4":
        e = host(scales)[rows_idx] if rows_idx is not None else host(scales)
        assert e.dtype == np.uint8 and (e == os_).all(), "E8M0 exponents differ"
        return
    assert (bits32(s) == bits32(os_)).all(), "scales differ"
    if oz is not None:
        assert (bits32(z) == bits32(oz)).all(), "zero points differ"


@pytest.mark.parametrize("kind", ["layer", "rms"])
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("rows,k,src", [(4, 512, "bf16"), (37, 4104, "bf16"), (8, 8192, "bf16"),
                                        (3, 16384, "f32"), (5, 8, "f32"), (6, 2056, "f32")])
def test_norm_quant_small(kind, fmt, rows, k, src):
    dev = device()
    print(f"norm_quant {kind} {fmt} rows={rows} K={k} {src}", flush=True)
    x = activations(rows, k, seed=rows * 7 + k)
    gamma, beta = norm_weights(k, seed=k)
    if src == "bf16":
        xt = to_bf16(x)
        x_dev, x_ref = to_dev(xt, dev), bf16_as_f32(xt)
    else:
        x_dev, x_ref = to_dev(x, dev), x
    check_against_oracle(x_dev, x_ref, gamma, beta, kind, fmt)


# K a multiple of 32 (one E8M0 exponent per 32 elements): one block, a
# ragged last vec stride (4128, 2080) and the largest row
@pytest.mark.parametrize("kind", ["layer", "rms"])
@pytest.mark.parametrize("rows,k,src", [(4, 512, "bf16"), (37, 4128, "bf16"), (8, 8192, "bf16"),
                                        (3, 16384, "f32"), (5, 32, "f32"), (6, 2080, "f32")])
def test_norm_quant_mx_small(kind, rows, k, src):
    dev = device()
    print(f"norm_quant {kind} mxfp4 rows={rows} K={k} {src}", flush=True)
    x = activations(rows, k, seed=rows * 5 + k)
    gamma, beta = norm_weights(k, seed=k + 1)
    if src == "bf16":
        xt = to_bf16(x)
        x_dev, x_ref = to_dev(xt, dev), bf16_as_f32(xt)
    else:
        x_dev, x_ref = to_dev(x, dev), x
    check_against_oracle(x_dev, x_ref, gamma, beta, kind, "mxfp4")


@pytest.mark.parametrize("kind", ["layer", "rms"])
def test_norm_quant_mx_activations_4096x8192_sampled(kind):
    # the MXFP4 GEMM's activations at full size; the oracle runs on sampled rows
    dev = device()
    c = workload_case("mxfp4_4096x8192")
    print(f"norm_quant {kind} mxfp4 4096 x 8192 bf16", flush=True)
    gamma, beta = norm_weights(8192, seed=5)
    rows = np.unique(np.concatenate([np.arange(8), np.arange(4088, 4096),
                                     rng_for(41).choice(4096, 48, replace=False)]))
    x_dev = to_dev(c["x"], dev)
    x_ref = bf16_as_f32(c["x"][torch.from_numpy(rows)])
    check_against_oracle(x_dev, x_ref, gamma, beta, kind, "mxfp4", rows_idx=rows)


@pytest.mark.parametrize("kind", ["layer", "rms"])
def test_norm_quant_fp8_activations_8192_sampled(kind):
    # the FP8 GEMM's activations at full size; the oracle runs on sampled rows
    dev = device()
    c = workload_case("fp8_8192")
    print(f"norm_quant {kind} fp8 8192 x 8192 bf16", flush=True)
    gamma, beta = norm_weights(8192, seed=4)
    rows = np.unique(np.concatenate([np.arange(8), np.arange(8184, 8192),
                                     rng_for(40).choice(8192, 48, replace=False)]))
    x_dev = to_dev(c["x"], dev)
    x_ref = bf16_as_f32(c["x"][torch.from_numpy(rows)])
    check_against_oracle(x_dev, x_ref, gamma, beta, kind, "fp8_e4m3", rows_idx=rows)


def test_fused_equals_quantize_of_normalized():
    # the fused codes are the per-row quantizer's codes of the normalized rows
    dev = device()
    x = activations(16, 4096, seed=5)
    gamma, beta = norm_weights(4096, seed=6)
    y = onq.normalize(x, gamma, beta, "layer", EPS["layer"])
    for fmt in FMTS:
        c1, s1, z1 = qg.norm_quant(to_dev(x, dev), to_dev(gamma, dev), to_dev(beta, dev), fmt,
                                   "layer", EPS["layer"])
        c2, s2, z2 = qg.quantize_pack(to_dev(y, dev), fmt)
        assert (host(c1) == host(c2)).all() and (bits32(host(s1)) == bits32(host(s2))).all()
        if z1 is not None:
            assert (bits32(host(z1)) == bits32(host(z2))).all()

    # MXFP4: the fused codes and exponents are those of qg_mx_quant on the
    # normalized rows
    c1, e1, _ = qg.norm_quant(to_dev(x, dev), to_dev(gamma, dev), to_dev(beta, dev), "mxfp4",
                              "layer", EPS["layer"])
    c2, e2 = qg.mx_quant(to_dev(y, dev))
    assert (host(c1) == host(c2)).all() and (host(e1) == host(e2)).all()
