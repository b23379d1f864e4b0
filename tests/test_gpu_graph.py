"""HIP-graph capture of the library's launches (the benchmark times graph
replays): every output of a captured sequence -- the decode GEMV at 1, 4 and
16 rows on tiled and canonical codes (per-wave, x-shared and 16-row
kernels), the SwiGLU GEMV, the W4A16 (also with its last wave of tiles in
quarters) / SwiGLU / FP8 / FP8-SwiGLU / INT8 / MXFP4 GEMMs, the per-token
quantizers, the fused norm + quantization and the FP8 KV-cache store -- is
bit-identical to the eager launch's on every one of
several replays.  Between replays the outputs are overwritten eagerly and
other eager library work runs, with synchronizations in between."""

import numpy as np
import pytest
import torch

import quantized_gemm_group_amd as qg
from synthetic import rng_for, small_case
from tests.gpu_util import device, to_dev

pytestmark = pytest.mark.gpu


def _bits(t: torch.Tensor) -> torch.Tensor:
    """Raw bits of a tensor (so NaN payloads and signed zeros compare too)."""
    t = t.contiguous()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16)
    if t.dtype == torch.float32:
        return t.view(torch.int32)
    return t


def _inputs(dev):
    c = small_case(16, 1024, 20000, seed=71, w_outlier=(0.01, 20.0))
    d = small_case(16, 2048, 4096, seed=72)
    p = small_case(300, 1024, 1000, seed=73)
    f = small_case(300, 512, 520, seed=74)
    m = small_case(256, 512, 384, seed=75)
    t = small_case(300, 512, 23040, seed=77)
    inp = {}
    inp["x"] = to_dev(c["x"], dev)
    inp["w"] = qg.quantize_pack(to_dev(c["w"], dev), "int4_asym", 128)
    inp["wt"] = qg.tile_gemv_weights(inp["w"][0])
    inp["xd"] = to_dev(d["x"], dev)
    inp["wd"] = qg.quantize_pack(to_dev(d["w"], dev), "int4_sym", 128)
    inp["wdt"] = qg.tile_gemv_weights(inp["wd"][0])
    inp["xp"] = to_dev(p["x"], dev)
    inp["wp"] = qg.quantize_pack(to_dev(p["w"], dev), "int4_sym", 128)
    inp["xf"] = to_dev(f["x"], dev)
    inp["wf"] = qg.quantize_pack(to_dev(f["w"], dev), "fp8_e4m3")
    inp["wi"] = qg.quantize_pack(to_dev(f["w"], dev), "int8_sym")
    inp["xt"] = to_dev(t["x"], dev)
    inp["wt4"] = qg.quantize_pack(to_dev(t["w"], dev), "int4_sym", 128)
    inp["xm"] = to_dev(m["x"], dev)
    inp["wm"] = qg.mx_quant(to_dev(m["w"], dev))
    k = inp["xp"].shape[1]
    g = rng_for(76)
    inp["gamma"] = torch.from_numpy((1.0 + 0.1 * g.standard_normal(k)).astype(np.float32)).to(dev)
    inp["beta"] = torch.from_numpy((0.1 * g.standard_normal(k)).astype(np.float32)).to(dev)
    kv = g.standard_normal((32, 8, 128)).astype(np.float32)
    inp["kv"] = to_dev(kv, dev).to(torch.bfloat16)
    inp["slots"] = torch.from_numpy(g.permutation(64)[:32].astype(np.int64)).to(dev)
    inp["cache"] = torch.zeros((64, 8, 128), dtype=torch.uint8, device=dev)
    inp["cache_s"] = torch.zeros((64, 8), dtype=torch.float32, device=dev)
    return inp


def _launches(inp):
    """One pass over every kernel family; returns the outputs by name."""
    out = {}
    x, (codes, s, z), wt = inp["x"], inp["w"], inp["wt"]
    for m in (1, 4, 16):
        out[f"gemv_tiled_m{m}"] = qg.qgemv_tiled(x[:m], wt, s, z, "int4_asym")
        out[f"gemv_m{m}"] = qg.qgemv(x[:m], codes, s, z, "int4_asym")
        out[f"swiglu_m{m}"] = qg.qgemv_swiglu(x[:m], wt, s, z, "int4_asym")
    dc, ds, _ = inp["wd"]
    out["gemv_down_m16"] = qg.qgemv_tiled(inp["xd"], inp["wdt"], ds, None, "int4_sym")
    out["gemv_down_m1"] = qg.qgemv(inp["xd"][:1], dc, ds, None, "int4_sym")
    pc, ps, _ = inp["wp"]
    out["w4a16"] = qg.qgemm(inp["xp"], pc, ps, None, "int4_sym", "bf16")
    out["w4a16_swiglu"] = qg.qgemm_swiglu(inp["xp"], pc, ps, None, "int4_sym")
    tc, ts, _ = inp["wt4"]     # 270 tiles: whole tiles, then a launch of quarter tiles
    out["w4a16_last_wave"] = qg.qgemm(inp["xt"], tc, ts, None, "int4_sym", "bf16")
    xq, sx, _ = qg.quantize_pack(inp["xf"], "fp8_e4m3")
    out["fp8_codes"], out["fp8_scales"] = xq, sx
    wq, sw, _ = inp["wf"]
    out["fp8"] = qg.qgemm(xq, wq, sw, None, "fp8_e4m3", "fp8_e4m3", a_scales=sx)
    out["fp8_swiglu"] = qg.qgemm_swiglu_fp8(xq, sx, wq, sw)
    iq, isc, iz = qg.quantize_pack(inp["xf"], "int8_asym")
    wiq, wis, _ = inp["wi"]
    out["int8"] = qg.qgemm(iq, wiq, wis, None, "int8_sym", "int8_asym", a_scales=isc, a_zeros=iz)
    ac, ae = qg.mx_quant(inp["xm"])
    out["mx_codes"], out["mx_e8m0"] = ac, ae
    bc, be = inp["wm"]
    out["mx"] = qg.mx_gemm(ac, ae, bc, be)
    nc, nsc, _ = qg.norm_quant(inp["xp"], inp["gamma"], None, "fp8_e4m3", norm="rms")
    out["rms_fp8_codes"], out["rms_fp8_scales"] = nc, nsc
    lc, le, _ = qg.norm_quant(inp["xp"], inp["gamma"], inp["beta"], "mxfp4", norm="layer")
    out["layer_mx_codes"], out["layer_mx_e8m0"] = lc, le
    qg.kv_cache_store(inp["kv"], inp["slots"], inp["cache"], cache_scales=inp["cache_s"])
    out["kv_codes"], out["kv_scales"] = inp["cache"], inp["cache_s"]
    return out


def test_graph_replays_match_eager_launches():
    dev = device()
    print("graph capture of every kernel family, 3 replays", flush=True)
    inp = _inputs(dev)
    eager = {k: v.clone() for k, v in _launches(inp).items()}
    torch.cuda.synchronize()
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _launches(inp)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        captured = _launches(inp)
    torch.cuda.synchronize()
    other = qg.quantize_pack(inp["xd"].float() * 0.5, "int4_sym", 128)
    for rep in range(3):
        # overwrite every output eagerly (a fill kernel, outside the graph),
        # and run unrelated library work, so each replay must rewrite them
        for name, t in captured.items():
            if name.startswith("kv_"):
                t.zero_()          # the store writes only the mapped slots
            else:
                t.fill_(7 if not t.is_floating_point() else -3.0)
        qg.qgemv(inp["xd"][:4], other[0], other[1], None, "int4_sym")
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, ref in eager.items():
            got = captured[name]
            assert got.shape == ref.shape, name
            assert torch.equal(_bits(got), _bits(ref)), f"replay {rep}: {name} differs from eager"
