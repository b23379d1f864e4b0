#!/usr/bin/env python3
"""Benchmark of the quantized linear layer on one MI355X.

Headline: W4A16 decode, Llama-3-8B projection shapes (K->N 4096->6144 QKV,
4096->4096 O, 4096->28672 gate+up, 14336->4096 down), asymmetric INT4 in
groups of 128, M = 1.  One step = the four GEMVs of one layer; steps rotate
over distinct weight copies (more than the 256 MiB last-level cache) so every
step streams its weights from HBM.  Steps are replayed from a HIP graph
(captured through torch), so launch overhead on the host is not measured.

value = algorithmic bytes of the timed steps / time (GB/s): packed codes +
fp16 scales and zero points + bf16 activations + bf16 outputs.

Also reported (``detail``): the same layer at M = 4 and 16, the 4096x4096
GEMV, and the prefill-size GEMMs -- FP8 E4M3 W8A8 (M=N=K=8192, dynamic
per-token activation quantization timed separately), MXFP4 W4A4 (M=4096,
N=K=8192) and W4A16 prefill (M=2048, Qwen2.5-72B FFN shapes) -- in TFLOP/s
against the matching dense matrix-core peak.

``roofline`` describes the dominant kernel (the gate+up GEMV launch), timed
with HIP events around a graph of back-to-back launches on its own stream.
``cpu_baseline`` times the CPU oracle (numpy) on one layer at M = 1.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
PEAK_TFLOPS = {"bf16": 2516.6, "fp8": 5033.2, "fp4": 10066.3}
MALL_BYTES = 256 << 20


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-detail", action="store_true", help="headline only")
    p.add_argument("--counters", action="store_true",
                   help="launch only the dominant kernel (gate+up GEMV, M=1) over rotating "
                        "weight copies, then a 256 MiB device copy of known size, for "
                        "rocprofv3 kernel-trace and counter runs; prints one line")
    p.add_argument("--traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="turn two rocprofv3 counter-collection CSVs of --counters runs "
                        "(FETCH_SIZE, WRITE_SIZE) into profiles/hbm_traffic.json and exit")
    return p.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ helpers

def graph_of(fn, stream):
    """Capture fn() (a sequence of library launches) into a CUDA/HIP graph."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        fn()                                   # warm (library and allocator)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=stream):
        fn()
    torch.cuda.synchronize()
    return g


def time_graph(g, stream, reps=1):
    import torch
    st = torch.cuda.Event(enable_timing=True)
    en = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        st.record(stream)
        for _ in range(reps):
            g.replay()
        en.record(stream)
    en.synchronize()
    return st.elapsed_time(en) * 1e-3


def source_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_from_profile(kernel_src, key):
    """HBM bytes per launch measured with rocprofv3 counters (committed under
    profiles/), or None if missing or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            data = json.load(f)
        ent = data[key]
        if ent.get("source_sha256_16") != source_hash(kernel_src):
            return None
        return float(ent["bytes_per_launch"])
    except Exception:
        return None


# ------------------------------------------------------------ decode layer

def build_decode_layer(dev):
    """Quantized weights of the four projections (asymmetric INT4 g128) and
    bf16 activations (16 rows; M rows are the first M)."""
    import torch
    import quantized_gemm_group_amd as qg
    from synthetic import WORKLOADS, workload_case
    layer = []
    for i, p in enumerate(WORKLOADS["llama3_8b_decode"].projections):
        c = workload_case("llama3_8b_decode", i)
        w = torch.from_numpy(c["w"]).to(dev)
        codes, s, z = qg.quantize_pack(w, "int4_asym", 128)
        del w
        layer.append(dict(name=p.name, k=p.k, n=p.n, codes=codes, s=s, z=z,
                          x=c["x"].to(dev), w_host=c["w"], x_host=c["x"]))
    torch.cuda.synchronize()
    return layer


def layer_bytes(layer, m):
    tot = 0
    for p in layer:
        tot += p["codes"].numel() * 4 + p["s"].numel() * 2 + p["z"].numel() * 2
        tot += m * p["k"] * 2 + m * p["n"] * 2
    return tot


def proj_bytes(p, m):
    return p["codes"].numel() * 4 + p["s"].numel() * 4 + m * p["k"] * 2 + m * p["n"] * 2


def decode_copies(layer, count):
    copies = [layer]
    for _ in range(count - 1):
        copies.append([dict(p, codes=p["codes"].clone(), s=p["s"].clone(), z=p["z"].clone())
                       for p in layer])
    return copies


def run_layer(qg, lay, m, outs):
    for p, y in zip(lay, outs):
        qg.qgemv(p["x"][:m], p["codes"], p["s"], p["z"], "int4_asym", out=y)


def bench_decode(qg, torch, copies, m, steps, warmup, stream):
    outs = [torch.empty((m, p["n"]), dtype=torch.bfloat16, device=p["x"].device)
            for p in copies[0]]

    def seq(nsteps):
        def f():
            for s in range(nsteps):
                run_layer(qg, copies[s % len(copies)], m, outs)
        return f
    gw = graph_of(seq(max(warmup, 1)), stream)
    gt = graph_of(seq(steps), stream)
    time_graph(gw, stream)
    torch.cuda.synchronize()
    t = time_graph(gt, stream)
    torch.cuda.synchronize()
    return t


def bench_dominant(qg, torch, copies, stream, reps=40):
    """Back-to-back launches of the gate+up GEMV (M=1) over rotating copies."""
    idx = [i for i, p in enumerate(copies[0]) if p["name"] == "gate_up"][0]
    p0 = copies[0][idx]
    y = torch.empty((1, p0["n"]), dtype=torch.bfloat16, device=p0["x"].device)

    def f():
        for r in range(reps):
            p = copies[r % len(copies)][idx]
            qg.qgemv(p["x"][:1], p["codes"], p["s"], p["z"], "int4_asym", out=y)
    g = graph_of(f, stream)
    time_graph(g, stream)
    t = time_graph(g, stream)
    return t / reps, proj_bytes(p0, 1)


# ---------------------------------------------------- clocks and power

def _card_dir(torch, dev):
    """sysfs device directory of the amdgpu card behind dev, or None."""
    import glob
    cards = [c for c in sorted(glob.glob("/sys/class/drm/card*/device"))
             if os.path.exists(os.path.join(c, "pp_dpm_sclk"))]
    try:
        pr = torch.cuda.get_device_properties(dev)
        bdf = f"{pr.pci_domain_id:04x}:{pr.pci_bus_id:02x}:{pr.pci_device_id:02x}."
        hit = [c for c in cards if os.path.basename(os.path.realpath(c)).startswith(bdf)]
        if len(hit) == 1:
            return hit[0]
    except Exception:
        pass
    return cards[0] if len(cards) == 1 else None


class HwSampler:
    """Engine clock, memory clock and board power sampled from sysfs (the
    current pp_dpm_sclk / pp_dpm_mclk level, hwmon power1_input in
    microwatts) by a background thread while a kernel runs back to back;
    medians of the samples, None where a file cannot be read."""

    def __init__(self, card, period_s=0.004):
        import threading
        self.card, self.period = card, period_s
        self.samples = {"sclk_mhz": [], "mclk_mhz": [], "power_w": []}
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    @staticmethod
    def _level(path):
        with open(path) as f:
            for line in f:
                if line.rstrip().endswith("*"):
                    return float(line.split(":")[1].strip().lower().split("mhz")[0])
        return None

    def _power(self):
        import glob
        with open(glob.glob(os.path.join(self.card, "hwmon", "hwmon*", "power1_input"))[0]) as f:
            return int(f.read()) * 1e-6

    def _read(self):
        c = self.card
        for key, fn in (("sclk_mhz", lambda: self._level(os.path.join(c, "pp_dpm_sclk"))),
                        ("mclk_mhz", lambda: self._level(os.path.join(c, "pp_dpm_mclk"))),
                        ("power_w", self._power)):
            try:
                v = fn()
                if v is not None:
                    self.samples[key].append(v)
            except (OSError, ValueError, IndexError):
                pass

    def _run(self):
        while not self._stop.wait(self.period):
            self._read()

    def __enter__(self):
        if self.card:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread.is_alive():
            self._thread.join()

    def summary(self):
        import statistics
        out = {k: (round(statistics.median(v), 1) if v else None) for k, v in self.samples.items()}
        out["samples"] = len(self.samples["sclk_mhz"])
        return out


# --------------------------------------------------------------- GEMMs

def bench_gemms(qg, torch, dev, stream):
    from synthetic import workload_case
    out = {}
    card = _card_dir(torch, dev)
    hw = {}

    def timed(fn, reps, warm_s=0.05, sample_s=0.0):
        # untimed warm-up of at least warm_s: after the host-side set-up
        # between cases the clocks need some tens of milliseconds of load to
        # come back up, and a single warm-up call leaves the first timed
        # launches slow.  With sample_s, clocks and power are sampled after
        # the timed launches, over sample_s of the same kernel back to back,
        # into hw["last"] (the sysfs reads stay out of the timed region).
        t0 = time.perf_counter()
        while True:
            fn()
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= warm_s:
                break
        st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        st.record()
        for _ in range(reps):
            fn()
        en.record()
        en.synchronize()
        t = st.elapsed_time(en) * 1e-3 / reps
        if sample_s > 0:
            with HwSampler(card) as smp:
                t0 = time.perf_counter()
                while time.perf_counter() - t0 < sample_s:
                    fn()
                    torch.cuda.synchronize()
            hw["last"] = smp.summary()
        return t

    # FP8 W8A8, M=N=K=8192
    c = workload_case("fp8_8192")
    x = c["x"].to(dev)
    wq, sw, _ = qg.quantize_pack(torch.from_numpy(c["w"]).to(dev), "fp8_e4m3")
    xq, sx, _ = qg.quantize_pack(x, "fp8_e4m3")
    y = torch.empty((8192, 8192), dtype=torch.bfloat16, device=dev)
    t = timed(lambda: qg.qgemm(xq, wq, sw, None, "fp8_e4m3", "fp8_e4m3", a_scales=sx, out=y), 10,
              0.05, 0.05)
    hw_gemm = hw["last"]
    tq = timed(lambda: qg.quantize_pack(x, "fp8_e4m3"), 10)
    fl = 2 * 8192 ** 3
    out["fp8_gemm_8192"] = dict(us=t * 1e6, tflops=fl / t / 1e12,
                                frac=fl / t / 1e12 / PEAK_TFLOPS["fp8"],
                                act_quant_us=tq * 1e6,
                                act_quant_gbs=(8192 * 8192 * 3 + 8192 * 4) / tq / 1e9,
                                end_to_end_tflops=fl / (t + tq) / 1e12, clocks_power=hw_gemm)
    # fused RMSNorm / LayerNorm + per-token FP8 quantization of the same
    # activations (one read of x, one write of codes and scales), against
    # the unfused path: torch's layer norm writing bf16, then the quantizer
    from synthetic import norm_weights
    gamma, beta = (torch.from_numpy(a).to(dev) for a in norm_weights(8192, 4))
    nbytes = 8192 * 8192 * 3 + 8192 * 4 + 2 * 8192 * 4
    for norm in ("rms", "layer"):
        b_ = beta if norm == "layer" else None
        tn = timed(lambda: qg.norm_quant(x, gamma, b_, "fp8_e4m3", norm, 1e-5), 10)
        out[f"{norm}_norm_fp8_quant_8192"] = dict(us=tn * 1e6, gbs=nbytes / tn / 1e9,
                                                  frac=nbytes / tn / 1e9 / HBM_PEAK_GBS)
    gb = gamma.to(torch.bfloat16)
    bb = beta.to(torch.bfloat16)
    tu = timed(lambda: qg.quantize_pack(torch.nn.functional.layer_norm(x, (8192,), gb, bb, 1e-5),
                                        "fp8_e4m3"), 10)
    out["layer_norm_fp8_quant_8192"]["unfused_us"] = tu * 1e6
    del x, wq, sw, xq, sx, y, c, gamma, beta, gb, bb
    # MXFP4, M=4096, N=K=8192
    c = workload_case("mxfp4_4096x8192")
    x = c["x"].to(dev)
    bc, be = qg.mx_quant(torch.from_numpy(c["w"]).to(dev))
    ac, ae = qg.mx_quant(x)
    y = torch.empty((4096, 8192), dtype=torch.bfloat16, device=dev)
    t = timed(lambda: qg.mx_gemm(ac, ae, bc, be, out=y), 10, 0.05, 0.05)
    hw_gemm = hw["last"]
    tq = timed(lambda: qg.mx_quant(x), 10)
    fl = 2 * 4096 * 8192 * 8192
    out["mxfp4_gemm_4096x8192"] = dict(us=t * 1e6, tflops=fl / t / 1e12,
                                       frac=fl / t / 1e12 / PEAK_TFLOPS["fp4"],
                                       act_quant_us=tq * 1e6,
                                       end_to_end_tflops=fl / (t + tq) / 1e12,
                                       clocks_power=hw_gemm)
    del x, bc, be, ac, ae, y, c
    # W4A16 prefill, Qwen2.5-72B FFN shapes
    for i, name in enumerate(["ffn_up", "ffn_down"]):
        c = workload_case("qwen72b_prefill", i)
        x = c["x"].to(dev)
        codes, s, _ = qg.quantize_pack(torch.from_numpy(c["w"]).to(dev), "int4_sym", 128)
        y = torch.empty((2048, c["n"]), dtype=torch.bfloat16, device=dev)
        t = timed(lambda: qg.qgemm(x, codes, s, None, "int4_sym", "bf16", out=y), 5, 0.05, 0.05)
        fl = 2 * 2048 * c["k"] * c["n"]
        out[f"w4a16_prefill_{name}"] = dict(us=t * 1e6, tflops=fl / t / 1e12,
                                            frac=fl / t / 1e12 / PEAK_TFLOPS["bf16"],
                                            clocks_power=hw["last"])
        if name == "ffn_up":
            # the up shape is a fused gate+up (29568 = 2 x 14784 rows): the
            # SwiGLU epilogue variant writes SiLU(gate) * up, [2048][14784]
            h = torch.empty((2048, c["n"] // 2), dtype=torch.bfloat16, device=dev)
            th = timed(lambda: qg.qgemm_swiglu(x, codes, s, None, "int4_sym", out=h), 5, 0.05, 0.05)
            hw_gemm = hw["last"]
            tm = timed(lambda: torch.mul(torch.nn.functional.silu(y[:, :c["n"] // 2]),
                                         y[:, c["n"] // 2:], out=h), 5)
            out["w4a16_prefill_ffn_gate_up_swiglu"] = dict(
                us=th * 1e6, tflops=fl / th / 1e12, frac=fl / th / 1e12 / PEAK_TFLOPS["bf16"],
                unfused_us=(t + tm) * 1e6, clocks_power=hw_gemm)
            del h
        del x, codes, s, y, c
    torch.cuda.empty_cache()
    return out


def bench_gemv_4096(qg, torch, dev, stream):
    from synthetic import workload_case
    c = workload_case("gemv_4096")
    codes, s, _ = qg.quantize_pack(torch.from_numpy(c["w"]).to(dev), "int4_sym", 128)
    per = codes.numel() * 4 + s.numel() * 2
    r = max(2, -(-2 * MALL_BYTES // per))
    bufs = [(codes.clone(), s.clone()) for _ in range(r)]
    x = c["x"][:1].to(dev)
    y = torch.empty((1, 4096), dtype=torch.bfloat16, device=dev)

    def f():
        for i in range(r):
            qg.qgemv(x, bufs[i][0], bufs[i][1], None, "int4_sym", out=y)
    g = graph_of(f, stream)
    time_graph(g, stream)
    t = time_graph(g, stream) / r
    b = per + 4096 * 2 * 2
    return dict(us=t * 1e6, gbs=b / t / 1e9, frac=b / t / 1e9 / HBM_PEAK_GBS, copies=r)


# ------------------------------------------------ SmoothQuant and KV cache

def bench_smooth_kv(qg, torch, dev, stream):
    """HBM-bound steps of the SmoothQuant and FP8 KV-cache rows, each replayed
    from a HIP graph over input copies totalling more than twice the
    last-level cache (algorithmic bytes / time)."""
    from synthetic import kv_case, smoothquant_case
    out = {}

    def rate(fn_of_copy, copies, nbytes, name, **extra):
        def f():
            for i in range(copies):
                fn_of_copy(i)
        g = graph_of(f, stream)
        time_graph(g, stream)
        t = time_graph(g, stream, reps=3) / (3 * copies)
        out[name] = dict(us=t * 1e6, gbs=nbytes / t / 1e9, frac=nbytes / t / 1e9 / HBM_PEAK_GBS,
                         **extra)
        del g

    # 8192 x 8192 activations with 1 % outlier channels (bf16), weights fp32
    c = smoothquant_case(8192, 8192, 8192, seed=6)
    k = 8192
    xs = [c["x"].to(dev)]
    xs += [xs[0].clone() for _ in range(-(-2 * MALL_BYTES // xs[0].nbytes) - 1)]
    ws = [torch.from_numpy(c["w"]).to(dev)]
    ws += [ws[0].clone() for _ in range(-(-2 * MALL_BYTES // ws[0].nbytes) - 1)]
    del c
    stat_x = torch.empty(k, dtype=torch.float32, device=dev)
    stat_w = torch.empty(k, dtype=torch.float32, device=dev)
    rate(lambda i: qg.channel_absmax(xs[i], out=stat_x), len(xs), xs[0].nbytes + 4 * k,
         "smoothquant_channel_absmax_x_8192_bf16")
    rate(lambda i: qg.channel_absmax(ws[i], out=stat_w), len(ws), ws[0].nbytes + 4 * k,
         "smoothquant_channel_absmax_w_8192_f32")
    s = qg.smooth_scales(qg.channel_absmax(xs[0]), qg.channel_absmax(ws[0]), 0.5)
    xbytes = xs[0].nbytes + 8192 * k + 4 * 8192 + 4 * k
    rate(lambda i: qg.quantize_pack_smooth(xs[i], s, "int8_sym", divide=True), len(xs), xbytes,
         "smoothquant_int8_token_quant_x_8192")
    rate(lambda i: qg.quantize_pack(xs[i], "int8_sym"), len(xs), xbytes - 4 * k,
         "int8_token_quant_x_8192_unsmoothed")
    del xs
    rate(lambda i: qg.quantize_pack_smooth(ws[i], s, "int8_sym"), len(ws),
         ws[0].nbytes + 8192 * k + 4 * 8192 + 4 * k, "smoothquant_int8_channel_quant_w_8192")
    del ws, s
    torch.cuda.empty_cache()

    # FP8 KV cache: a Llama-3-8B prefill chunk (8192 tokens, 8 KV heads x 128)
    # into a 16-token paged cache of 32768 slots, values per token, keys
    # with static per-channel scales; and one decode step of 256 tokens
    t, h, d, slots = 8192, 8, 128, 32768
    c = kv_case(t, h, d, slots, seed=13)
    ks = [c["k"].to(dev)]
    ks += [ks[0].clone() for _ in range(-(-2 * MALL_BYTES // ks[0].nbytes) - 1)]
    vs = [c["v"].to(dev)] + [c["v"].to(dev) for _ in range(len(ks) - 1)]
    sl = torch.from_numpy(c["slots"]).to(dev)
    cache = torch.zeros((slots, h, d), dtype=torch.uint8, device=dev)
    cscale = torch.zeros(slots * h, dtype=torch.float32, device=dev)
    chs = qg.channel_scales(qg.channel_absmax(ks[0].reshape(t, h * d)), 448.0).reshape(h, d)
    nb = ks[0].nbytes + t * h * d + sl.nbytes
    rate(lambda i: qg.kv_cache_store(vs[i], sl, cache, cscale), len(vs), nb + 4 * t * h,
         "kv_cache_store_per_token_llama3_8b_8192tok", tokens=t)
    rate(lambda i: qg.kv_cache_store(ks[i], sl, cache, None, chs), len(ks), nb + 4 * h * d,
         "kv_cache_store_per_channel_llama3_8b_8192tok", tokens=t)
    kd, sd = ks[0][:256].contiguous(), sl[:256].contiguous()
    rate(lambda i: qg.kv_cache_store(kd, sd, cache, cscale), 64, kd.nbytes + 256 * h * d + 2048
         + 4 * 256 * h, "kv_cache_store_per_token_decode_256tok", tokens=256)
    del ks, vs, sl, cache, cscale, chs, kd, sd
    torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------ CPU baseline

def cpu_baseline(layer, min_seconds=10.0, max_passes=12):
    """The oracle as it stands on one layer at M = 1 (quantize the weights,
    then the fp64 product of the dequantized operands), repeated over whole
    layers until at least min_seconds of CPU work."""
    from oracle import gemm as og, intquant as oi
    from synthetic import bf16_as_f32
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    t0 = time.perf_counter()
    nbytes = 0
    passes = 0
    while passes < max_passes and (passes == 0 or time.perf_counter() - t0 < min_seconds):
        for p in layer:
            q, s, z = oi.quantize_asym(p["w_host"], 128)
            packed = oi.pack_int4(q)
            og.w4a16_reference(bf16_as_f32(p["x_host"][:1]), packed, s, z, 128)
            nbytes += packed.nbytes + s.nbytes + z.nbytes + p["k"] * 2 + p["n"] * 2
        passes += 1
    t = time.perf_counter() - t0
    return dict(value=nbytes / t / 1e9, unit="GB/s", cores=int(blas_threads), kind="oracle",
                sample=f"{passes} passes over one Llama-3-8B layer (QKV, O, gate+up, down) at "
                       f"M=1: oracle asymmetric INT4 g128 quantization + fp64 product of the "
                       f"dequantized operands, {t:.1f} s")


# ------------------------------------------------------- counter runs

COPY_BYTES = 256 << 20
DOMINANT_KEY = "qgemv_gate_up_m1"
DOMINANT_SRC = os.path.join(ROOT, "quantized_gemm_group_amd", "csrc", "qg_gemv.hip")


def run_counters(reps=8):
    """Launches for rocprofv3: the gate+up GEMV (4096 -> 28672, asymmetric
    INT4 g128, M=1) over weight copies spanning > 2x the last-level cache,
    then three plain copies of COPY_BYTES (read COPY_BYTES, write COPY_BYTES)
    whose counter readings calibrate FETCH_SIZE and WRITE_SIZE."""
    import torch
    import quantized_gemm_group_amd as qg
    from synthetic import WORKLOADS, workload_case
    dev = torch.device("cuda:0")
    idx = [i for i, p in enumerate(WORKLOADS["llama3_8b_decode"].projections)
           if p.name == "gate_up"][0]
    c = workload_case("llama3_8b_decode", idx)
    codes, s, z = qg.quantize_pack(torch.from_numpy(c["w"]).to(dev), "int4_asym", 128)
    per = codes.numel() * 4 + s.numel() * 4
    ncopies = max(2, -(-2 * MALL_BYTES // per))
    bufs = [(codes, s, z)] + [(codes.clone(), s.clone(), z.clone()) for _ in range(ncopies - 1)]
    x = c["x"][:1].to(dev)
    y = torch.empty((1, c["n"]), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    for _ in range(reps):
        for b in bufs:
            qg.qgemv(x, b[0], b[1], b[2], "int4_asym", out=y)
    torch.cuda.synchronize()
    src = torch.ones(COPY_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"counters": DOMINANT_KEY, "launches": reps * ncopies,
                      "bytes_per_launch": proj_bytes(dict(codes=codes, s=s, k=c["k"], n=c["n"]), 1),
                      "copy_bytes": COPY_BYTES}), flush=True)


def _counter_rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def write_traffic(fetch_csv, write_csv):
    """profiles/hbm_traffic.json from the counter CSVs of two --counters runs.
    Per dispatch, FETCH_SIZE and WRITE_SIZE (KiB) of the GEMV launches are
    averaged and scaled by COPY_BYTES over the same counter's median reading
    for the plain copies that follow the GEMV launches."""
    out = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = [r for r in _counter_rows(path) if r.get("Counter_Name") == counter]
        gemv = [r for r in rows if "qgemv" in r["Kernel_Name"]]
        if not gemv:
            raise SystemExit(f"{path}: no {counter} rows for the GEMV")
        last = max(int(r["Dispatch_Id"]) for r in gemv)
        copies = sorted(float(r["Counter_Value"]) for r in rows
                        if int(r["Dispatch_Id"]) > last and "copyBuffer" in r["Kernel_Name"])
        if not copies:
            raise SystemExit(f"{path}: no {counter} rows for the calibration copy")
        copy_kib = copies[len(copies) // 2]
        scale = COPY_BYTES / (copy_kib * 1024.0)
        vals = [float(r["Counter_Value"]) for r in gemv]
        out[counter] = dict(gemv_kib_per_dispatch=sum(vals) / len(vals), dispatches=len(vals),
                            copy_kib=copy_kib, scale=scale,
                            bytes_per_launch=sum(vals) / len(vals) * 1024.0 * scale)
    ent = dict(source_sha256_16=source_hash(DOMINANT_SRC),
               bytes_per_launch=out["FETCH_SIZE"]["bytes_per_launch"]
               + out["WRITE_SIZE"]["bytes_per_launch"], counters=out)
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    data = {}
    if os.path.exists(path):
        with open(path) as f:
            data = json.load(f)
    data[DOMINANT_KEY] = ent
    with open(path, "w") as f:
        json.dump(data, f, indent=1)
    print(json.dumps({DOMINANT_KEY: ent}))


# ------------------------------------------------------------------- main

def main():
    args = parse()
    if args.traffic:
        write_traffic(*args.traffic)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    import quantized_gemm_group_amd as qg
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    qg.load_library()
    if args.counters:
        run_counters()
        return
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(dev)

    log("building the decode layer ...")
    layer = build_decode_layer(dev)
    per_layer = layer_bytes(layer, 1)
    ncopies = max(2, -(-2 * MALL_BYTES // per_layer))      # > 2x the last-level cache
    copies = decode_copies(layer, ncopies)
    log(f"layer {per_layer / 1e6:.1f} MB x {ncopies} copies")

    t = bench_decode(qg, torch, copies, 1, args.steps, args.warmup, stream)
    value = args.steps * per_layer / t / 1e9
    ms_per_step = t / args.steps * 1e3

    dom_t, dom_b = bench_dominant(qg, torch, copies, stream)
    achieved = dom_b / dom_t / 1e9
    traffic = traffic_from_profile(DOMINANT_SRC, DOMINANT_KEY)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic, "kernel": "qgemv_wave_kernel<asym, 8 groups/wave, M<=1> (gate+up 4096->28672, M=1)",
                "us_per_launch": round(dom_t * 1e6, 3), "bytes_per_launch": dom_b}

    detail = {}
    if not args.no_detail:
        for m in (4, 16):
            tm = bench_decode(qg, torch, copies, m, max(20, args.steps // 4), 5, stream)
            b = layer_bytes(layer, m) * max(20, args.steps // 4)
            detail[f"decode_layer_m{m}"] = dict(gbs=b / tm / 1e9,
                                                frac=b / tm / 1e9 / HBM_PEAK_GBS,
                                                us_per_layer=tm / max(20, args.steps // 4) * 1e6)
        detail["decode_layer_m1"] = dict(gbs=value, frac=value / HBM_PEAK_GBS,
                                         us_per_layer=ms_per_step * 1e3)
        del copies
        torch.cuda.empty_cache()
        detail["gemv_4096"] = bench_gemv_4096(qg, torch, dev, stream)
        log("GEMMs ...")
        detail.update(bench_gemms(qg, torch, dev, stream))
        log("SmoothQuant and KV cache ...")
        detail.update(bench_smooth_kv(qg, torch, dev, stream))

    cpu = None
    if not args.no_cpu_baseline:
        log("CPU oracle baseline ...")
        cpu = cpu_baseline(layer)

    line = {
        "metric": "W4A16 GEMV HBM GB/s (% peak) + MXFP4/FP8 GEMM TFLOPS (% MFMA peak)",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) weights with 1% outlier input channels x20, N(0,1) bf16 activations)",
        "config": {"workload": "llama3_8b_decode: one layer's QKV 4096->6144, O 4096->4096, "
                               "gate+up 4096->28672, down 14336->4096 W4A16 GEMVs, M=1, "
                               "asymmetric INT4 group 128",
                   "bytes_per_step": per_layer, "weight_copies": ncopies},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "detail": detail,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
