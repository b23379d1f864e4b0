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
    p.add_argument("--trace-summary", metavar="KERNEL_TRACE_CSV",
                   help="print a markdown summary of a rocprofv3 kernel trace of a bench.py "
                        "run (per kernel and grid; the roofline kernel's timed replays) and exit")
    p.add_argument("--gemm-counters", action="store_true",
                   help="launch only the prefill GEMMs (FP8, MXFP4, W4A16 up/down) a few times, "
                        "for rocprofv3 counter passes; prints one line")
    p.add_argument("--counter-summary", nargs="+", metavar="COUNTER_CSV",
                   help="print a markdown summary of rocprofv3 counter CSVs of --gemm-counters "
                        "runs and exit")
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
                          tiled=qg.tile_gemv_weights(codes),
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
        copies.append([dict(p, codes=p["codes"].clone(), s=p["s"].clone(), z=p["z"].clone(),
                            tiled=type(p["tiled"])(p["tiled"].data.clone(), p["n"], p["k"]))
                       for p in layer])
    return copies


def gemv(qg, p, m, y, tiled=True):
    """One projection's W4A16 GEMV: on the tiled codes (the deployment path:
    codes re-laid-out once after loading) or on the canonical packing."""
    if tiled:
        qg.qgemv_tiled(p["x"][:m], p["tiled"], p["s"], p["z"], "int4_asym", out=y)
    else:
        qg.qgemv(p["x"][:m], p["codes"], p["s"], p["z"], "int4_asym", out=y)


def run_layer(qg, lay, m, outs, tiled=True):
    for p, y in zip(lay, outs):
        gemv(qg, p, m, y, tiled)


def bench_decode(qg, torch, copies, m, steps, warmup, stream, tiled=True):
    outs = [torch.empty((m, p["n"]), dtype=torch.bfloat16, device=p["x"].device)
            for p in copies[0]]

    def seq(nsteps):
        def f():
            for s in range(nsteps):
                run_layer(qg, copies[s % len(copies)], m, outs, tiled)
        return f
    gw = graph_of(seq(max(warmup, 1)), stream)
    gt = graph_of(seq(steps), stream)
    time_graph(gw, stream)
    torch.cuda.synchronize()
    t = time_graph(gt, stream)
    torch.cuda.synchronize()
    return t


ROOFLINE_REPS, ROOFLINE_TRIALS = 40, 25


def bench_dominant(qg, torch, copies, stream):
    """The gate+up GEMV (M=1) launched ROOFLINE_REPS times back to back over
    rotating weight copies from one HIP graph; the graph is replayed
    ROOFLINE_TRIALS times, each replay between its own pair of events on the
    graph's stream, and the median replay / ROOFLINE_REPS is the time per
    launch.  One eager launch warms the library; the graph is captured
    without running it, so a kernel trace of this function holds one eager
    launch and then only replayed ones (1 + ROOFLINE_TRIALS + 1 replays)."""
    idx = [i for i, p in enumerate(copies[0]) if p["name"] == "gate_up"][0]
    p0 = copies[0][idx]
    y = torch.empty((1, p0["n"]), dtype=torch.bfloat16, device=p0["x"].device)

    def launch(r):
        gemv(qg, copies[r % len(copies)][idx], 1, y)

    with torch.cuda.stream(stream):
        launch(0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for r in range(ROOFLINE_REPS):
            launch(r)
    torch.cuda.synchronize()
    time_graph(g, stream)                      # warm replay
    ts = sorted(time_graph(g, stream) for _ in range(ROOFLINE_TRIALS))
    return ts[len(ts) // 2] / ROOFLINE_REPS, proj_bytes(p0, 1), ts[0] / ROOFLINE_REPS, \
        ts[-1] / ROOFLINE_REPS


def bench_projections(qg, torch, copies, stream, reps=40, tiled=True):
    """Each projection's GEMV (M=1) alone: a graph of `reps` launches over
    the rotating weight copies, median of 9 replays."""
    out = {}
    for idx, p0 in enumerate(copies[0]):
        y = torch.empty((1, p0["n"]), dtype=torch.bfloat16, device=p0["x"].device)

        def f():
            for r in range(reps):
                gemv(qg, copies[r % len(copies)][idx], 1, y, tiled)
        g = graph_of(f, stream)
        time_graph(g, stream)
        ts = sorted(time_graph(g, stream) / reps for _ in range(9))
        t = ts[4]
        b = proj_bytes(p0, 1)
        out[p0["name"]] = dict(us=round(t * 1e6, 3), gbs=round(b / t / 1e9, 1),
                               frac=round(b / t / 1e9 / HBM_PEAK_GBS, 4))
        del g
    return out


def bench_swiglu_decode(qg, torch, copies, stream, reps=40):
    """The fused SwiGLU GEMV on the gate+up projection (tiled codes) at
    M = 1, 4, 16, against the unfused path (the GEMV writing [M][2I], then
    torch's SiLU(g) * u): graphs of `reps` launches over the rotating copies,
    median of 9 replays."""
    idx = [i for i, p in enumerate(copies[0]) if p["name"] == "gate_up"][0]
    p0 = copies[0][idx]
    n2, k = p0["n"], p0["k"]
    i = n2 // 2
    dev = p0["x"].device
    out = {}
    for m in (1, 4, 16):
        h = torch.empty((m, i), dtype=torch.bfloat16, device=dev)
        y = torch.empty((m, n2), dtype=torch.bfloat16, device=dev)

        def fused():
            for r in range(reps):
                p = copies[r % len(copies)][idx]
                qg.qgemv_swiglu(p["x"][:m], p["tiled"], p["s"], p["z"], "int4_asym", out=h)

        def unfused():
            for r in range(reps):
                p = copies[r % len(copies)][idx]
                qg.qgemv_tiled(p["x"][:m], p["tiled"], p["s"], p["z"], "int4_asym", out=y)
                torch.mul(torch.nn.functional.silu(y[:, :i]), y[:, i:], out=h)
        res = {}
        for name, fn in (("fused", fused), ("unfused", unfused)):
            g = graph_of(fn, stream)
            time_graph(g, stream)
            ts = sorted(time_graph(g, stream) / reps for _ in range(9))
            res[name] = ts[4]
            del g
        b = p0["codes"].numel() * 4 + p0["s"].numel() * 4 + m * k * 2 + m * i * 2
        out[f"m{m}"] = dict(us=round(res["fused"] * 1e6, 3), gbs=round(b / res["fused"] / 1e9, 1),
                            frac=round(b / res["fused"] / 1e9 / HBM_PEAK_GBS, 4),
                            unfused_us=round(res["unfused"] * 1e6, 3))
    return out


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

def bench_gemms(qg, torch, dev, stream, cpu=None):
    """GEMM throughput (median of 25 single-launch trials each); with `cpu` a
    dict, the CPU oracle is also timed on a bounded sample of each workload's
    host inputs into it."""
    from synthetic import workload_case
    out = {}
    card = _card_dir(torch, dev)
    hw = {}

    def timed(fn, trials=25, warm_s=0.05, sample_s=0.0):
        # untimed warm-up of at least warm_s: after the host-side set-up
        # between cases the clocks need some tens of milliseconds of load to
        # come back up, and a single warm-up call leaves the first timed
        # launches slow.  Then `trials` launches back to back, each between
        # its own pair of events; the median is the figure (min / max kept).
        # With sample_s, clocks and power are sampled after the timed
        # launches, over sample_s of the same kernel back to back, into
        # hw["last"] (the sysfs reads stay out of the timed region).
        t0 = time.perf_counter()
        while True:
            fn()
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= warm_s:
                break
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(trials)]
        for st, en in evs:
            st.record()
            fn()
            en.record()
        evs[-1][1].synchronize()
        ts = sorted(st.elapsed_time(en) * 1e-3 for st, en in evs)
        hw["trials"] = dict(trials=trials, min_us=round(ts[0] * 1e6, 2),
                            max_us=round(ts[-1] * 1e6, 2))
        t = ts[len(ts) // 2] if trials % 2 else 0.5 * (ts[trials // 2 - 1] + ts[trials // 2])
        if sample_s > 0:
            with HwSampler(card) as smp:
                t0 = time.perf_counter()
                while time.perf_counter() - t0 < sample_s:
                    fn()
                    torch.cuda.synchronize()
            hw["last"] = smp.summary()
        return t

    def rec(t, fl, peak, **extra):
        return dict(us=t * 1e6, tflops=fl / t / 1e12, frac=fl / t / 1e12 / PEAK_TFLOPS[peak],
                    trials=hw["trials"], **extra)

    # FP8 W8A8, M=N=K=8192
    c = workload_case("fp8_8192")
    x = c["x"].to(dev)
    wq, sw, _ = qg.quantize_pack(torch.from_numpy(c["w"]).to(dev), "fp8_e4m3")
    xq, sx, _ = qg.quantize_pack(x, "fp8_e4m3")
    y = torch.empty((8192, 8192), dtype=torch.bfloat16, device=dev)
    fl = 2 * 8192 ** 3
    t = timed(lambda: qg.qgemm(xq, wq, sw, None, "fp8_e4m3", "fp8_e4m3", a_scales=sx, out=y),
              sample_s=0.05)
    out["fp8_gemm_8192"] = rec(t, fl, "fp8", clocks_power=hw["last"])
    tq = timed(lambda: qg.quantize_pack(x, "fp8_e4m3"))
    out["fp8_gemm_8192"].update(act_quant_us=tq * 1e6,
                                act_quant_gbs=(8192 * 8192 * 3 + 8192 * 4) / tq / 1e9,
                                end_to_end_tflops=fl / (t + tq) / 1e12)
    # the same operands read as [W_gate; W_up] of 4096 channels each: the
    # SwiGLU epilogue writes SiLU(g) * u, [8192][4096], against the GEMM
    # followed by torch's SiLU and product
    h8 = torch.empty((8192, 4096), dtype=torch.bfloat16, device=dev)
    th = timed(lambda: qg.qgemm_swiglu_fp8(xq, sx, wq, sw, out=h8), sample_s=0.05)
    rh = rec(th, fl, "fp8", clocks_power=hw["last"])
    tm = timed(lambda: torch.mul(torch.nn.functional.silu(y[:, :4096]), y[:, 4096:], out=h8))
    rh["unfused_us"] = (t + tm) * 1e6
    out["fp8_gemm_8192_swiglu"] = rh
    del h8
    if cpu is not None:
        cpu["fp8_8192"] = cpu_fp8_sample(c, rows=1024)
    # fused RMSNorm / LayerNorm + per-token FP8 quantization of the same
    # activations (one read of x, one write of codes and scales), against
    # the unfused path: torch's layer norm writing bf16, then the quantizer
    from synthetic import norm_weights
    gamma, beta = (torch.from_numpy(a).to(dev) for a in norm_weights(8192, 4))
    nbytes = 8192 * 8192 * 3 + 8192 * 4 + 2 * 8192 * 4
    for norm in ("rms", "layer"):
        b_ = beta if norm == "layer" else None
        tn = timed(lambda: qg.norm_quant(x, gamma, b_, "fp8_e4m3", norm, 1e-5))
        out[f"{norm}_norm_fp8_quant_8192"] = dict(us=tn * 1e6, gbs=nbytes / tn / 1e9,
                                                  frac=nbytes / tn / 1e9 / HBM_PEAK_GBS)
    gb = gamma.to(torch.bfloat16)
    bb = beta.to(torch.bfloat16)
    tu = timed(lambda: qg.quantize_pack(torch.nn.functional.layer_norm(x, (8192,), gb, bb, 1e-5),
                                        "fp8_e4m3"))
    out["layer_norm_fp8_quant_8192"]["unfused_us"] = tu * 1e6
    del x, wq, sw, xq, sx, y, c, gamma, beta, gb, bb
    # MXFP4, M=4096, N=K=8192
    c = workload_case("mxfp4_4096x8192")
    x = c["x"].to(dev)
    bc, be = qg.mx_quant(torch.from_numpy(c["w"]).to(dev))
    ac, ae = qg.mx_quant(x)
    y = torch.empty((4096, 8192), dtype=torch.bfloat16, device=dev)
    fl = 2 * 4096 * 8192 * 8192
    t = timed(lambda: qg.mx_gemm(ac, ae, bc, be, out=y), sample_s=0.05)
    out["mxfp4_gemm_4096x8192"] = rec(t, fl, "fp4", clocks_power=hw["last"])
    tq = timed(lambda: qg.mx_quant(x))
    out["mxfp4_gemm_4096x8192"].update(act_quant_us=tq * 1e6,
                                       end_to_end_tflops=fl / (t + tq) / 1e12)
    if cpu is not None:
        cpu["mxfp4_4096x8192"] = cpu_mx_sample(c, rows=1024)
    # fused RMSNorm / LayerNorm + MXFP4 quantization of the same activations
    # (codes and E8M0 exponents written once), against torch's layer norm
    # writing bf16 followed by the MX quantizer
    gamma, beta = (torch.from_numpy(a).to(dev) for a in norm_weights(8192, 5))
    nbytes = 4096 * 8192 * 2 + 4096 * 4096 + 4096 * 256 + 2 * 8192 * 4
    for norm in ("rms", "layer"):
        b_ = beta if norm == "layer" else None
        tn = timed(lambda: qg.norm_quant(x, gamma, b_, "mxfp4", norm, 1e-5))
        out[f"{norm}_norm_mxfp4_quant_4096x8192"] = dict(us=tn * 1e6, gbs=nbytes / tn / 1e9,
                                                         frac=nbytes / tn / 1e9 / HBM_PEAK_GBS)
    gb, bb = gamma.to(torch.bfloat16), beta.to(torch.bfloat16)
    tu = timed(lambda: qg.mx_quant(torch.nn.functional.layer_norm(x, (8192,), gb, bb, 1e-5)))
    out["layer_norm_mxfp4_quant_4096x8192"]["unfused_us"] = tu * 1e6
    del x, bc, be, ac, ae, y, c, gamma, beta, gb, bb
    # W4A16 prefill, Qwen2.5-72B FFN shapes
    for i, name in enumerate(["ffn_up", "ffn_down"]):
        c = workload_case("qwen72b_prefill", i)
        x = c["x"].to(dev)
        codes, s, _ = qg.quantize_pack(torch.from_numpy(c["w"]).to(dev), "int4_sym", 128)
        y = torch.empty((2048, c["n"]), dtype=torch.bfloat16, device=dev)
        fl = 2 * 2048 * c["k"] * c["n"]
        t = timed(lambda: qg.qgemm(x, codes, s, None, "int4_sym", "bf16", out=y), sample_s=0.05)
        out[f"w4a16_prefill_{name}"] = rec(t, fl, "bf16", clocks_power=hw["last"])
        if cpu is not None and name == "ffn_up":
            cpu["qwen72b_prefill_ffn_up"] = cpu_w4a16_sample(c, channels=2048)
        if name == "ffn_up":
            # the up shape is a fused gate+up (29568 = 2 x 14784 rows): the
            # SwiGLU epilogue variant writes SiLU(gate) * up, [2048][14784]
            h = torch.empty((2048, c["n"] // 2), dtype=torch.bfloat16, device=dev)
            th = timed(lambda: qg.qgemm_swiglu(x, codes, s, None, "int4_sym", out=h),
                       sample_s=0.05)
            rh = rec(th, fl, "bf16", clocks_power=hw["last"])
            tm = timed(lambda: torch.mul(torch.nn.functional.silu(y[:, :c["n"] // 2]),
                                         y[:, c["n"] // 2:], out=h))
            rh["unfused_us"] = (t + tm) * 1e6
            out["w4a16_prefill_ffn_gate_up_swiglu"] = rh
            del h
        del x, codes, s, y, c
    torch.cuda.empty_cache()
    return out


def bench_gemv_4096(qg, torch, dev, stream, cpu=None):
    from synthetic import workload_case
    c = workload_case("gemv_4096")
    codes, s, _ = qg.quantize_pack(torch.from_numpy(c["w"]).to(dev), "int4_sym", 128)
    per = codes.numel() * 4 + s.numel() * 2
    r = max(2, -(-2 * MALL_BYTES // per))
    bufs = [(codes.clone(), s.clone()) for _ in range(r)]
    tiled = [qg.tile_gemv_weights(b[0]) for b in bufs]
    x = c["x"][:1].to(dev)
    y = torch.empty((1, 4096), dtype=torch.bfloat16, device=dev)
    b = per + 4096 * 2 * 2
    out = {}
    for layout in ("tiled", "canonical"):
        def f():
            for i in range(r):
                if layout == "tiled":
                    qg.qgemv_tiled(x, tiled[i], bufs[i][1], None, "int4_sym", out=y)
                else:
                    qg.qgemv(x, bufs[i][0], bufs[i][1], None, "int4_sym", out=y)
        g = graph_of(f, stream)
        time_graph(g, stream)
        ts = sorted(time_graph(g, stream) / r for _ in range(9))
        t = ts[len(ts) // 2]
        out[layout] = dict(us=t * 1e6, gbs=b / t / 1e9, frac=b / t / 1e9 / HBM_PEAK_GBS)
        del g
    if cpu is not None:
        cpu["gemv_4096"] = cpu_gemv4096_sample(c)
    return dict(out["tiled"], canonical=out["canonical"], copies=r,
                timing="median of 9 graph replays")


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

def host_cores():
    return len(os.sched_getaffinity(0))


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:
        return 1


def _cpu_repeat(fn, min_seconds, max_passes):
    """Run fn() (the oracle on one sample) until min_seconds have passed."""
    t0 = time.perf_counter()
    passes = 0
    while passes < max_passes and (passes == 0 or time.perf_counter() - t0 < min_seconds):
        fn()
        passes += 1
    return passes, time.perf_counter() - t0


def cpu_baseline(layer, min_seconds=6.0, max_passes=12):
    """The oracle as it stands on one decode layer at M = 1 (quantize the
    weights, then the fp64 product of the dequantized operands), repeated
    over whole layers until at least min_seconds of CPU work."""
    from oracle import gemm as og, intquant as oi
    from synthetic import bf16_as_f32
    nbytes = 0

    def one():
        nonlocal nbytes
        for p in layer:
            q, s, z = oi.quantize_asym(p["w_host"], 128)
            packed = oi.pack_int4(q)
            og.w4a16_reference(bf16_as_f32(p["x_host"][:1]), packed, s, z, 128)
            nbytes += packed.nbytes + s.nbytes + z.nbytes + p["k"] * 2 + p["n"] * 2
    passes, t = _cpu_repeat(one, min_seconds, max_passes)
    return dict(value=nbytes / t / 1e9, unit="GB/s", seconds=round(t, 2),
                sample=f"{passes} passes over one Llama-3-8B layer (QKV, O, gate+up, down) at "
                       f"M=1: oracle asymmetric INT4 g128 quantization + fp64 product of the "
                       f"dequantized operands")


def cpu_gemv4096_sample(c, min_seconds=2.0):
    """Config 1 whole: INT4 sym g128 quantization of the 4096 x 4096 weight and
    the fp64 product with one row of x; GB/s of the GPU's algorithmic bytes."""
    from oracle import gemm as og, intquant as oi
    from synthetic import bf16_as_f32
    per = 4096 * 4096 // 2 + 4096 * 32 * 2 + 4096 * 2 * 2

    def one():
        q, s = oi.quantize_sym(c["w"], 128)
        og.w4a16_reference(bf16_as_f32(c["x"][:1]), oi.pack_int4(q), s, None, 128)
    passes, t = _cpu_repeat(one, min_seconds, 8)
    return dict(value=passes * per / t / 1e9, unit="GB/s", seconds=round(t, 2),
                sample=f"{passes} x the whole 4096x4096 GEMV (quantization + product)")


def cpu_w4a16_sample(c, channels):
    """W4A16 prefill (up shape): the first `channels` weight rows quantized
    (INT4 sym g128) and their fp64 product with all 2048 token rows."""
    from oracle import gemm as og, intquant as oi
    from synthetic import bf16_as_f32
    fl = 2 * 2048 * channels * c["k"]
    x = bf16_as_f32(c["x"])

    def one():
        q, s = oi.quantize_sym(c["w"][:channels], 128)
        og.w4a16_reference(x, oi.pack_int4(q), s, None, 128)
    passes, t = _cpu_repeat(one, 0.0, 1)
    return dict(value=passes * fl / t / 1e12, unit="TFLOP/s", seconds=round(t, 2),
                sample=f"2048 tokens x {channels} of {c['n']} channels x K={c['k']}")


def cpu_fp8_sample(c, rows):
    """FP8 W8A8: the first `rows` token rows and weight rows quantized
    (per token / per channel E4M3) and their fp64 product over K = 8192."""
    from oracle import fp8 as of8, gemm as og
    from synthetic import bf16_as_f32
    fl = 2 * rows * rows * 8192

    def one():
        xq, sx = of8.quantize_rows(bf16_as_f32(c["x"][:rows]))
        wq, sw = of8.quantize_rows(c["w"][:rows])
        og.fp8_reference(xq, sx, wq, sw)
    passes, t = _cpu_repeat(one, 0.0, 1)
    return dict(value=passes * fl / t / 1e12, unit="TFLOP/s", seconds=round(t, 2),
                sample=f"{rows} tokens x {rows} channels x K=8192 of 8192^3")


def cpu_mx_sample(c, rows):
    """MXFP4: the first `rows` rows of both operands MX-quantized and their
    fp64 product over K = 8192."""
    from oracle import gemm as og, mx as omx
    from synthetic import bf16_as_f32
    fl = 2 * rows * rows * 8192

    def one():
        ac, ae = omx.quantize(bf16_as_f32(c["x"][:rows]))
        bc, be = omx.quantize(c["w"][:rows])
        og.mx_reference(ac, ae, bc, be)
    passes, t = _cpu_repeat(one, 0.0, 1)
    return dict(value=passes * fl / t / 1e12, unit="TFLOP/s", seconds=round(t, 2),
                sample=f"{rows} x {rows} x K=8192 of 4096x8192x8192")


# ------------------------------------------------------ roofline calibration

def calibration(qg, torch, dev, stream):
    """The two roofs measured on this GPU (the library's calibration probes):
    read-only HBM streams (one launch over >= 1 GiB, and 62.5 MB launches
    rotating over distinct buffers > 2x the last-level cache, the gate+up
    GEMV's size) and MFMA-only loops per data type.  Median of trials."""
    out = {}

    def med(ts):
        ts = sorted(ts)
        return ts[len(ts) // 2]

    big = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(7)
    sink = torch.empty((1 << 30) // 65536, dtype=torch.int32, device=dev)
    qg.calib_stream_read(big, out=sink)
    torch.cuda.synchronize()
    ts = []
    for _ in range(21):
        st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        st.record()
        qg.calib_stream_read(big, out=sink)
        en.record()
        en.synchronize()
        ts.append(st.elapsed_time(en) * 1e-3)
    out["hbm_read_1gib_gbs"] = round(big.numel() / med(ts) / 1e9, 1)
    # 62.5 MB pieces of the same allocation (16 of them span 1 GiB)
    piece = 62455808 // 65536 * 65536
    views = [big[i * piece:(i + 1) * piece] for i in range((1 << 30) // piece)]
    psink = torch.empty(piece // 65536, dtype=torch.int32, device=dev)

    def f():
        for v in views:
            qg.calib_stream_read(v, out=psink)
    g = graph_of(f, stream)
    time_graph(g, stream)
    t = med([time_graph(g, stream) for _ in range(9)]) / len(views)
    out["hbm_read_62mb_gbs"] = round(piece / t / 1e9, 1)
    out["hbm_read_62mb_us"] = round(t * 1e6, 3)
    del big, sink, views, psink, g
    torch.cuda.empty_cache()
    # MFMA-only loops: 2 waves per SIMD on 256 CUs
    waves, iters = 2048, 2048
    sinkf = torch.empty(waves * 64, dtype=torch.float32, device=dev)
    for kind in ("bf16", "fp8", "fp4", "int8"):
        ops = waves * iters * 8 * 2 * 32 * 32 * qg.CALIB_K[kind]
        qg.calib_mfma(kind, waves, iters, sinkf)
        torch.cuda.synchronize()
        ts = []
        for _ in range(11):
            st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            st.record()
            qg.calib_mfma(kind, waves, iters, sinkf)
            en.record()
            en.synchronize()
            ts.append(st.elapsed_time(en) * 1e-3)
        out[f"mfma_{kind}_tflops"] = round(ops / med(ts) / 1e12, 1)
    return out


# ----------------------------------------------------------------- context

# The pages' own figures for this path (context only: other hardware, mostly
# without a number), restated.
CONTEXT = [
    {"figure": "Marlin W4A16 kernels come close to the bandwidth utilization of an FP16 GEMM",
     "hardware": "A100", "source": "推理优化与量化算子深度技术调研, section 1.3"},
    {"figure": "INT4 weights give about a 2x decode speed-up (batch 1, memory bound)",
     "hardware": "not stated", "source": "推理优化与量化算子深度技术调研, section 1.3"},
    {"figure": "well-built W4A16 small-batch decode kernels fill 85 % or more of HBM bandwidth",
     "hardware": "not stated", "source": "第 6 课：量化源码走读, answer to question 2"},
    {"figure": "FP8 tensor cores run at twice the FP16 rate",
     "hardware": "H100", "source": "推理优化与量化算子深度技术调研, section 1.4"},
]


# ------------------------------------------------------- counter runs

COPY_BYTES = 256 << 20
DOMINANT_KEY = "qgemv_gate_up_m1"
DOMINANT_SRC = os.path.join(ROOT, "quantized_gemm_group_amd", "csrc", "qg_gemv.hip")


def run_counters(reps=8):
    """Launches for rocprofv3: the gate+up GEMV (4096 -> 28672, asymmetric
    INT4 g128, M=1, tiled codes) over weight copies spanning > 2x the
    last-level cache,
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
    tiled = [qg.tile_gemv_weights(b[0]) for b in bufs]
    torch.cuda.synchronize()
    for _ in range(reps):
        for b, t in zip(bufs, tiled):
            qg.qgemv_tiled(x, t, b[1], b[2], "int4_asym", out=y)
    torch.cuda.synchronize()
    src = torch.ones(COPY_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"counters": DOMINANT_KEY, "launches": reps * ncopies,
                      "bytes_per_launch": proj_bytes(dict(codes=codes, s=s, k=c["k"], n=c["n"]), 1),
                      "copy_bytes": COPY_BYTES}), flush=True)


def run_gemm_counters(reps=3):
    """Launches for rocprofv3 counter passes over the prefill GEMMs: FP8 W8A8
    8192^3, MXFP4 4096x8192x8192 and the W4A16 Qwen2.5-72B FFN up and down
    GEMMs, each `reps` times after one warm launch; prints one line."""
    import torch
    import quantized_gemm_group_amd as qg
    from synthetic import workload_case
    dev = torch.device("cuda:0")
    c = workload_case("fp8_8192")
    xq, sx, _ = qg.quantize_pack(c["x"].to(dev), "fp8_e4m3")
    wq, sw, _ = qg.quantize_pack(torch.from_numpy(c["w"]).to(dev), "fp8_e4m3")
    y = torch.empty((8192, 8192), dtype=torch.bfloat16, device=dev)
    for _ in range(reps + 1):
        qg.qgemm(xq, wq, sw, None, "fp8_e4m3", "fp8_e4m3", a_scales=sx, out=y)
    torch.cuda.synchronize()
    del c, xq, sx, wq, sw, y
    c = workload_case("mxfp4_4096x8192")
    ac, ae = qg.mx_quant(c["x"].to(dev))
    bc, be = qg.mx_quant(torch.from_numpy(c["w"]).to(dev))
    y = torch.empty((4096, 8192), dtype=torch.bfloat16, device=dev)
    for _ in range(reps + 1):
        qg.mx_gemm(ac, ae, bc, be, out=y)
    torch.cuda.synchronize()
    del c, ac, ae, bc, be, y
    for i in range(2):
        c = workload_case("qwen72b_prefill", i)
        x = c["x"].to(dev)
        codes, s, _ = qg.quantize_pack(torch.from_numpy(c["w"]).to(dev), "int4_sym", 128)
        y = torch.empty((2048, c["n"]), dtype=torch.bfloat16, device=dev)
        for _ in range(reps + 1):
            qg.qgemm(x, codes, s, None, "int4_sym", "bf16", out=y)
        torch.cuda.synchronize()
        del c, x, codes, s, y
    print(json.dumps({"gemm_counters": ["fp8_8192", "mxfp4_4096x8192", "w4a16_qwen72b_up",
                                        "w4a16_qwen72b_down"], "launches_each": reps + 1}),
          flush=True)


GEMM_COUNTER_KERNELS = [("gemm_f8f4_kernel<false", "FP8 W8A8 8192^3", 2 * 8192 ** 3),
                        ("gemm_f8f4_kernel<true", "MXFP4 4096x8192x8192", 2 * 4096 * 8192 * 8192),
                        ("gemm_w4a16_kernel", "W4A16 Qwen2.5-72B up / down", 2 * 2048 * 8192 * 29568)]


def counter_summary(paths):
    """Markdown summary of rocprofv3 counter CSVs of --gemm-counters runs: per
    GEMM kernel (and launch grid) and counter, the mean per dispatch; with
    SQ_BUSY_CU_CYCLES and SQ_VALU_MFMA_BUSY_CYCLES present, the effective
    engine clock (busy CU cycles / 256 CUs / kernel duration) and the share
    of cycles the matrix cores are busy (MFMA-busy cycles / 4 SIMDs / busy
    CU cycles)."""
    import statistics
    groups = {}
    for path in paths:
        for r in _counter_rows(path):
            name = r["Kernel_Name"].replace("(anonymous namespace)::", "").split("(")[0]
            name = name.replace("void ", "")
            key = (name, int(r.get("Grid_Size", r.get("Grid_Size_X", 0)) or 0))
            d = groups.setdefault(key, {})
            d.setdefault(r["Counter_Name"], {})[r["Dispatch_Id"]] = float(r["Counter_Value"])
            if "Start_Timestamp" in r and r["Start_Timestamp"]:
                d.setdefault("_dur_us", {})[r["Dispatch_Id"]] = (
                    int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3
    lines = []
    for (name, grid), d in sorted(groups.items()):
        if not any(k in name for k, _, _ in GEMM_COUNTER_KERNELS):
            continue
        lines.append(f"### `{name}` (grid {grid})")
        lines.append("")
        lines.append("| counter | mean per dispatch | dispatches |")
        lines.append("|---|---:|---:|")
        for cn in sorted(k for k in d if not k.startswith("_")):
            v = list(d[cn].values())
            lines.append(f"| {cn} | {statistics.mean(v):.4g} | {len(v)} |")
        busy = d.get("SQ_BUSY_CU_CYCLES")
        mfma = d.get("SQ_VALU_MFMA_BUSY_CYCLES")
        dur = d.get("_dur_us")
        if busy and mfma:
            b = statistics.mean(busy.values())
            lines.append(f"| MFMA busy share (MFMA-busy / 4 / busy CU cycles) | "
                         f"{statistics.mean(mfma.values()) / 4 / b:.3f} | |")
            if dur:
                lines.append(f"| effective clock (busy CU cycles / 256 / duration), GHz | "
                             f"{b / 256 / statistics.mean(dur.values()) / 1e3:.3f} | |")
        lines.append("")
    print("\n".join(lines))


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


# ------------------------------------------------------------ trace summary

def trace_summary(trace_csv):
    """Markdown summary of a rocprofv3 kernel trace (CSV) of a bench.py run:
    per kernel and launch grid, the dispatch count and the mean, median,
    minimum and maximum duration; then the dominant kernel (the qgemv launch
    with the largest grid, the gate+up projection) over its last
    ROOFLINE_TRIALS * ROOFLINE_REPS dispatches, the graph replays that
    bench.py times for the roofline."""
    import csv
    import statistics
    with open(trace_csv) as f:
        rows = list(csv.DictReader(f))
    groups = {}
    for r in rows:
        key = (r["Kernel_Name"], int(r["Grid_Size_X"]), int(r["Workgroup_Size_X"]))
        groups.setdefault(key, []).append(
            (int(r["Dispatch_Id"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3))
    total = sum(d for v in groups.values() for _, d in v)
    lines = ["| kernel | grid (workgroups x threads) | calls | mean (us) | median (us) | "
             "min (us) | max (us) | share |", "|---|---|---:|---:|---:|---:|---:|---:|"]
    for (name, grid, wg), v in sorted(groups.items(), key=lambda kv: -sum(d for _, d in kv[1])):
        d = [x for _, x in v]
        short = name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")
        lines.append(f"| `{short}` | {grid // wg} x {wg} | {len(d)} | {statistics.mean(d):.2f} | "
                     f"{statistics.median(d):.2f} | {min(d):.2f} | {max(d):.2f} | "
                     f"{100 * sum(d) / total:.1f} % |")
    gemv = [k for k in groups if "qgemv" in k[0]]
    if gemv:
        dom = max(gemv, key=lambda k: (k[1], len(groups[k])))
        last = [d for _, d in sorted(groups[dom])][-ROOFLINE_TRIALS * ROOFLINE_REPS:]
        lines += ["", f"Dominant kernel (largest qgemv grid, {dom[1] // dom[2]} workgroups): "
                      f"last {len(last)} dispatches (the timed graph replays) mean "
                      f"{statistics.mean(last):.3f} us, median {statistics.median(last):.3f} us; "
                      f"{62455808 / statistics.mean(last) / 1e3:.1f} GB/s of the gate+up "
                      f"projection's 62,455,808 algorithmic bytes."]
    print("\n".join(lines))


# ------------------------------------------------------------------- main

def main():
    args = parse()
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.counter_summary:
        counter_summary(args.counter_summary)
        return
    if args.traffic:
        write_traffic(*args.traffic)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
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
    if args.gemm_counters:
        run_gemm_counters()
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

    dom_t, dom_b, dom_min, dom_max = bench_dominant(qg, torch, copies, stream)
    achieved = dom_b / dom_t / 1e9
    traffic = traffic_from_profile(DOMINANT_SRC, DOMINANT_KEY)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic,
                "kernel": "qgemv_wave_kernel<asym, 4 groups/wave, M<=1, tiled codes> (gate+up "
                          "4096->28672, M=1; grid 1792 x 512)",
                "us_per_launch": round(dom_t * 1e6, 3),
                "us_per_launch_min_max": [round(dom_min * 1e6, 3), round(dom_max * 1e6, 3)],
                "timing": f"median of {ROOFLINE_TRIALS} graph replays of {ROOFLINE_REPS} launches",
                "bytes_per_launch": dom_b}

    detail = {}
    cpu = None if args.no_cpu_baseline else {}
    if not args.no_detail:
        detail["decode_projections_m1"] = bench_projections(qg, torch, copies, stream)
        detail["decode_projections_m1_canonical"] = bench_projections(qg, torch, copies, stream,
                                                                      tiled=False)
        detail["decode_swiglu_gate_up"] = bench_swiglu_decode(qg, torch, copies, stream)
        tc = bench_decode(qg, torch, copies, 1, args.steps, args.warmup, stream, tiled=False)
        detail["decode_layer_m1_canonical"] = dict(
            gbs=args.steps * per_layer / tc / 1e9,
            frac=args.steps * per_layer / tc / 1e9 / HBM_PEAK_GBS,
            us_per_layer=tc / args.steps * 1e6)
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
        detail["gemv_4096"] = bench_gemv_4096(qg, torch, dev, stream, cpu)
        log("GEMMs ...")
        detail.update(bench_gemms(qg, torch, dev, stream, cpu))
        log("SmoothQuant and KV cache ...")
        detail.update(bench_smooth_kv(qg, torch, dev, stream))
        log("roofline calibration ...")
        cal = calibration(qg, torch, dev, stream)
        detail["calibration"] = cal
        roofline["calibrated_peak"] = cal["hbm_read_62mb_gbs"]
        roofline["calibrated_peak_note"] = ("read-only stream of the same 62.5 MB per launch "
                                            "(library probe), same graph timing")
        roofline["frac_of_calibrated"] = round(achieved / cal["hbm_read_62mb_gbs"], 4)
        for key, kind in (("fp8_gemm_8192", "fp8"), ("mxfp4_gemm_4096x8192", "fp4"),
                          ("w4a16_prefill_ffn_up", "bf16"), ("w4a16_prefill_ffn_down", "bf16")):
            if key in detail:
                detail[key]["frac_of_calibrated"] = round(
                    detail[key]["tflops"] / cal[f"mfma_{kind}_tflops"], 4)

    if cpu is not None:
        log("CPU oracle baseline ...")
        lay = cpu_baseline(layer)
        cpu = dict(value=lay["value"], unit="GB/s", cores=blas_threads(), kind="oracle",
                   sample=lay["sample"] + f", {lay['seconds']} s",
                   host_cores=host_cores(), blas_threads=blas_threads(),
                   threads_note="quantization in numpy runs on one core; the fp64 products "
                                "use the BLAS threads",
                   per_config=cpu)

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
                               "asymmetric INT4 group 128 (codes in the GEMV tile layout, "
                               "re-laid-out once after quantization)",
                   "bytes_per_step": per_layer, "weight_copies": ncopies},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "context": CONTEXT,
        "detail": detail,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
