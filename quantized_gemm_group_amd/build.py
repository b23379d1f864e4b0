"""Build the HIP library libqgemm.so in-tree for gfx950.

Each translation unit under csrc/ is compiled with hipcc in parallel, then
linked into quantized_gemm_group_amd/libqgemm.so; the same sources built
with QG_DEBUG_FP32 give libqgemm_debug.so (fp32 outputs before the bf16
rounding recorded on request).  Run as a script or call ``build()``; it
always recompiles.
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libqgemm.so")
ARCH = os.environ.get("QG_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions stay off (the compiler would otherwise form them)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # exact IEEE division for quantization decisions; keep fp32 denormals
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
    "-ffp-contract=fast",
    "-I", os.path.join(ROOT, "include"),
    "-Wno-unused-command-line-argument",
]


LIB_DEBUG = os.path.join(HERE, "libqgemm_debug.so")


def _compile(job) -> str:
    src, debug = job
    odir = OBJ + ("_debug" if debug else "")
    obj = os.path.join(odir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *(["-DQG_DEBUG_FP32"] if debug else []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = True) -> str:
    """Build libqgemm.so (the product) and libqgemm_debug.so (the same
    sources with QG_DEBUG_FP32: kernels also record their fp32 outputs
    before the bf16 rounding)."""
    os.makedirs(OBJ, exist_ok=True)
    os.makedirs(OBJ + "_debug", exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = [(s, False) for s in srcs] + [(s, True) for s in srcs]
    workers = max(1, min(8, os.cpu_count() or 1))
    with cf.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(_compile, jobs))
    _link(objs[:len(srcs)], LIB)
    _link(objs[len(srcs):], LIB_DEBUG)
    if verbose:
        print(f"built {LIB} and {LIB_DEBUG} from {len(srcs)} sources")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
