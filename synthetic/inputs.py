"""Seeded input generators (numpy PCG64), shaped like the pages' workloads.

Weights are fp32 ~ N(0, 0.02^2); activations are N(0, 1) drawn in fp32 and
rounded to bf16 (torch's round-to-nearest-even conversion).  Outliers are
applied by multiplying chosen entries or input channels before any rounding.
Draw order for every case: W, then X, then outlier indices.

Workloads (shapes from the Llama-3-8B and Qwen2.5-72B tables of
《第 1 章：推理加速全景》 and the configurations of the quantized layer):

* ``gemv_4096``       M=1, K=N=4096, symmetric INT4 group 128, seed 1.
* ``llama3_8b_decode`` K->N = 4096->6144 (QKV), 4096->4096 (O),
  4096->28672 (gate+up), 14336->4096 (down) at M in {1, 4, 16}; asymmetric
  INT4 group 128; 1 % of the input channels of W scaled x20; one child seed
  per shape from SeedSequence(2); M rows are the first M of one 16-row X.
* ``qwen72b_prefill`` M=2048, 8192->29568 and 29568->8192, symmetric INT4,
  seed 3 (child seeds per shape).
* ``fp8_8192``        M=N=K=8192; 0.1 % of the entries of X scaled x100; seed 4.
* ``mxfp4_4096x8192`` M=4096, N=K=8192; 1 % of the input channels of W scaled
  x50; seed 5.

Two further generators: ``smoothquant_case`` (activations whose outliers
sit in 1 % of the input channels, x10, the 5-15x range that
《第 1 章：推理加速全景》 section 4.3 describes) and ``kv_case`` (keys and
values of new tokens for a paged cache: keys with outlier channels, as
《量化与加速》 describes them; a slot mapping through a shuffled block table
with padding entries).
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

__all__ = [
    "rng_for", "normal_weights", "normal_activations", "to_bf16", "bf16_as_f32",
    "scale_input_channels", "scale_random_entries", "Projection", "WORKLOADS",
    "workload_case", "small_case", "norm_weights", "smoothquant_case", "kv_case",
]


def rng_for(seed) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def normal_weights(rng: np.random.Generator, n: int, k: int, std: float = 0.02) -> np.ndarray:
    return (rng.standard_normal((n, k), dtype=np.float32) * np.float32(std)).astype(np.float32)


def normal_activations(rng: np.random.Generator, m: int, k: int) -> np.ndarray:
    return rng.standard_normal((m, k), dtype=np.float32)


def to_bf16(x_f32: np.ndarray) -> torch.Tensor:
    """fp32 numpy -> bf16 torch tensor (CPU), round to nearest even."""
    return torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32)).to(torch.bfloat16)


def bf16_as_f32(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> the same values as fp32 numpy (exact widening)."""
    return t.detach().to("cpu").float().numpy()


def scale_input_channels(rng: np.random.Generator, w: np.ndarray, frac: float, mult: float):
    """Multiply round(frac*K) distinct input channels (columns) of w by mult."""
    k = w.shape[1]
    cnt = int(round(frac * k))
    idx = np.sort(rng.choice(k, size=cnt, replace=False))
    w[:, idx] *= np.float32(mult)
    return idx


def scale_random_entries(rng: np.random.Generator, x: np.ndarray, frac: float, mult: float):
    """Multiply round(frac*size) distinct entries of x by mult."""
    cnt = int(round(frac * x.size))
    idx = rng.choice(x.size, size=cnt, replace=False)
    x.reshape(-1)[idx] *= np.float32(mult)
    return idx


@dataclass
class Projection:
    name: str
    k: int
    n: int


@dataclass
class Workload:
    name: str
    kind: str                      # "w4a16" | "fp8" | "mxfp4"
    projections: list
    ms: tuple
    asym: bool = False
    seed: int = 0
    w_outlier: tuple = field(default=(0.0, 1.0))   # (fraction of input channels, multiplier)
    x_outlier: tuple = field(default=(0.0, 1.0))   # (fraction of entries, multiplier)


WORKLOADS = {
    "gemv_4096": Workload("gemv_4096", "w4a16", [Projection("gemv", 4096, 4096)], (1,), False, 1),
    "llama3_8b_decode": Workload(
        "llama3_8b_decode", "w4a16",
        [Projection("qkv", 4096, 6144), Projection("o", 4096, 4096),
         Projection("gate_up", 4096, 28672), Projection("down", 14336, 4096)],
        (1, 4, 16), True, 2, w_outlier=(0.01, 20.0)),
    "qwen72b_prefill": Workload(
        "qwen72b_prefill", "w4a16",
        [Projection("ffn_up", 8192, 29568), Projection("ffn_down", 29568, 8192)],
        (2048,), False, 3),
    "fp8_8192": Workload("fp8_8192", "fp8", [Projection("gemm", 8192, 8192)], (8192,), False, 4,
                         x_outlier=(0.001, 100.0)),
    "mxfp4_4096x8192": Workload("mxfp4_4096x8192", "mxfp4", [Projection("gemm", 8192, 8192)],
                                (4096,), False, 5, w_outlier=(0.01, 50.0)),
}


def _child_seeds(wl: Workload):
    if len(wl.projections) == 1:
        return [wl.seed]
    return np.random.SeedSequence(wl.seed).spawn(len(wl.projections))


def workload_case(name: str, proj_index: int = 0):
    """Inputs of one projection of a named workload.

    Returns dict(w=fp32 [N][K], x=bf16 torch tensor [max(M)][K], k, n, ms, asym).
    """
    wl = WORKLOADS[name]
    p = wl.projections[proj_index]
    rng = rng_for(_child_seeds(wl)[proj_index])
    w = normal_weights(rng, p.n, p.k)
    x = normal_activations(rng, max(wl.ms), p.k)
    if wl.w_outlier[0] > 0:
        scale_input_channels(rng, w, *wl.w_outlier)
    if wl.x_outlier[0] > 0:
        scale_random_entries(rng, x, *wl.x_outlier)
    return dict(w=w, x=to_bf16(x), k=p.k, n=p.n, ms=wl.ms, asym=wl.asym, name=p.name)


def norm_weights(k: int, seed: int):
    """Seeded normalization weights of K channels: gamma ~ 1 + 0.1 N(0,1),
    beta ~ 0.05 N(0,1), fp32 (the shape of trained norm weights: near one,
    small shifts)."""
    rng = rng_for(seed)
    gamma = (np.float32(1.0) + np.float32(0.1) * rng.standard_normal(k, dtype=np.float32))
    beta = np.float32(0.05) * rng.standard_normal(k, dtype=np.float32)
    return gamma.astype(np.float32), beta.astype(np.float32)


def small_case(m: int, k: int, n: int, seed: int, w_outlier=(0.0, 1.0), x_outlier=(0.0, 1.0),
               w_std: float = 0.02):
    """A small case with the same distributions (for parity at oracle-friendly
    sizes).  Returns dict(w=fp32 [N][K], x=bf16 torch [M][K])."""
    rng = rng_for(seed)
    w = normal_weights(rng, n, k, w_std)
    x = normal_activations(rng, m, k)
    if w_outlier[0] > 0:
        scale_input_channels(rng, w, *w_outlier)
    if x_outlier[0] > 0:
        scale_random_entries(rng, x, *x_outlier)
    return dict(w=w, x=to_bf16(x), k=k, n=n, m=m)


def smoothquant_case(m: int, k: int, n: int, seed: int, frac: float = 0.01, mult: float = 10.0):
    """W fp32 [N][K] ~ N(0, 0.02^2) and X [M][K] ~ N(0, 1) with round(frac*K)
    input channels of X multiplied by mult, rounded to bf16.  Returns
    dict(w, x (bf16 torch), outlier_channels)."""
    rng = rng_for(seed)
    w = normal_weights(rng, n, k)
    x = normal_activations(rng, m, k)
    cnt = int(round(frac * k))
    idx = np.sort(rng.choice(k, size=cnt, replace=False))
    x[:, idx] *= np.float32(mult)
    return dict(w=w, x=to_bf16(x), k=k, n=n, m=m, outlier_channels=idx)


def kv_case(tokens: int, heads: int, head_dim: int, num_slots: int, seed: int,
            block: int = 16, key_outlier=(2, 10.0), padding: int = 0):
    """Keys and values of `tokens` new tokens, bf16 [tokens][heads][head_dim]
    ~ N(0, 1), with key_outlier[0] channels of every key head multiplied by
    key_outlier[1]; and a slot mapping: the tokens fill blocks of `block`
    slots taken in a shuffled order from the num_slots / block blocks of the
    cache (distinct slots), then `padding` entries become -1.  Returns
    dict(k, v (bf16 torch), slots (int64 numpy), key_channels)."""
    rng = rng_for(seed)
    kx = rng.standard_normal((tokens, heads, head_dim), dtype=np.float32)
    vx = rng.standard_normal((tokens, heads, head_dim), dtype=np.float32)
    ch = np.sort(rng.choice(head_dim, size=key_outlier[0], replace=False))
    kx[:, :, ch] *= np.float32(key_outlier[1])
    nblocks = num_slots // block
    need = -(-tokens // block)
    if need > nblocks:
        raise ValueError("cache too small for the tokens")
    order = rng.permutation(nblocks)[:need]
    slots = (order[:, None] * block + np.arange(block)[None, :]).reshape(-1)[:tokens]
    slots = slots.astype(np.int64)
    if padding:
        slots[rng.choice(tokens, size=padding, replace=False)] = -1
    return dict(k=to_bf16(kx), v=to_bf16(vx), slots=slots, key_channels=ch)
