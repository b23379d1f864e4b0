"""FP8 E4M3 KV-cache quantization into a paged cache.

Test infrastructure only (see the package docstring).

Definitions followed: 《推理优化与量化算子深度技术调研》 section 1.6 (FP8 KV
cache at two granularities: per token, a scale from the token's absolute
maximum over the head dimension; per channel, one scale per element of the
head dimension taken over the tokens); 《量化与加速》 KV-cache section (keys
carry outlier channels and suit per-channel scales, values suit per-token
scales; FP8 halves the cache).

Readings (each also listed in the design notes):

* E4M3 is OCP E4M3FN with maximum 448, as everywhere in this library; the
  section's divisor 240 is the maximum of the FNUZ variant of older hardware.
* Per-token granularity is per token and per KV head: the scale of head h of
  token t is max_d |x[t][h][d]| / 448 (float32), 1 when that is zero; the code
  is the saturating, ties-to-even E4M3 value of fl32(x / scale).
* Per-channel granularity uses static scales [heads][head_dim] fixed before
  the tokens arrive (a cache cannot rescale codes already written): by
  calibration, the channel absolute maximum over calibration tokens / 448,
  1 where that is zero.  Values beyond the calibrated range saturate to
  +-448.
* Paged layout: codes [num_slots][heads][head_dim] bytes, per-token scales
  [num_slots][heads] float32; token t goes to slot slot_mapping[t]; a slot
  outside [0, num_slots) (negative marks padding) is skipped; the slots of
  one call are distinct.
"""
from __future__ import annotations

import numpy as np

from . import fp8
from .formats import encode

E4M3_MAX = 448.0


def channel_scales(absmax, qmax: float = E4M3_MAX) -> np.ndarray:
    """Static per-channel scales from calibration maxima: absmax / qmax in
    float32, 1 where zero."""
    a = np.asarray(absmax, dtype=np.float32)
    s = (a / np.float32(qmax)).astype(np.float32)
    return np.where(s == 0, np.float32(1.0), s).astype(np.float32)


def quantize_tokens(x, channel_scale=None):
    """x [T][H][D] (float32 values).  Per-token (channel_scale None): returns
    (codes uint8 [T][H][D], scales float32 [T][H]).  Per-channel: returns
    (codes, None) with scales [H][D] given."""
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 3 or 0 in x.shape:
        raise ValueError("invalid quantization geometry")
    t, h, d = x.shape
    if channel_scale is None:
        codes, s = fp8.quantize_rows(x.reshape(t * h, d))
        return codes.reshape(t, h, d), np.asarray(s, np.float32).reshape(t, h)
    cs = np.asarray(channel_scale, dtype=np.float32)
    if cs.shape != (h, d):
        raise ValueError("invalid quantization geometry")
    v = (x / cs[None, :, :]).astype(np.float32)
    return encode(v, "e4m3").reshape(t, h, d), None


def cache_store(x, slot_mapping, cache_codes, cache_scales=None, channel_scale=None):
    """Quantize x [T][H][D] and write token t into slot slot_mapping[t] of
    copies of cache_codes [S][H][D] (and cache_scales [S][H] in the per-token
    mode).  Returns the updated copies."""
    codes, scales = quantize_tokens(x, channel_scale)
    cc = np.array(cache_codes, dtype=np.uint8, copy=True)
    cs = None if cache_scales is None else np.array(cache_scales, dtype=np.float32, copy=True)
    slots = np.asarray(slot_mapping, dtype=np.int64).reshape(-1)
    if slots.shape[0] != codes.shape[0] or cc.shape[1:] != codes.shape[1:]:
        raise ValueError("invalid quantization geometry")
    for t, slot in enumerate(slots):
        if 0 <= slot < cc.shape[0]:
            cc[slot] = codes[t]
            if scales is not None:
                cs[slot] = scales[t]
    return cc, cs
