"""GPU parity of the FP8 KV-cache store (qg_kv_cache_store) against the CPU
oracle: per token and head, and with static per-channel scales calibrated by
qg_channel_absmax + qg_channel_scales; codes and scales bit-exact in every
written slot, every other slot untouched (padding and out-of-range slots
skipped), bf16 and fp32 sources, head dims from 8 to 512 (including ones
that are not a power of two times 8), a single token, no tokens at all, and
a Llama-3-8B prefill chunk (8192 tokens, 8 KV heads of 128) into a 16-token
paged cache."""

import numpy as np
import pytest
import torch

import quantized_gemm_group_amd as qg
from oracle import kvcache as okv, smooth as osm
from synthetic import bf16_as_f32, kv_case, rng_for
from tests.gpu_util import bits32, device, host, to_dev

pytestmark = pytest.mark.gpu

SENTINEL_CODE = 0xAB
SENTINEL_SCALE = -7.0


def fresh_cache(slots, heads, d, dev, per_token=True):
    codes = torch.full((slots, heads, d), SENTINEL_CODE, dtype=torch.uint8, device=dev)
    scales = (torch.full((slots * heads,), SENTINEL_SCALE, dtype=torch.float32, device=dev)
              if per_token else None)
    return codes, scales


def check_store(x_dev, x_ref, slots, num_slots, per_channel, dev, calib_ref=None):
    t, h, d = x_ref.shape
    codes, scales = fresh_cache(num_slots, h, d, dev, per_token=not per_channel)
    cs_dev = cs_ref = None
    if per_channel:
        # static scales from calibration keys: channel maxima over tokens
        calib = x_ref if calib_ref is None else calib_ref
        amax = osm.channel_absmax(calib.reshape(calib.shape[0], h * d) * np.float32(0.8))
        cs_ref = okv.channel_scales(amax).reshape(h, d)
        cs_dev = qg.channel_scales(qg.channel_absmax(
            to_dev(calib.reshape(calib.shape[0], h * d) * np.float32(0.8), dev)), 448.0).reshape(h, d)
        assert (bits32(host(cs_dev)) == bits32(cs_ref)).all()
    qg.kv_cache_store(x_dev, to_dev(slots, dev), codes, scales, cs_dev)
    rc, rs = okv.cache_store(x_ref, slots, np.full((num_slots, h, d), SENTINEL_CODE, np.uint8),
                             None if per_channel else np.full((num_slots, h), SENTINEL_SCALE,
                                                              np.float32), cs_ref)
    got = host(codes)
    bad = np.argwhere(got != rc)
    assert len(bad) == 0, f"{len(bad)} code mismatches, first {bad[:4].tolist()}"
    if not per_channel:
        assert (bits32(host(scales).reshape(num_slots, h)) == bits32(rs)).all()


@pytest.mark.parametrize("per_channel", [False, True])
@pytest.mark.parametrize("src", ["bf16", "f32"])
@pytest.mark.parametrize("t,h,d,slots", [(37, 8, 128, 640), (1, 4, 64, 16), (50, 3, 8, 64),
                                         (20, 2, 96, 48), (9, 1, 512, 32), (65, 5, 200, 96),
                                         (33, 32, 256, 48)])
def test_kv_cache_store_bit_exact(t, h, d, slots, src, per_channel):
    dev = device()
    print(f"kv_cache_store T={t} H={h} D={d} slots={slots} {src} per_channel={per_channel}",
          flush=True)
    c = kv_case(t, h, d, slots, seed=t * 31 + d, block=1 if slots < 2 * t else 8,
                padding=min(3, t // 4))
    x = bf16_as_f32(c["k"])
    # two tokens pointed past the cache: skipped like padding
    sl = c["slots"].copy()
    if t > 4:
        sl[2], sl[4] = slots, slots + 1000
    if src == "bf16":
        x_dev = to_dev(c["k"], dev)
    else:
        x = x * np.float32(1.7)
        x_dev = to_dev(x, dev)
    check_store(x_dev, x, sl, slots, per_channel, dev)


def test_kv_cache_store_no_tokens_and_all_zero_head():
    dev = device()
    codes, scales = fresh_cache(16, 2, 64, dev)
    empty = torch.empty((0, 2, 64), dtype=torch.bfloat16, device=dev)
    qg.kv_cache_store(empty, torch.empty(0, dtype=torch.int64, device=dev), codes, scales)
    assert (host(codes) == SENTINEL_CODE).all() and (host(scales) == SENTINEL_SCALE).all()
    # an all-zero head gets scale 1 and zero codes
    x = np.zeros((3, 2, 64), np.float32)
    x[1, 1, 5] = -3.0
    check_store(to_dev(x, dev), x, np.array([4, 0, 15], np.int64), 16, False, dev)


def test_values_beyond_calibration_saturate():
    dev = device()
    rng = rng_for(12)
    calib = rng.standard_normal((64, 2, 32), dtype=np.float32)
    x = calib[:8] * np.float32(4)          # up to 4 / 0.8 = 5x the calibrated range
    check_store(to_dev(x, dev), x, np.arange(8, dtype=np.int64), 8, True, dev, calib_ref=calib)


def test_llama3_8b_prefill_chunk_into_paged_cache():
    # 8192 new tokens, 8 KV heads x 128 (Llama-3-8B), 16-token blocks of a
    # 32768-slot cache; keys with static per-channel scales, values per token
    dev = device()
    print("kv_cache_store Llama-3-8B prefill chunk 8192 x 8 x 128", flush=True)
    c = kv_case(8192, 8, 128, 32768, seed=13, padding=16)
    k_ref, v_ref = bf16_as_f32(c["k"]), bf16_as_f32(c["v"])
    check_store(to_dev(c["v"], dev), v_ref, c["slots"], 32768, False, dev)
    check_store(to_dev(c["k"], dev), k_ref, c["slots"], 32768, True, dev)


def test_per_token_cache_reads_back_through_dequant():
    # the per-token layout is FP8 rows of heads * head_dim with one scale
    # per head: qg_dequant with group = head_dim decodes it
    dev = device()
    t, h, d, slots = 24, 4, 128, 32
    c = kv_case(t, h, d, slots, seed=21, block=8)
    codes, scales = fresh_cache(slots, h, d, dev)
    qg.kv_cache_store(to_dev(c["v"], dev), to_dev(c["slots"], dev), codes, scales)
    got = host(qg.dequant(codes.reshape(slots, h * d), scales.reshape(slots, h), None,
                          "fp8_e4m3", h * d, group=d))
    rc, rs = okv.quantize_tokens(bf16_as_f32(c["v"]))
    from oracle import formats as F
    ref = (F.decode(rc, "e4m3") * rs[:, :, None].astype(np.float64)).astype(np.float32)
    assert (bits32(got[c["slots"]].reshape(t, h, d)) == bits32(ref)).all()
