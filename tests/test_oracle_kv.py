"""Pins of the oracle's FP8 KV-cache quantization (《推理优化与量化算子深度技术调研》
section 1.6; 《量化与加速》 KV-cache section): hand-worked per-token and
per-channel codes, saturation beyond the calibrated range, the slot mapping
against a brute-force dictionary of writes (padding and out-of-range slots
skipped, other slots untouched), the error bound of the per-token scale, and
the pages' claim that keys with outlier channels quantize better per
channel."""

import numpy as np
import pytest

from oracle import formats as F
from oracle import kvcache as KV


def test_per_token_hand_example():
    # one token, two heads of 4: head 0 has max 448 -> scale 1, codes of the
    # exact E4M3 values; head 1 has max 896 -> scale 2; an all-zero head -> 1
    x = np.array([[[448, -224, 1, 0], [896, 3, -0.5, 2]]], np.float32)
    codes, s = KV.quantize_tokens(x)
    assert s.tolist() == [[1.0, 2.0]]
    assert codes[0, 0].tolist() == [0x7E, 0xF6, 0x38, 0x00]       # 448, -224, 1, 0
    assert codes[0, 1].tolist() == [0x7E, 0x3C, 0xA8, 0x38]       # 448, 1.5, -0.25, 1
    z, sz = KV.quantize_tokens(np.zeros((2, 1, 8), np.float32))
    assert (z == 0).all() and (sz == 1).all()


def test_per_token_error_bound():
    # |x - s dec(q)| <= s * 2^-4 * 2^e(|x|/s) per element (half an E4M3 step)
    rng = np.random.default_rng(1)
    x = rng.standard_normal((16, 8, 128)).astype(np.float32)
    codes, s = KV.quantize_tokens(x)
    xh = F.decode(codes, "e4m3") * s[:, :, None].astype(np.float64)
    v = np.abs(x.astype(np.float64) / s[:, :, None])
    step = np.exp2(np.floor(np.log2(np.maximum(v, 2.0 ** -6))) - 3)
    assert (np.abs(x - xh) <= 0.5 * step * s[:, :, None] * (1 + 1e-6)).all()
    # the per-head maximum is represented exactly (it maps to 448)
    amax_code = np.take_along_axis(codes, np.abs(x).argmax(-1)[..., None], -1)
    assert ((amax_code & 0x7F) == 0x7E).all()


def test_channel_scales_and_saturation():
    s = KV.channel_scales(np.float32([448, 0, 896, 1]))
    assert s[:3].tolist() == [1.0, 1.0, 2.0] and s[3] == np.float32(1) / np.float32(448)
    cs = np.array([[1.0, 1.0, 2.0, 1.0]], np.float32)
    x = np.array([[[500, -1000, 1792, 448]]], np.float32)
    codes, none = KV.quantize_tokens(x, cs)
    assert none is None
    # 500 and 1000 exceed the calibrated range and saturate to +-448; 1792 / 2
    # = 896 saturates too; 448 is exact
    assert codes[0, 0].tolist() == [0x7E, 0xFE, 0x7E, 0x7E]
    with pytest.raises(ValueError, match="invalid quantization geometry"):
        KV.quantize_tokens(x, np.ones((1, 3), np.float32))


@pytest.mark.parametrize("per_channel", [False, True])
def test_cache_store_brute_force(per_channel):
    rng = np.random.default_rng(2)
    t, h, d, slots = 9, 2, 16, 32
    x = rng.standard_normal((t, h, d)).astype(np.float32)
    mapping = np.array([5, 0, -1, 31, 7, 40, 12, -3, 2], np.int64)   # padding, out of range
    cache = np.full((slots, h, d), 0xAB, np.uint8)
    scales = np.full((slots, h), -7.0, np.float32)
    cs = KV.channel_scales(np.abs(x).max(axis=0) * 0.9) if per_channel else None
    cc, sc = KV.cache_store(x, mapping, cache, None if per_channel else scales, cs)
    codes, s = KV.quantize_tokens(x, cs)
    written = {int(m): i for i, m in enumerate(mapping) if 0 <= m < slots}
    for slot in range(slots):
        if slot in written:
            assert (cc[slot] == codes[written[slot]]).all()
            if not per_channel:
                assert (sc[slot] == s[written[slot]]).all()
        else:
            assert (cc[slot] == 0xAB).all()
            if not per_channel:
                assert (sc[slot] == -7.0).all()
    assert sc is None if per_channel else sc.shape == (slots, h)


def test_outlier_key_channels_prefer_per_channel_scales():
    # keys with a few very large channels (the page's reason for per-channel
    # key scales): under a per-token scale the small channels fall below
    # E4M3's normal range and lose their precision; per-channel scales keep
    # each channel's relative error at E4M3's half step
    rng = np.random.default_rng(3)
    t, h, d = 256, 4, 128
    k = rng.standard_normal((t, h, d)).astype(np.float32) * 0.01
    k[:, :, [3, 77]] *= 1e5
    cs = KV.channel_scales(np.abs(k).max(axis=0))
    c_tok, s_tok = KV.quantize_tokens(k)
    c_ch, _ = KV.quantize_tokens(k, cs)
    small = np.ones(d, bool)
    small[[3, 77]] = False
    k64 = k.astype(np.float64)[..., small]
    e_tok = np.abs(F.decode(c_tok, "e4m3")[..., small] * s_tok[..., None] - k64)
    e_ch = np.abs(F.decode(c_ch, "e4m3")[..., small] * cs[None][..., small] - k64)
    assert e_ch.sum() < 0.25 * e_tok.sum()
    assert (e_ch <= np.abs(k64) * 2.0 ** -4 + cs[None][..., small] * 2.0 ** -10).all()
