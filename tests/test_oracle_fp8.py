"""Pins of the oracle's FP8 E4M3 decoding and FP8-cache attention against facts
fixed outside it: the format's landmark values, torch's own float8_e4m3fn
conversion of all 256 codes, ordering and sign symmetry, and attention over a
cache whose codes are exact small integers."""
import math

import numpy as np
import torch

import attn_inputs as A
from oracle import attention_fp8kv_ref, attention_ref, dequant_e4m3, e4m3_value


def test_landmark_values_of_the_format():
    assert e4m3_value(0x00) == 0.0 and math.copysign(1, e4m3_value(0x80)) == -1
    assert e4m3_value(0x38) == 1.0 and e4m3_value(0xB8) == -1.0     # exponent field 7 = bias
    assert e4m3_value(0x7E) == 448.0                                  # largest finite
    assert e4m3_value(0x08) == 2.0 ** -6                              # smallest normal
    assert e4m3_value(0x01) == 2.0 ** -9                              # smallest subnormal
    assert e4m3_value(0x07) == 7 * 2.0 ** -9                          # largest subnormal
    assert e4m3_value(0x40) == 2.0 and e4m3_value(0x3C) == 1.5
    assert math.isnan(e4m3_value(0x7F)) and math.isnan(e4m3_value(0xFF))
    assert not any(math.isinf(e4m3_value(c)) for c in range(256))


def test_all_codes_match_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = dequant_e4m3(np.arange(256, dtype=np.uint8), 1.0)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(ref[~nan], ours[~nan])


def test_positive_codes_are_ordered_and_signs_mirror():
    v = [e4m3_value(c) for c in range(0x7F)]
    assert all(a < b for a, b in zip(v, v[1:]))
    for c in range(0x7F):
        assert e4m3_value(c | 0x80) == -e4m3_value(c)


def test_scale_multiplies_every_value():
    codes = np.arange(0, 0x7F, dtype=np.uint8)
    np.testing.assert_array_equal(dequant_e4m3(codes, 0.25), dequant_e4m3(codes, 1.0) / 4)


def test_fp8_attention_is_attention_over_dequantised_values():
    # codes 0x38 (1.0), 0x40 (2.0), 0x30 (0.5): with scale 2 the cache is {2, 4, 1}
    B, Hq, Hkv, N, d = 1, 2, 1, 3, 4
    kc = np.array([0x38, 0x40, 0x30], np.uint8)[None, None, :, None].repeat(d, axis=3)
    vc = np.array([0x30, 0x38, 0x40], np.uint8)[None, None, :, None].repeat(d, axis=3)
    q = np.ones((B, Hq, 1, d), np.float32) * np.float32(0.125)
    o, lse = attention_fp8kv_ref(q, kc, vc, 2.0, 2.0, False, 0.5)
    # scores: 0.5 * (0.125 * 4 * k) = 0.25 * k for k in {2, 4, 1}
    s = np.array([0.5, 1.0, 0.25])
    w = np.exp(s - s.max()) / np.exp(s - s.max()).sum()
    vals = np.array([1.0, 2.0, 4.0])
    np.testing.assert_allclose(o[0, 0, 0], np.full(d, (w * vals).sum()), rtol=1e-15)
    np.testing.assert_allclose(lse[0, 0, 0], np.log(np.exp(s).sum()), rtol=1e-15)
    o2, _ = attention_ref(q, 2.0 * np.array([1.0, 2.0, 0.5])[None, None, :, None].repeat(d, 3),
                          2.0 * np.array([0.5, 1.0, 2.0])[None, None, :, None].repeat(d, 3), False, 0.5)
    np.testing.assert_array_equal(o, o2)


def test_fp8_codes_generator_round_trips_through_the_format():
    codes = A.fp8_codes((4, 1000), seed=3, scale=2.0 ** -6)
    assert codes.dtype == np.uint8
    vals = dequant_e4m3(codes, 2.0 ** -6)
    assert np.all(np.isfinite(vals)) and np.abs(vals).max() <= 448 * 2.0 ** -6
    x = A.fp8_codes((4, 1000), seed=3, scale=2.0 ** -6)
    assert np.array_equal(codes, x)
    # values of N(0, 1): the spread of the decoded cache is about 1
    assert 0.9 < float(vals.std()) < 1.1
