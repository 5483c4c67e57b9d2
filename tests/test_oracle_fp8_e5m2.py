"""Pins of the oracle's OCP E5M2 codec against the format definition (E5M2 is
IEEE binary16 cut to its top byte) and an independent library conversion
(torch.float8_e5m2, round to nearest even; it overflows to inf where the
oracle saturates, so the two are compared inside the finite range)."""
import numpy as np
import torch

from oracle import whisper_oracle as O


def test_grid_is_binary16_top_byte():
    codes = np.arange(256, dtype=np.uint16)
    half = (codes << 8).view(np.float16).astype(np.float64)
    v = O.e5m2_value(codes)
    fin = np.isfinite(half)
    assert np.array_equal(v[fin], half[fin])
    assert np.array_equal(np.isnan(v), np.isnan(half))
    assert np.array_equal(np.isinf(v) & (v > 0), np.isinf(half) & (half > 0))
    assert np.array_equal(np.isinf(v) & (v < 0), np.isinf(half) & (half < 0))


def test_grid_closed_form():
    v = O.e5m2_value(np.arange(256))
    pos = v[:124]
    assert np.all(np.diff(pos) > 0)
    assert pos[0] == 0.0 and pos[1] == 2.0 ** -16            # smallest subnormal
    assert pos[4] == 2.0 ** -14                                # smallest normal
    assert pos[123] == 57344.0 == O.E5M2_MAX == 1.75 * 2.0 ** 15
    assert v[0x7C] == np.inf and v[0xFC] == -np.inf
    assert all(np.isnan(v[c]) for c in (0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF))
    assert np.all(v[128:252] == -v[:124])


def _torch_codes(y32):
    return torch.from_numpy(np.asarray(y32, np.float32)).to(torch.float8_e5m2).view(torch.uint8).numpy()


def test_encode_matches_torch_all_bf16_patterns():
    bits = np.arange(65536, dtype=np.uint32) << 16
    y = bits.view(np.float32)
    ok = np.isfinite(y) & (np.abs(y) <= 57344.0)
    assert np.array_equal(O.e5m2_encode(y[ok]), _torch_codes(y[ok]))


def test_encode_matches_torch_random_fp32():
    rng = np.random.default_rng(0)
    y = np.concatenate([rng.standard_normal(200000) * s for s in (1e-5, 1e-3, 1.0, 300.0, 2e4)])
    y = y.astype(np.float32)
    y = y[np.abs(y) <= 57344]
    assert np.array_equal(O.e5m2_encode(y), _torch_codes(y))


def test_midpoints_go_to_even_code():
    g = O.e5m2_value(np.arange(124))
    mids = ((g[:-1] + g[1:]) / 2).astype(np.float32)
    assert np.all(mids.astype(np.float64) == (g[:-1] + g[1:]) / 2)  # exact in fp32
    codes = O.e5m2_encode(mids).astype(int)
    lo = np.arange(123)
    assert np.array_equal(codes, np.where(lo % 2 == 0, lo, lo + 1))


def test_normal_range_rounding_closed_form():
    # in the normal range the code's value is |y| rounded to 2 fraction bits
    # of its binade: rint(|y| / 2^(e-2)) * 2^(e-2), e = floor(log2 |y|)
    rng = np.random.default_rng(3)
    y = (np.exp2(rng.uniform(-14, 15.8, 100000)) * rng.choice([-1, 1], 100000)).astype(np.float32)
    a = np.abs(y.astype(np.float64))
    e = np.floor(np.log2(a))
    want = np.minimum(np.rint(a / 2.0 ** (e - 2)) * 2.0 ** (e - 2), 57344.0) * np.sign(y)
    assert np.array_equal(O.e5m2_value(O.e5m2_encode(y)), want)


def test_saturation_sign_and_nan():
    y = np.array([57344.0, 57345.0, 61439.0, 61440.0, 1e9, np.inf, -6e4, -np.inf], np.float32)
    assert O.e5m2_encode(y).tolist() == [0x7B] * 6 + [0xFB] * 2
    assert O.e5m2_encode(np.array([np.nan], np.float32))[0] & 0x7F == 0x7F
    assert O.e5m2_encode(np.array([-0.0], np.float32))[0] == 0x80


def test_round_trip_grid_and_error_bound():
    g = O.e5m2_value(np.arange(124))
    for s in (2.0 ** -10, 0.5, 1.0, 4.0):
        codes = O.e5m2_quantize(g * s, s)
        assert np.array_equal(codes, np.arange(124, dtype=np.uint8))
        assert np.array_equal(O.e5m2_dequantize(codes, s), g * s)
    rng = np.random.default_rng(1)
    x = rng.uniform(-57344, 57344, 100000) * np.exp2(rng.integers(-20, 1, 100000))
    back = O.e5m2_dequantize(O.e5m2_quantize(x, 1.0), 1.0)
    a = np.abs(np.float32(x).astype(np.float64))
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -14))) - 2)
    assert np.all(np.abs(back - np.float32(x)) <= ulp / 2 + 1e-30)


def test_scale_from_amax_and_format_table():
    x = np.array([0.5, -3.5, 2.0])
    s = O.e5m2_scale_from_amax(x)
    assert s == np.float32(3.5) / np.float32(57344)
    assert O.e5m2_quantize(x, s)[1] == 0xFB   # the largest magnitude maps to -57344
    assert O.e5m2_scale_from_amax(np.zeros(3)) == 1.0
    assert O.FP8_FORMATS["e5m2"][0] is O.e5m2_quantize and O.FP8_FORMATS["e4m3"][0] is O.e4m3_quantize


def test_e5m2_keeps_range_e4m3_clips_without_scaling():
    # with unit scale a value of 1000 is kept (to 1/8 relative) by E5M2 and
    # clipped to 448 by E4M3: the range argument for E5M2 on cross-attention
    x = np.array([1000.0, 1e-5])
    assert abs(O.e5m2_dequantize(O.e5m2_quantize(x, 1.0), 1.0)[0] - 1000.0) <= 1000.0 / 8
    assert O.e4m3_dequantize(O.e4m3_quantize(x, 1.0), 1.0)[0] == 448.0
    assert O.e5m2_dequantize(O.e5m2_quantize(x, 1.0), 1.0)[1] != 0.0
    assert O.e4m3_dequantize(O.e4m3_quantize(x, 1.0), 1.0)[1] == 0.0
