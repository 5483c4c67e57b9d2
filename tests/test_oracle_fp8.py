"""Pins of the oracle's OCP E4M3 codec against the format definition and an
independent library conversion (torch.float8_e4m3fn, round to nearest even)."""
import numpy as np
import pytest
import torch

from oracle import whisper_oracle as O


def test_grid_closed_form():
    v = O.e4m3_value(np.arange(256))
    pos = v[:127]
    assert np.all(np.diff(pos) > 0), "codes 0..126 must be strictly increasing"
    assert pos[0] == 0.0 and pos[1] == 2.0 ** -9          # smallest subnormal
    assert pos[8] == 2.0 ** -6                              # smallest normal
    assert pos[126] == 448.0 == O.E4M3_MAX                  # saturation value (pages: 448)
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.all(v[128:255] == -v[:127])
    # 127 finite non-negative values
    assert np.count_nonzero(np.isfinite(pos)) == 127


def _torch_codes(y32):
    return torch.from_numpy(np.asarray(y32, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encode_matches_torch_all_bf16_patterns():
    bits = np.arange(65536, dtype=np.uint32) << 16
    y = bits.view(np.float32)
    ok = np.isfinite(y) & (np.abs(y) <= 448.0)
    ours = O.e4m3_encode(y[ok])
    ref = _torch_codes(y[ok])
    # torch keeps -0 -> 0x80 and rounds to nearest even, like the oracle
    assert np.array_equal(ours, ref)


def test_encode_matches_torch_random_fp32():
    rng = np.random.default_rng(0)
    y = np.concatenate([rng.standard_normal(200000) * s for s in (1e-3, 0.05, 1.0, 30.0, 150.0)])
    y = y.astype(np.float32)
    y = y[np.abs(y) <= 448]
    assert np.array_equal(O.e4m3_encode(y), _torch_codes(y))


def test_midpoints_go_to_even_code():
    g = O.e4m3_value(np.arange(127))
    mids = ((g[:-1] + g[1:]) / 2).astype(np.float32)
    assert np.all(mids.astype(np.float64) == (g[:-1] + g[1:]) / 2)  # exact in fp32
    codes = O.e4m3_encode(mids).astype(int)
    lo = np.arange(126)
    expect = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(codes, expect)


def test_saturation_and_nan():
    y = np.array([448.0, 449.0, 463.9, 464.0, 1e6, np.inf, -500.0, -np.inf], np.float32)
    assert O.e4m3_encode(y).tolist() == [0x7E] * 6 + [0xFE] * 2
    assert O.e4m3_encode(np.array([np.nan], np.float32))[0] & 0x7F == 0x7F


def test_round_trip_grid_times_power_of_two_scale():
    g = O.e4m3_value(np.arange(127))
    for s in (2.0 ** -8, 0.25, 1.0, 8.0):
        codes = O.e4m3_quantize(g * s, s)
        assert np.array_equal(codes, np.arange(127, dtype=np.uint8))
        assert np.array_equal(O.e4m3_dequantize(codes, s), g * s)
        assert np.array_equal(O.e4m3_quantize(-g[1:] * s, s), (np.arange(1, 127) | 0x80).astype(np.uint8))


def test_quantize_is_single_fp32_multiply_then_round():
    # scale 3 is not a power of two: y = fl32(x * fl32(1/3)) differs from x/3
    x = np.float32(1.3)
    s = np.float32(3.0)
    inv = np.float32(1.0) / s
    y = np.float32(x * inv)
    assert O.e4m3_quantize(np.array([x]), s)[0] == _torch_codes(np.array([y]))[0]


def test_round_trip_error_within_half_ulp():
    rng = np.random.default_rng(1)
    x = rng.uniform(-448, 448, 100000)
    c = O.e4m3_quantize(x, 1.0)
    back = O.e4m3_dequantize(c, 1.0)
    a = np.abs(np.float32(x).astype(np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    ulp = 2.0 ** (e - 3)
    assert np.all(np.abs(back - np.float32(x)) <= ulp / 2 + 1e-30)


def test_scale_from_amax():
    x = np.array([0.5, -3.5, 2.0])
    s = O.e4m3_scale_from_amax(x)
    assert s == np.float32(3.5) / np.float32(448)
    assert O.e4m3_quantize(x, s)[1] == 0xFE   # the largest magnitude maps to -448
    assert O.e4m3_scale_from_amax(np.zeros(3)) == 1.0
