"""The branch-free E4M3 rounding of the fp8 decode GEMM's second site
(whisper_e4m3_round_host: the same source the kernel runs, evaluated on the
host) against the oracle's codec: the value of the OCP E4M3FN code, round to
nearest even, saturating at 448 (fp8_quantize.cu card of the showcase page;
OCP format definition), for every finite bf16 value (the site's inputs are
bf16 rows times a reciprocal scale) and for fp32 values on and next to every
rounding midpoint."""
import numpy as np

from oracle import whisper_oracle as O
from speech_recognition_amd import _lib as L


def _oracle_round(y):
    y = np.asarray(y, np.float32)
    return O.e4m3_value(O.e4m3_encode(y)).astype(np.float32)


def test_every_finite_bf16_value():
    bits = np.arange(1 << 16, dtype=np.uint32)
    y = (bits << 16).view(np.float32)
    y = y[np.isfinite(y)]
    got = L.whisper_e4m3_round_host(y)
    want = _oracle_round(y)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_midpoints_and_neighbours():
    # every E4M3 magnitude and the midpoints between neighbours, with the
    # fp32 values one step either side, both signs, plus the range above 448
    mags = np.unique(np.abs(O.e4m3_value(np.arange(0x7f, dtype=np.uint8))))
    mid = (mags[:-1] + mags[1:]) / 2
    pts = np.concatenate([mags, mid, [448.0, 456.0, 460.0, 464.0, 500.0, 1e6]]).astype(np.float32)
    pts = np.concatenate([pts, np.nextafter(pts, np.float32(0)), np.nextafter(pts, np.float32(np.inf))])
    pts = np.concatenate([pts, -pts]).astype(np.float32)
    got = L.whisper_e4m3_round_host(pts)
    want = _oracle_round(pts)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_random_fp32():
    rng = np.random.default_rng(5)
    y = (rng.standard_normal(1 << 20) * np.exp2(rng.uniform(-14, 9, 1 << 20))).astype(np.float32)
    got = L.whisper_e4m3_round_host(y)
    want = _oracle_round(y)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
