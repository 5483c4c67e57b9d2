"""Pins of the oracle's log-mel front end: torch.stft (independent framing,
reflect padding and FFT), a direct O(N^2) DFT, closed forms for a pure tone
and for silence, and the Slaney filterbank's defining properties."""
import numpy as np
import torch

from oracle import whisper_oracle as O


def _audio(seconds=3.0, seed=0):
    rng = np.random.default_rng(seed)
    n = int(seconds * 16000)
    t = np.arange(n) / 16000
    x = 0.2 * np.sin(2 * np.pi * 440 * t) + 0.1 * np.sin(2 * np.pi * 1700 * t + 1) + 0.05 * rng.standard_normal(n)
    return x


def test_power_spectrum_matches_torch_stft():
    a = _audio(30.0)
    ref = torch.stft(torch.from_numpy(a), n_fft=400, hop_length=160, window=torch.hann_window(400, dtype=torch.float64),
                     center=True, pad_mode="reflect", return_complex=True)
    ref = (ref.abs() ** 2).numpy()[:, :3000].T
    got = O.power_spectrum(a)
    assert got.shape == (3000, 201)
    assert np.allclose(got, ref, rtol=1e-9, atol=1e-12 * ref.max())


def test_rfft_equals_direct_dft():
    fr = O.frames(_audio(1.0))[37] * O.hann_periodic()
    n = np.arange(400)
    k = np.arange(201)[:, None]
    direct = (fr[None, :] * np.exp(-2j * np.pi * k * n / 400)).sum(axis=1)
    assert np.allclose(np.abs(direct) ** 2, O.power_spectrum(_audio(1.0))[37], rtol=1e-9, atol=1e-9)


def test_periodic_hann():
    w = O.hann_periodic()
    assert w[0] == 0.0 and abs(w[200] - 1.0) < 1e-15 and abs(w[100] - 0.5) < 1e-15
    assert np.allclose(w[1:], w[1:][::-1])      # periodic: symmetric about n = 200


def test_pure_tone_at_bin_centre():
    # f = 40 k Hz falls on bin k of a 400-point DFT at 16 kHz; the periodic Hann
    # window's DFT is N/2 at 0 and -N/4 at +-1, so |X[k]| = A N/4 = 100 A,
    # |X[k+-1]| = 50 A and every other bin is 0.
    for k0, amp, ph in ((2, 0.3, 0.0), (37, 0.7, 1.1), (150, 0.25, 2.0), (198, 1.0, 0.3)):
        t = np.arange(480000) / 16000
        p = O.power_spectrum(amp * np.cos(2 * np.pi * 40 * k0 * t + ph))
        mag = np.sqrt(p[1500])
        assert abs(mag[k0] - 100 * amp) < 1e-8
        assert abs(mag[k0 - 1] - 50 * amp) < 1e-8 and abs(mag[k0 + 1] - 50 * amp) < 1e-8
        others = np.delete(mag, [k0 - 1, k0, k0 + 1])
        assert others.max() < 1e-8


def test_silence_gives_minus_one_and_a_half():
    out = O.log_mel(np.zeros(480000), 128)
    assert out.shape == (128, 3000)
    assert np.all(out == -1.5)


def test_padding_frames_sit_at_clamp_floor():
    a = _audio(10.0)                      # 10 s of signal, then 20 s of zeros
    out = O.log_mel(a, 80)
    raw = O.log_mel_unnormalised(a, 80)
    floor = (raw.max() - 8.0 + 4.0) / 4.0
    first_silent = (160000 + 200) // 160 + 1  # frames wholly inside the zero tail
    assert np.all(out[:, first_silent:] == floor)
    assert out.max() == (raw.max() + 4.0) / 4.0


def test_slaney_mel_scale():
    assert abs(O.hz_to_mel(1000.0) - 15.0) < 1e-12
    assert abs(O.hz_to_mel(6400.0) - 42.0) < 1e-12      # one log step of 6.4 = 27 mel
    assert np.allclose(O.hz_to_mel(np.array([0.0, 200.0, 500.0])), [0.0, 3.0, 7.5])
    f = np.linspace(0, 8000, 1001)
    assert np.allclose(O.mel_to_hz(O.hz_to_mel(f)), f, atol=1e-9)


def test_filterbank_shape_support_and_area():
    for n_mels in (80, 128):
        fb = O.mel_filterbank(n_mels)
        assert fb.shape == (n_mels, 201)
        assert np.all(fb >= 0)
        assert np.all((fb > 0).sum(axis=1) >= 1)              # no empty filter
        pts = O.mel_to_hz(np.linspace(0, O.hz_to_mel(8000.0), n_mels + 2))
        freqs = np.arange(201) * 40.0
        for m in range(n_mels):
            lo, c, hi = pts[m], pts[m + 1], pts[m + 2]
            nz = freqs[fb[m] > 0]
            assert nz.min() > lo and nz.max() < hi
            # piecewise-linear interpolation of the triangle's three vertices
            tri = np.interp(freqs, [lo, c, hi], [0.0, 2.0 / (hi - lo), 0.0], left=0.0, right=0.0)
            assert np.allclose(fb[m], tri, atol=1e-15)
            # the continuous triangle has unit area: base (hi-lo) * height / 2
            assert abs((hi - lo) * (2.0 / (hi - lo)) / 2 - 1.0) < 1e-15
        # filters tile the axis: the sum of areas seen on the 40 Hz grid is ~ n_mels
        # for the wide (upper) filters
        assert abs(fb[n_mels // 2:].sum() * 40.0 - n_mels // 2) < 0.05 * n_mels


def test_log_mel_composition():
    a = _audio(30.0, seed=3)
    out = O.log_mel(a, 128)
    mel = O.power_spectrum(a) @ O.mel_filterbank(128).T
    lg = np.log10(np.maximum(mel, 1e-10)).T
    assert np.allclose(out, (np.maximum(lg, lg.max() - 8) + 4) / 4)
    assert out.min() >= (lg.max() - 8 + 4) / 4 - 1e-12


# ------------------------------------------------------------------ overlapping chunks of one recording
def test_chunk_plan_owned_frames_partition_the_recording():
    """Owned frames (chunk-local plus the chunk's first frame) tile the frames
    of the recording exactly once, for strides with and without overlap and
    lengths around the window edge; chunk starts step by the stride; the last
    chunk reaches the last sample; valid counts are what is left."""
    for n in (1, 1000, 479999, 480000, 480001, 880000, 1_200_000, 2_700_000 + 123):
        for stride in (480000, 400000, 240000, 160160, 160):
            if stride < 160000 and n > 1_000_000:
                continue
            plan = O.chunk_plan(n, stride)
            owned = []
            for i, (start, valid, b, e) in enumerate(plan):
                assert start == i * stride and valid == min(480000, n - start) and valid > 0
                assert 0 <= b <= e <= 3000
                owned.extend(range(start // 160 + b, start // 160 + e))
            assert plan[-1][0] + plan[-1][1] == n
            assert owned == list(range(-(-n // 160))), (n, stride)


def test_chunked_log_mel_without_overlap_is_the_per_chunk_log_mel():
    """stride = 30 s: the chunks are the plain 30 s slices (the last one
    zero-padded), so each chunk equals log_mel of its slice."""
    rng = np.random.default_rng(9)
    audio = rng.standard_normal(480000 * 2 + 123_456) * 0.1
    got = O.log_mel_chunked(audio, 480000, 80)
    assert got.shape == (3, 80, 3000)
    for i in range(3):
        clip = np.zeros(480000)
        part = audio[i * 480000:(i + 1) * 480000]
        clip[:len(part)] = part
        assert np.array_equal(got[i], O.log_mel(clip, 80))


def test_overlapping_chunks_share_interior_frames_before_the_clamp():
    """With a stride of S samples (S / 160 frames), chunk i + 1's frame t
    sees exactly the samples of chunk i's frame t + S / 160 wherever neither
    window touches a chunk edge, so their unclamped log-mel columns agree."""
    rng = np.random.default_rng(10)
    stride = 400000
    audio = rng.standard_normal(880000) * 0.1
    plan = O.chunk_plan(len(audio), stride)
    assert len(plan) == 2
    c0 = audio[:480000]
    c1 = np.zeros(480000)
    c1[:plan[1][1]] = audio[stride:stride + plan[1][1]]
    u0 = O.log_mel_unnormalised(c0, 80)
    u1 = O.log_mel_unnormalised(c1, 80)
    sf = stride // 160
    ts = np.arange(2, 3000 - sf - 2)   # windows of 400 samples stay inside both chunks
    assert np.allclose(u0[:, ts + sf], u1[:, ts], rtol=0, atol=1e-9)
    # at the edges they do differ (reflection at a chunk's own start)
    assert not np.allclose(u0[:, sf], u1[:, 0], rtol=0, atol=1e-9)
