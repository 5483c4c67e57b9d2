"""CPU oracle of the Whisper large-v3 inference hot path.

TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and
the CPU-baseline leg of the benchmark may import or run anything in this
directory; the GPU library never does, and this module imports nothing from
the GPU library.

Plain NumPy in float64 (floating point) with a library primitive per step
(matmul, rfft, erf), no blocking or fusion. It follows the pages:

* whisper_blaze showcase page, "The Solution": mel_spectrogram.cu card (STFT,
  128-bin mel filterbank, log-mel front end on the GPU), layernorm_fused.cu
  card (residual add + LayerNorm in one pass), flash_attn_hopper.cu card
  (encoder self, decoder causal self and decoder cross attention, online
  softmax, no score matrix in memory), fp8_quantize.cu card (E4M3, and
  E5M2 for range, with a per-tensor scale from the activation maximum).
* whisper-blaze project page, "Direct Kernel API": quantise_e4m3 returns codes
  plus a per-tensor scale; dequantise_e4m3 takes codes, scale and shape;
  layernorm_fused_residual returns (normed, total).
* whisper_blaze showcase page, "Learnings": the largest E4M3 magnitude is
  448, and the scales follow the activations' maxima.
* "Blazingly fast whisper transcriptions with Inference Endpoints", section
  "Inference Stack": activations computed in bfloat16, KV cache stored as
  float8 (one byte per element), quantised dynamically on the way in.

Where the pages are silent (STFT parameters, mel scale, log floor, layer
structure, attention scale, GELU form, fp8 rounding) the oracle takes the
public Whisper model definition and the OCP E4M3FN / E5M2 format
definitions; each
reading is stated at the function that uses it.
"""
import numpy as np
from scipy.special import erf

# =========================================================================== fp8 e4m3
# OCP 8-bit float E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits, no
# infinities, S.1111.111 is NaN, largest finite magnitude 1.75 * 2^8 = 448
# (the bound the whisper_blaze showcase page's "Learnings" gives for E4M3).

E4M3_MAX = 448.0


def e4m3_value(code):
    """Real value of each e4m3 code (NaN for 0x7F / 0xFF)."""
    c = np.asarray(code, dtype=np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = (1.0 + m / 8.0) * np.exp2(e - 7.0)
    sub = (m / 8.0) * 2.0 ** -6
    v = s * np.where(e == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, v)


# The 127 non-negative finite values, ascending; index == code.
_E4M3_POS = e4m3_value(np.arange(127))


def e4m3_encode(y):
    """Code of the e4m3 value nearest to each fp32 input.

    Ties go to the code with an even mantissa (round to nearest even);
    magnitudes above 448 saturate to +-448 rather than become NaN; NaN maps
    to the NaN code; the sign bit of the input is kept (so -0 -> 0x80).
    """
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y.astype(np.float64))
    neg = np.signbit(y)
    nan = np.isnan(y)
    a_ = np.where(nan, 0.0, a)
    i = np.clip(np.searchsorted(_E4M3_POS, a_, side="right") - 1, 0, 126)
    j = np.minimum(i + 1, 126)
    lo, hi = _E4M3_POS[i], _E4M3_POS[j]
    d_lo, d_hi = a_ - lo, hi - a_
    up = (d_hi < d_lo) | ((d_hi == d_lo) & (j % 2 == 0) & (j != i))
    code = np.where(up, j, i)
    code = np.where(a_ >= E4M3_MAX, 126, code)
    code = np.where(nan, 127, code)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


def e4m3_quantize(x, scale):
    """Quantise-on-write: code = e4m3(fl32(fl32(x) * fl32(1 / scale))).

    One fp32 reciprocal of the scale, one fp32 multiply, then a single
    rounding to e4m3. The input is first rounded to fp32 (the accumulator
    precision the values are produced in)."""
    inv = np.float32(1.0) / np.float32(scale)
    y = np.asarray(x, dtype=np.float64).astype(np.float32) * inv
    return e4m3_encode(y)


def e4m3_pre_quant(x, scale):
    """The fp32 value that e4m3_quantize rounds (for near-tie analysis)."""
    inv = np.float32(1.0) / np.float32(scale)
    return np.asarray(x, dtype=np.float64).astype(np.float32) * inv


def e4m3_dequantize(codes, scale):
    """Dequantise-on-read: fl32(value(code) * scale)."""
    v = e4m3_value(codes).astype(np.float32)
    return (v * np.float32(scale)).astype(np.float64)


def e4m3_scale_from_amax(x):
    """Per-tensor scale from the activation maximum: fl32(amax) / 448 in fp32
    (1.0 for an all-zero tensor), so the largest magnitude maps to 448."""
    amax = np.float32(np.max(np.abs(np.asarray(x, dtype=np.float64)))) if np.size(x) else np.float32(0)
    if amax == 0:
        return np.float32(1.0)
    return np.float32(amax) / np.float32(E4M3_MAX)


# =========================================================================== fp8 e5m2
# OCP 8-bit float E5M2: 1 sign, 5 exponent (bias 15), 2 mantissa bits. It is
# laid out like IEEE binary16 cut to its top byte: exponent 31 holds +-inf
# (mantissa 0) and NaN (mantissa != 0); largest finite magnitude
# 1.75 * 2^15 = 57344; subnormal step 2^-16. The pages offer it beside E4M3
# for its wider range (whisper_blaze showcase page: fp8_quantize.cu card and
# the aggressive_fp8 preset of the precision.py card).

E5M2_MAX = 57344.0


def e5m2_value(code):
    """Real value of each e5m2 code (+-inf for 0x7C / 0xFC, NaN for
    0x7D..0x7F and 0xFD..0xFF)."""
    c = np.asarray(code, dtype=np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 2) & 0x1F
    m = c & 0x3
    normal = (1.0 + m / 4.0) * np.exp2(e - 15.0)
    sub = (m / 4.0) * 2.0 ** -14
    v = s * np.where(e == 0, sub, normal)
    return np.where(e == 31, np.where(m == 0, s * np.inf, np.nan), v)


# The 124 non-negative finite values, ascending; index == code (0x7B = 57344).
_E5M2_POS = e5m2_value(np.arange(124))


def e5m2_encode(y):
    """Code of the e5m2 value nearest to each fp32 input.

    Ties go to the code with an even mantissa (round to nearest even);
    magnitudes above 57344, infinities included, saturate to +-57344 (the
    saturating conversion, as the e4m3 encoder does at 448, so no finite input
    becomes inf); NaN maps to the NaN code 0x7F with the input's sign; the sign
    bit of the input is kept (so -0 -> 0x80)."""
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y.astype(np.float64))
    neg = np.signbit(y)
    nan = np.isnan(y)
    a_ = np.where(nan, 0.0, a)
    i = np.clip(np.searchsorted(_E5M2_POS, a_, side="right") - 1, 0, 123)
    j = np.minimum(i + 1, 123)
    lo, hi = _E5M2_POS[i], _E5M2_POS[j]
    d_lo, d_hi = a_ - lo, hi - a_
    up = (d_hi < d_lo) | ((d_hi == d_lo) & (j % 2 == 0) & (j != i))
    code = np.where(up, j, i)
    code = np.where(a_ >= E5M2_MAX, 123, code)
    code = np.where(nan, 127, code)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


def e5m2_quantize(x, scale):
    """code = e5m2(fl32(fl32(x) * fl32(1 / scale))), as e4m3_quantize."""
    inv = np.float32(1.0) / np.float32(scale)
    y = np.asarray(x, dtype=np.float64).astype(np.float32) * inv
    return e5m2_encode(y)


def e5m2_dequantize(codes, scale):
    """Dequantise-on-read: fl32(value(code) * scale)."""
    v = e5m2_value(codes).astype(np.float32)
    return (v * np.float32(scale)).astype(np.float64)


def e5m2_scale_from_amax(x):
    """fl32(amax) / 57344 in fp32 (1.0 for an all-zero tensor)."""
    amax = np.float32(np.max(np.abs(np.asarray(x, dtype=np.float64)))) if np.size(x) else np.float32(0)
    if amax == 0:
        return np.float32(1.0)
    return np.float32(amax) / np.float32(E5M2_MAX)


FP8_FORMATS = {
    "e4m3": (e4m3_quantize, e4m3_dequantize, e4m3_scale_from_amax),
    "e5m2": (e5m2_quantize, e5m2_dequantize, e5m2_scale_from_amax),
}


# =========================================================================== log-mel
# Reading of the pages' "STFT -> 128-bin mel filterbank" (mel_spectrogram.cu
# card): 16 kHz audio, 30 s chunks of 480000 samples, 400-point frames with a
# periodic Hann window, hop 160 (3000 frames per chunk), centre framing with
# reflect padding of 200 samples, last frame dropped; power spectrum over
# 201 bins; Slaney mel filterbank 0-8 kHz with area normalisation; log10
# with a 1e-10 floor; values clamped to (chunk maximum - 8); then (x+4)/4.

SAMPLE_RATE = 16000
N_FFT = 400
HOP = 160
N_SAMPLES = 480000
N_FRAMES = 3000


def hann_periodic(n=N_FFT):
    k = np.arange(n)
    return 0.5 - 0.5 * np.cos(2.0 * np.pi * k / n)


def hz_to_mel(f):
    """Slaney mel scale: linear (3 mel per 200 Hz) below 1 kHz, logarithmic
    above with 27 mel per factor 6.4."""
    f = np.asarray(f, dtype=np.float64)
    f_sp = 200.0 / 3.0
    min_log_hz, min_log_mel = 1000.0, 1000.0 / f_sp
    logstep = np.log(6.4) / 27.0
    safe = np.maximum(f, min_log_hz)
    return np.where(f >= min_log_hz, min_log_mel + np.log(safe / min_log_hz) / logstep, f / f_sp)


def mel_to_hz(m):
    m = np.asarray(m, dtype=np.float64)
    f_sp = 200.0 / 3.0
    min_log_hz, min_log_mel = 1000.0, 1000.0 / f_sp
    logstep = np.log(6.4) / 27.0
    return np.where(m >= min_log_mel, min_log_hz * np.exp(logstep * (m - min_log_mel)), f_sp * m)


def mel_filterbank(n_mels, sr=SAMPLE_RATE, n_fft=N_FFT, fmin=0.0, fmax=None):
    """[n_mels, n_fft/2+1] triangular filters with corners equally spaced on
    the Slaney mel scale, each scaled by 2/(upper corner - lower corner) so its
    area in Hz is one."""
    fmax = sr / 2.0 if fmax is None else fmax
    freqs = np.arange(n_fft // 2 + 1) * sr / n_fft
    pts = mel_to_hz(np.linspace(hz_to_mel(fmin), hz_to_mel(fmax), n_mels + 2))
    fb = np.zeros((n_mels, n_fft // 2 + 1))
    for m in range(n_mels):
        lo, c, hi = pts[m], pts[m + 1], pts[m + 2]
        rising = (freqs - lo) / (c - lo)
        falling = (hi - freqs) / (hi - c)
        fb[m] = np.maximum(0.0, np.minimum(rising, falling)) * (2.0 / (hi - lo))
    return fb


def frames(audio):
    """[3000, 400] windowless frames of one chunk (zero-padded to 480000 samples,
    then reflect-padded by 200 on each side)."""
    x = np.zeros(N_SAMPLES)
    a = np.asarray(audio, dtype=np.float64)[:N_SAMPLES]
    x[:a.size] = a
    xp = np.pad(x, N_FFT // 2, mode="reflect")
    idx = HOP * np.arange(N_FRAMES)[:, None] + np.arange(N_FFT)[None, :]
    return xp[idx]


def power_spectrum(audio):
    """[3000, 201] squared magnitude of the DFT of each Hann-windowed frame."""
    spec = np.fft.rfft(frames(audio) * hann_periodic(), axis=1)
    return np.abs(spec) ** 2


def log_mel_unnormalised(audio, n_mels):
    """[n_mels, 3000] log10(max(mel power, 1e-10)) before the range clamp."""
    mel = power_spectrum(audio) @ mel_filterbank(n_mels).T
    return np.log10(np.maximum(mel, 1e-10)).T


def log_mel(audio, n_mels):
    """[n_mels, 3000] Whisper log-mel features of one 30 s chunk."""
    lg = log_mel_unnormalised(audio, n_mels)
    lg = np.maximum(lg, lg.max() - 8.0)
    return (lg + 4.0) / 4.0


def chunk_plan(n_samples, stride, window=480000, hop=160, n_frames=3000):
    """Overlapping 30 s chunks of one long recording (showcase page,
    mel_spectrogram.cu card: overlapping-chunk support for long audio).
    Reading: chunk i covers samples [i*stride, i*stride + window), zero past
    the end of the recording; the chunk count is the smallest that reaches
    the last sample. Each shared span of (window - stride) / hop frames is
    split at its midpoint (the earlier chunk keeps its first floor(span / 2)
    frames, the later one the rest), so every frame of the recording belongs
    to one chunk; the last chunk's owned frames end at its last frame centred
    on real audio. Returns a list of (first sample, valid samples,
    first owned frame, end of owned frames), frames chunk-local."""
    assert n_samples > 0 and 0 < stride <= window and stride % hop == 0
    n = 1 if n_samples <= window else 1 + -(-(n_samples - window) // stride)
    overlap = n_frames - stride // hop
    plan = []
    for i in range(n):
        start = i * stride
        valid = min(window, n_samples - start)
        begin = 0 if i == 0 else overlap // 2
        end = min(n_frames, -(-valid // hop)) if i == n - 1 else n_frames - (overlap - overlap // 2)
        plan.append((start, valid, begin, end))
    return plan


def log_mel_chunked(audio, stride, n_mels, window=480000):
    """[n_chunks, n_mels, 3000] log-mel of the overlapping chunks of one
    recording: each chunk sliced, zero-padded to 30 s and processed as a
    standalone clip (its own max - 8 clamp)."""
    audio = np.asarray(audio, dtype=np.float64)
    out = []
    for start, valid, _, _ in chunk_plan(len(audio), stride, window):
        chunk = np.zeros(window)
        chunk[:valid] = audio[start:start + valid]
        out.append(log_mel(chunk, n_mels))
    return np.stack(out)


# =========================================================================== layers

def gelu(x):
    """Exact GELU x * Phi(x) with the Gaussian CDF (erf form)."""
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def linear(x, w, b=None):
    """x @ w.T + b with w in PyTorch [out, in] layout."""
    y = x @ w.T
    return y if b is None else y + b


def layer_norm(x, gamma, beta, eps=1e-5):
    """LayerNorm over the last axis: biased variance, eps inside the root."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * gamma + beta


def residual_layer_norm(h, residual, gamma, beta, eps=1e-5):
    """Fused residual + LayerNorm of the pages' layernorm_fused_residual:
    total = h + residual (or h alone), normed = LayerNorm(total); returns
    (normed, total)."""
    total = h if residual is None else h + residual
    return layer_norm(total, gamma, beta, eps), total


def conv1d(x, w, b, stride=1, pad=1):
    """Cross-correlation of x [C_in, T] with w [C_out, C_in, k], zero padding."""
    c_out, _, k = w.shape
    xp = np.pad(x, ((0, 0), (pad, pad)))
    t_out = (x.shape[1] + 2 * pad - k) // stride + 1
    y = np.repeat(b[:, None], t_out, axis=1).astype(np.float64)
    for j in range(k):
        y += w[:, :, j] @ xp[:, j: j + stride * (t_out - 1) + 1: stride]
    return y


def sinusoids(length, channels, max_timescale=10000.0):
    """Fixed encoder positions: first half sin, second half cos, timescales
    geometric from 1 to max_timescale over channels/2 steps."""
    inc = np.log(max_timescale) / (channels // 2 - 1)
    inv = np.exp(-inc * np.arange(channels // 2))
    st = np.arange(length)[:, None] * inv[None, :]
    return np.concatenate([np.sin(st), np.cos(st)], axis=1)


def softmax(s, axis=-1):
    z = s - s.max(axis=axis, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=axis, keepdims=True)


def attention(q, k, v, n_heads):
    """Multi-head attention without mask: per head softmax(q k^T / sqrt(dh)) v.
    q [Tq, d], k and v [Tk, d]; heads are contiguous slices of d."""
    d = q.shape[-1]
    dh = d // n_heads
    out = np.empty((q.shape[0], d))
    for h in range(n_heads):
        sl = slice(h * dh, (h + 1) * dh)
        p = softmax(q[:, sl] @ k[:, sl].T / np.sqrt(dh))
        out[:, sl] = p @ v[:, sl]
    return out


# =========================================================================== encoder

def conv_stem(mel, W):
    """mel [n_mels, 3000] -> [1500, d]: GELU(conv k3 s1 p1), GELU(conv k3 s2 p1),
    transpose, plus the sinusoidal positions."""
    x = gelu(conv1d(mel, W["encoder.conv1.weight"], W["encoder.conv1.bias"], 1, 1))
    x = gelu(conv1d(x, W["encoder.conv2.weight"], W["encoder.conv2.bias"], 2, 1))
    x = x.T
    return x + sinusoids(x.shape[0], x.shape[1])


def encoder_layer(x, W, layer, n_heads):
    """Pre-LN encoder block: x += out(attn(LN1 x)); x += fc2(GELU(fc1(LN2 x))).
    Query and value projections have biases, the key projection has none."""
    p = f"encoder.blocks.{layer}."
    a = layer_norm(x, W[p + "attn_ln.weight"], W[p + "attn_ln.bias"])
    q = linear(a, W[p + "attn.query.weight"], W[p + "attn.query.bias"])
    k = linear(a, W[p + "attn.key.weight"])
    v = linear(a, W[p + "attn.value.weight"], W[p + "attn.value.bias"])
    x = x + linear(attention(q, k, v, n_heads), W[p + "attn.out.weight"], W[p + "attn.out.bias"])
    m = layer_norm(x, W[p + "mlp_ln.weight"], W[p + "mlp_ln.bias"])
    hdn = gelu(linear(m, W[p + "mlp.0.weight"], W[p + "mlp.0.bias"]))
    return x + linear(hdn, W[p + "mlp.2.weight"], W[p + "mlp.2.bias"])


def encoder_layers(x, W, n_heads, layers, ln_post=True):
    for layer in layers:
        x = encoder_layer(x, W, layer, n_heads)
    if ln_post:
        x = layer_norm(x, W["encoder.ln_post.weight"], W["encoder.ln_post.bias"])
    return x


def encoder(mel, W, n_heads, n_layers):
    """One chunk: mel [n_mels, 3000] -> encoder output [1500, d]."""
    return encoder_layers(conv_stem(mel, W), W, n_heads, range(n_layers), ln_post=True)


# =========================================================================== mixed_fp8 encoder
# Reading of the whisper_blaze showcase page's precision.py card (the
# mixed_fp8 preset's table of layer sites): the encoder FFN (both matmuls)
# and the encoder attention's query/key/value projections take fp8 E4M3
# weights and activations; the attention itself, its output projection and
# the conv stem keep the activation precision. Scales, after the
# fp8_quantize.cu card and "Learnings" (per-tensor scales from maxima):
# one per weight tensor (query, key, value, fc1, fc2: fl32(amax) / 448), and
# one per activation tensor at each site, taken over one chunk's activation
# (one 30 s clip, so a chunk's result does not depend on the batch it runs
# in): fl32(amax) / 448, of the oracle's own activation values. The product
# sums value(code_x) * value(code_w) and multiplies by both scales; the bias
# is added after.

def fp8_linear(x, w, b, sx, sw):
    """y = sx * sw * (value(e4m3(x / sx)) @ value(e4m3(w / sw))^T) + b."""
    cx = e4m3_quantize(x, sx)
    cw = e4m3_quantize(w, sw)
    y = (e4m3_value(cx) @ e4m3_value(cw).T) * (float(np.float32(sx)) * float(np.float32(sw)))
    return y if b is None else y + b


def bf16_round(x):
    """x rounded to bfloat16 (through fp32, round to nearest even), as float64."""
    u = np.asarray(x, dtype=np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    return r.view(np.float32).astype(np.float64)


def _site(x, w, b, fp8, act_transform=None):
    """One mixed_fp8 matmul site: fp8 with amax scales of exactly the site's
    input and weight, or the plain linear. The oracle quantises its own
    activation values (no intermediate rounding). act_transform, when given,
    is applied to the activation before its scale and codes are taken:
    bf16_round there gives the activation as an inference stack that computes
    in bfloat16 holds it (Endpoints post, "Inference Stack"), which is how the
    oracle's sensitivity to that rounding is measured."""
    if not fp8:
        return linear(x, w, b)
    xq = x if act_transform is None else act_transform(x)
    return fp8_linear(xq, w, b, e4m3_scale_from_amax(xq), e4m3_scale_from_amax(w))


def encoder_layer_mixed_fp8(x, W, layer, n_heads, fp8=True, act_transform=None):
    """encoder_layer with the mixed_fp8 sites (query, key, value, fc1, fc2)
    in fp8 E4M3 for one chunk x [1500, d]; with fp8=False it is
    encoder_layer. act_transform: see _site."""
    p = f"encoder.blocks.{layer}."
    a = layer_norm(x, W[p + "attn_ln.weight"], W[p + "attn_ln.bias"])
    q = _site(a, W[p + "attn.query.weight"], W[p + "attn.query.bias"], fp8, act_transform)
    k = _site(a, W[p + "attn.key.weight"], None, fp8, act_transform)
    v = _site(a, W[p + "attn.value.weight"], W[p + "attn.value.bias"], fp8, act_transform)
    x = x + linear(attention(q, k, v, n_heads), W[p + "attn.out.weight"], W[p + "attn.out.bias"])
    m = layer_norm(x, W[p + "mlp_ln.weight"], W[p + "mlp_ln.bias"])
    hdn = gelu(_site(m, W[p + "mlp.0.weight"], W[p + "mlp.0.bias"], fp8, act_transform))
    return x + _site(hdn, W[p + "mlp.2.weight"], W[p + "mlp.2.bias"], fp8, act_transform)


def encoder_layers_mixed_fp8(x, W, n_heads, layers, ln_post=True, fp8=True, act_transform=None):
    for layer in layers:
        x = encoder_layer_mixed_fp8(x, W, layer, n_heads, fp8, act_transform)
    if ln_post:
        x = layer_norm(x, W["encoder.ln_post.weight"], W["encoder.ln_post.bias"])
    return x


def encoder_mixed_fp8(mel, W, n_heads, n_layers, act_transform=None):
    """One chunk with the mixed_fp8 sites: mel [n_mels, 3000] -> [1500, d]
    (the conv stem keeps the activation precision)."""
    return encoder_layers_mixed_fp8(conv_stem(mel, W), W, n_heads, range(n_layers), ln_post=True,
                                    act_transform=act_transform)


def cross_kv(enc, W, n_heads, n_layers):
    """Per decoder layer the cross-attention keys and values of one chunk's
    encoder output enc [T, d]: K = enc Wk^T, V = enc Wv^T + bv, each returned
    head-major [H, T, dh]. Returns a list of (K, V)."""
    t, d = enc.shape
    dh = d // n_heads
    out = []
    for layer in range(n_layers):
        p = f"decoder.blocks.{layer}.cross_attn."
        k = linear(enc, W[p + "key.weight"]).reshape(t, n_heads, dh).transpose(1, 0, 2)
        v = linear(enc, W[p + "value.weight"], W[p + "value.bias"]).reshape(t, n_heads, dh).transpose(1, 0, 2)
        out.append((k, v))
    return out


def cross_kv_fp8(cross, scales, fmt="e4m3", kv_transform=None):
    """fp8 cross-attention keys and values: each layer's K and V are
    quantised on write with the caller's per-(layer, K|V) scale and read back
    dequantised, so decode_step then attends over the fp8 values (whisper_blaze
    showcase page, precision.py card and its preset table: the aggressive
    preset puts the cross-attention site in fp8, there in E5M2 for range;
    fp8_quantize.cu card: E4M3 and E5M2 codes with a per-tensor scale).
    fmt picks the format, "e4m3" or "e5m2", with one scale per (layer, K|V)
    tensor either way. The oracle quantises its own K and V values;
    kv_transform, when given, is applied to them first (bf16_round: the
    tensors as a bfloat16 inference stack holds them, for measuring the
    oracle's sensitivity to that rounding).

    cross: list over layers of (K, V), each an array [B, H, T, dh] or a dict
    b -> [H, T, dh]; scales: [L, 2]. Returns the same structure holding
    dequantize(quantize(x, s), s) in the chosen format."""
    quant, dequant, _ = FP8_FORMATS[fmt]
    tr = (lambda a: a) if kv_transform is None else kv_transform

    def q(x, s):
        if isinstance(x, dict):
            return {b: dequant(quant(tr(v), s), s) for b, v in x.items()}
        return dequant(quant(tr(x), s), s)
    return [(q(k, scales[layer][0]), q(v, scales[layer][1])) for layer, (k, v) in enumerate(cross)]


# =========================================================================== decoder step

_WEIGHT_CODES = {}


def _quantised_weight(w):
    """(scale, dequantised codes) of a weight with its per-tensor scale. The
    result is kept per weight array (keyed by identity, checked by a weak
    reference and the array's sum) since a decoder step quantises the same
    weights at every step; it is the same computation each time."""
    import weakref
    key = id(w)
    fp = float(np.sum(w))
    hit = _WEIGHT_CODES.get(key)
    if hit is not None and hit[0]() is w and hit[1] == fp and hit[2] == w.shape:
        return hit[3], hit[4]
    sw = e4m3_scale_from_amax(w)
    wv = e4m3_value(e4m3_quantize(w, sw))
    for k in [k for k, v in _WEIGHT_CODES.items() if v[0]() is None]:  # arrays gone since
        del _WEIGHT_CODES[k]
    try:
        ref = weakref.ref(w)
    except TypeError:  # an array that takes no weak reference is not kept
        return sw, wv
    _WEIGHT_CODES[key] = (ref, fp, w.shape, sw, wv)
    return sw, wv


def fp8_linear_rows(x, w, b, rows=None, act_transform=None):
    """A mixed_fp8 site with one activation scale per row of x: row r is
    fp8_linear(x[r], w, b, fl32(amax(x[r])) / 448, fl32(amax(w)) / 448)
    (per-tensor weight scale). Rows outside `rows` are left zero.
    act_transform: as at the encoder sites (see _site)."""
    n = x.shape[0]
    out = np.zeros((n, w.shape[0]))
    sw, wv = _quantised_weight(w)
    for r in (range(n) if rows is None else rows):
        xr = x[r] if act_transform is None else act_transform(x[r])
        sx = e4m3_scale_from_amax(xr)
        out[r] = (e4m3_value(e4m3_quantize(xr, sx)) @ wv.T) * (float(np.float32(sx)) * float(np.float32(sw)))
        if b is not None:
            out[r] += b
    return out


def decode_step(W, n_heads, tokens, lengths, cache, scales, cross, rows=None, kv_transform=None, mixed_fp8=False,
                act_transform=None):
    """One batched decoder step with teacher-forced tokens.

    tokens, lengths: [B] ints; lengths[b] is both the cache slot the new
        token's K/V go to and its position index.
    cache: indexable as cache[layer][kv][b] -> [H, cap, dh] (an array
        [L, 2, B, H, cap, dh] or nested containers holding only the rows
        used); uint8 e4m3 codes when scales is given (updated in place at
        slot lengths[b] with this step's own codes), or float values when
        scales is None (exact cache, used to pin the step against a full
        causal pass).
    scales: [L, 2] fp32 per-layer K and V scales, or None.
    cross: list over layers of (K_c, V_c), each indexable as K_c[b] -> [H, T, dh].
    rows: optional list of batch rows to compute (others are skipped);
        rows are independent, so a subset gives exactly those rows' results.
    kv_transform: optional function applied to the new token's K and V before
        the codec (sensitivity analysis: how far the step moves when the
        quantised values change by a rounding, e.g. bf16_round). None: off.
    mixed_fp8: the decoder MLP's two matmuls as mixed_fp8 sites (the
        showcase page's precision.py card: decoder FFN in fp8 E4M3, weights
        and activations): fp8_linear_rows, a per-tensor weight scale and one
        activation scale per row (one token of one chunk). act_transform
        applies to those sites' inputs (sensitivity runs).

    The new token's K and V are written first and then read back from the
    cache with the rest (quantise-on-write, dequantise-on-read).
    Returns (logits [B, V] float64, trace dict: "kv" the new token's K and V
    before quantisation [L, 2, B, H, dh] float64, "codes" the codes written
    for them [L, 2, B, H, dh] uint8, "x" the last residual stream).
    """
    n_layers = len(cross)
    bsz = len(tokens)
    rows = list(range(bsz)) if rows is None else list(rows)
    d = W["decoder.token_embedding"].shape[1]
    dh = d // n_heads
    x = np.zeros((bsz, d))
    for b in rows:
        x[b] = W["decoder.token_embedding"][tokens[b]] + W["decoder.positional_embedding"][lengths[b]]
    kv_new = np.zeros((n_layers, 2, bsz, n_heads, dh))
    codes = np.zeros((n_layers, 2, bsz, n_heads, dh), dtype=np.uint8)
    for layer in range(n_layers):
        p = f"decoder.blocks.{layer}."
        a = layer_norm(x, W[p + "attn_ln.weight"], W[p + "attn_ln.bias"])
        q = linear(a, W[p + "attn.query.weight"], W[p + "attn.query.bias"])
        k = linear(a, W[p + "attn.key.weight"])
        v = linear(a, W[p + "attn.value.weight"], W[p + "attn.value.bias"])
        o = np.zeros((bsz, d))
        for b in rows:
            pos = int(lengths[b])
            for kv, val in ((0, k), (1, v)):
                vb = val[b].reshape(n_heads, dh)
                slot = cache[layer][kv][b]
                kv_new[layer, kv, b] = vb
                if scales is None:
                    slot[:, pos, :] = vb
                else:
                    xq = vb if kv_transform is None else kv_transform(vb)
                    codes[layer, kv, b] = e4m3_quantize(xq, scales[layer][kv])
                    slot[:, pos, :] = codes[layer, kv, b]
            for h in range(n_heads):
                kc_ = cache[layer][0][b][h, :pos + 1, :]
                vc_ = cache[layer][1][b][h, :pos + 1, :]
                if scales is None:
                    kh, vh = kc_.astype(np.float64), vc_.astype(np.float64)
                else:
                    kh = e4m3_dequantize(kc_, scales[layer][0])
                    vh = e4m3_dequantize(vc_, scales[layer][1])
                qh = q[b, h * dh:(h + 1) * dh]
                o[b, h * dh:(h + 1) * dh] = softmax(kh @ qh / np.sqrt(dh)) @ vh
        x = x + linear(o, W[p + "attn.out.weight"], W[p + "attn.out.bias"])
        c = layer_norm(x, W[p + "cross_attn_ln.weight"], W[p + "cross_attn_ln.bias"])
        qc = linear(c, W[p + "cross_attn.query.weight"], W[p + "cross_attn.query.bias"])
        kc, vc = cross[layer]
        oc = np.zeros((bsz, d))
        for b in rows:
            for h in range(n_heads):
                qh = qc[b, h * dh:(h + 1) * dh]
                oc[b, h * dh:(h + 1) * dh] = softmax(kc[b][h] @ qh / np.sqrt(dh)) @ vc[b][h]
        x = x + linear(oc, W[p + "cross_attn.out.weight"], W[p + "cross_attn.out.bias"])
        m = layer_norm(x, W[p + "mlp_ln.weight"], W[p + "mlp_ln.bias"])
        if mixed_fp8:
            hdn = gelu(fp8_linear_rows(m, W[p + "mlp.0.weight"], W[p + "mlp.0.bias"], rows, act_transform))
            x = x + fp8_linear_rows(hdn, W[p + "mlp.2.weight"], W[p + "mlp.2.bias"], rows, act_transform)
        else:
            x = x + linear(gelu(linear(m, W[p + "mlp.0.weight"], W[p + "mlp.0.bias"])),
                           W[p + "mlp.2.weight"], W[p + "mlp.2.bias"])
    y = layer_norm(x, W["decoder.ln.weight"], W["decoder.ln.bias"])
    logits = y @ W["decoder.token_embedding"].T
    return logits, {"kv": kv_new, "codes": codes, "x": x}


def decode_prefill(W, n_heads, tokens, lengths, cache, scales, cross, rows=None, kv_transform=None, mixed_fp8=False,
                   act_transform=None):
    """P prompt tokens per row fed causally: token p of row b goes to slot and
    position lengths[b] + p and attends over slots 0 .. lengths[b] + p, which is
    P successive teacher-forced steps (the decoder's causal self-attention
    with several queries, flash_attn_hopper.cu card of the whisper_blaze
    showcase page). tokens: [B, P]. Returns (logits of each row's last
    token, list of the P steps' traces)."""
    tokens = np.asarray(tokens)
    lengths = np.asarray(lengths).copy()
    traces = []
    logits = None
    for p in range(tokens.shape[1]):
        logits, tr = decode_step(W, n_heads, tokens[:, p], lengths, cache, scales, cross, rows=rows,
                                 kv_transform=kv_transform, mixed_fp8=mixed_fp8, act_transform=act_transform)
        traces.append(tr)
        lengths = lengths + 1
    return logits, traces


def greedy_token(logits):
    """Argmax over the vocabulary, lowest index on ties."""
    return np.argmax(logits, axis=-1)


def top2_gap(logits):
    """Per row, the largest logit minus the second largest (0 on a tie)."""
    s = np.sort(np.asarray(logits, dtype=np.float64), axis=-1)
    return s[..., -1] - s[..., -2]
