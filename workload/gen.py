"""Seeded random draws for every workload input.

Each tensor comes from its own torch.Generator, seeded from
(cfg_id, stream, extra...) through numpy's SeedSequence, so any tensor can be
drawn alone (the oracle only needs a few rows of the big ones). Draws are
made on the device given by the caller; a given seed gives the same numbers
on every device of the same type, and the oracle reads device draws through
a host copy.

Streams: 0 weights, 1 audio, 2 token ids, 3 prefill lengths, 4 prefill K/V,
5 encoder output, 6 hidden states.

Nothing here computes any step of the Whisper path; the only arithmetic is
shaping random numbers (scaling, bf16 storage rounding, sinusoid synthesis).
"""
import zlib

import numpy as np
import torch

from .configs import Dims


def _seed(cfg_id: int, stream: int, *extra: int) -> int:
    ss = np.random.SeedSequence([int(cfg_id), int(stream), *[int(e) for e in extra]])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


def rng_for(device, cfg_id: int, stream: int, *extra: int) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(_seed(cfg_id, stream, *extra))
    return g


def round_to_bf16(x: torch.Tensor) -> torch.Tensor:
    """Round fp32 values to the nearest bf16 (ties to even), kept as fp32."""
    return x.to(torch.bfloat16).to(torch.float32)


def gen_normal(device, shape, cfg_id, stream, *extra, std=1.0, bf16=False):
    g = rng_for(device, cfg_id, stream, *extra)
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x = x * std
    return round_to_bf16(x) if bf16 else x


# --------------------------------------------------------------------------- weights

ENC_LAYER_TENSORS = [
    ("attn_ln.weight", "d", "ln_w"), ("attn_ln.bias", "d", "ln_b"),
    ("attn.query.weight", "dd", "w"), ("attn.query.bias", "d", "w"),
    ("attn.key.weight", "dd", "w"),
    ("attn.value.weight", "dd", "w"), ("attn.value.bias", "d", "w"),
    ("attn.out.weight", "dd", "w"), ("attn.out.bias", "d", "w"),
    ("mlp_ln.weight", "d", "ln_w"), ("mlp_ln.bias", "d", "ln_b"),
    ("mlp.0.weight", "fd", "w"), ("mlp.0.bias", "f", "w"),
    ("mlp.2.weight", "df", "w"), ("mlp.2.bias", "d", "w"),
]

DEC_LAYER_TENSORS = [
    ("attn_ln.weight", "d", "ln_w"), ("attn_ln.bias", "d", "ln_b"),
    ("attn.query.weight", "dd", "w"), ("attn.query.bias", "d", "w"),
    ("attn.key.weight", "dd", "w"),
    ("attn.value.weight", "dd", "w"), ("attn.value.bias", "d", "w"),
    ("attn.out.weight", "dd", "w"), ("attn.out.bias", "d", "w"),
    ("cross_attn_ln.weight", "d", "ln_w"), ("cross_attn_ln.bias", "d", "ln_b"),
    ("cross_attn.query.weight", "dd", "w"), ("cross_attn.query.bias", "d", "w"),
    ("cross_attn.key.weight", "dd", "w"),
    ("cross_attn.value.weight", "dd", "w"), ("cross_attn.value.bias", "d", "w"),
    ("cross_attn.out.weight", "dd", "w"), ("cross_attn.out.bias", "d", "w"),
    ("mlp_ln.weight", "d", "ln_w"), ("mlp_ln.bias", "d", "ln_b"),
    ("mlp.0.weight", "fd", "w"), ("mlp.0.bias", "f", "w"),
    ("mlp.2.weight", "df", "w"), ("mlp.2.bias", "d", "w"),
]


def _shape(code: str, dims: Dims):
    m = {"d": dims.d_model, "f": dims.d_ffn}
    return tuple(m[c] for c in code)


def weight_specs(dims: Dims):
    """Canonical (name, shape, kind) list; same order as the C-ABI weight table."""
    d, nm = dims.d_model, dims.n_mels
    out = []
    if dims.n_enc_layers > 0:
        out += [("encoder.conv1.weight", (d, nm, 3), "w"), ("encoder.conv1.bias", (d,), "w"),
                ("encoder.conv2.weight", (d, d, 3), "w"), ("encoder.conv2.bias", (d,), "w")]
        for layer in range(dims.n_enc_layers):
            out += [(f"encoder.blocks.{layer}.{n}", _shape(s, dims), k) for n, s, k in ENC_LAYER_TENSORS]
        out += [("encoder.ln_post.weight", (d,), "ln_w"), ("encoder.ln_post.bias", (d,), "ln_b")]
    if dims.n_dec_layers > 0:
        out += [("decoder.token_embedding", (dims.n_vocab, d), "w"),
                ("decoder.positional_embedding", (dims.n_text_ctx, d), "w")]
        for layer in range(dims.n_dec_layers):
            out += [(f"decoder.blocks.{layer}.{n}", _shape(s, dims), k) for n, s, k in DEC_LAYER_TENSORS]
        out += [("decoder.ln.weight", (d,), "ln_w"), ("decoder.ln.bias", (d,), "ln_b")]
    return out


def gen_weight(device, dims: Dims, name: str, shape, kind: str, ln_random=False):
    """One weight tensor in PyTorch layout, fp32 (bf16-representable for bf16 configs).

    Linear/conv/embedding parameters and biases ~ N(0, 0.02); LayerNorm gamma=1,
    beta=0 unless ln_random (then gamma ~ 1+N(0,0.1), beta ~ N(0,0.1)).
    """
    bf16 = dims.act == "bf16"
    tag = zlib.crc32(name.encode())
    if kind == "w":
        return gen_normal(device, shape, dims.cfg_id, 0, tag, std=0.02, bf16=bf16)
    if not ln_random:
        fill = 1.0 if kind == "ln_w" else 0.0
        return torch.full(shape, fill, dtype=torch.float32, device=device)
    x = gen_normal(device, shape, dims.cfg_id, 0, tag, std=0.1)
    return x + 1.0 if kind == "ln_w" else x


def gen_weights(device, dims: Dims, ln_random=False):
    return {n: gen_weight(device, dims, n, s, k, ln_random) for n, s, k in weight_specs(dims)}


# --------------------------------------------------------------------------- audio

def _tones(t, freqs, amps, phases):
    x = torch.zeros_like(t)
    for f, a, p in zip(freqs, amps, phases):
        x += a * torch.sin(2.0 * np.pi * f * t + p)
    return x


def gen_audio_tones(device, cfg_id, batch, seconds=30.0, total=480000, sr=16000, n_tones=3,
                    noise=0.05):
    """[batch, total] fp32: `seconds` of 3 sinusoids (200-3000 Hz, amplitude 0.1-0.3,
    random phase) plus N(0, noise^2), then zeros up to `total` samples."""
    n = int(round(seconds * sr))
    out = torch.zeros(batch, total, dtype=torch.float32, device=device)
    t = torch.arange(n, dtype=torch.float64, device=device) / sr
    for b in range(batch):
        g = rng_for("cpu", cfg_id, 1, b)
        u = torch.rand(3 * n_tones, generator=g, dtype=torch.float64)
        freqs = 200.0 + 2800.0 * u[:n_tones]
        amps = 0.1 + 0.2 * u[n_tones:2 * n_tones]
        phases = 2 * np.pi * u[2 * n_tones:]
        gn = rng_for(device, cfg_id, 1, b, 1)
        x = _tones(t, freqs.tolist(), amps.tolist(), phases.tolist())
        x += noise * torch.randn(n, generator=gn, device=device, dtype=torch.float64)
        out[b, :n] = x.to(torch.float32)
    return out


def gen_audio_longform(device, cfg_id, minutes=45.0, sr=16000, chunk=480000):
    """Long-form audio split into 30 s chunks: [n_chunks, chunk] fp32.

    Piecewise segments of U[2,8] s; each is, with probability 1/2, 1-3 tones
    (200-3000 Hz, amplitude 0.1-0.3) plus N(0, 0.05^2), else pure noise with
    sigma ~ U[0.01, 0.1]."""
    total = int(round(minutes * 60 * sr))
    g = rng_for("cpu", cfg_id, 1)
    x = torch.empty(total, dtype=torch.float64, device=device)
    pos, seg = 0, 0
    while pos < total:
        u = torch.rand(12, generator=g, dtype=torch.float64).tolist()
        n = min(total - pos, int(round((2.0 + 6.0 * u[0]) * sr)))
        gn = rng_for(device, cfg_id, 1, 1000 + seg)
        noise = torch.randn(n, generator=gn, device=device, dtype=torch.float64)
        if u[1] < 0.5:
            k = 1 + int(u[2] * 3) if u[2] < 1.0 else 3
            t = torch.arange(pos, pos + n, dtype=torch.float64, device=device) / sr
            freqs = [200.0 + 2800.0 * u[3 + i] for i in range(k)]
            amps = [0.1 + 0.2 * u[6 + i] for i in range(k)]
            phases = [2 * np.pi * u[9 + i] for i in range(k)]
            x[pos:pos + n] = _tones(t, freqs, amps, phases) + 0.05 * noise
        else:
            x[pos:pos + n] = (0.01 + 0.09 * u[2]) * noise
        pos += n
        seg += 1
    n_chunks = (total + chunk - 1) // chunk
    out = torch.zeros(n_chunks * chunk, dtype=torch.float32, device=device)
    out[:total] = x.to(torch.float32)
    return out.view(n_chunks, chunk)


# --------------------------------------------------------------------------- decoder inputs

def gen_tokens(device, cfg_id, steps, batch, n_vocab):
    """Teacher-forced token ids [steps, batch] int32, uniform over [0, n_vocab)."""
    g = rng_for(device, cfg_id, 2)
    return torch.randint(0, n_vocab, (steps, batch), generator=g, device=device, dtype=torch.int32)


def gen_prefill_lengths(device, cfg_id, batch, max_len, low=1):
    """Prefilled cache lengths [batch] int32, uniform over {low..max_len}."""
    g = rng_for("cpu", cfg_id, 3) if low == 1 else rng_for("cpu", cfg_id, 3, low)
    return torch.randint(low, max_len + 1, (batch,), generator=g, dtype=torch.int32).to(device)


def gen_prefill_kv(device, cfg_id, layer, kv, batch, heads, n, head_dim=64):
    """Pre-quantisation prefill K (kv=0) or V (kv=1) of one decoder layer,
    [batch, heads, n, head_dim] fp32 ~ N(0,1)."""
    return gen_normal(device, (batch, heads, n, head_dim), cfg_id, 4, layer, kv)
