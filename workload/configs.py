"""Model shapes of the five synthetic workloads.

large-v3 facts used here: 128 mel bins and 30 s chunks of 16 kHz audio
(whisper_blaze showcase page, mel_spectrogram.cu card); the remaining
widths are the public Whisper large-v3 / tiny / large-v3-turbo shapes.
"""
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Dims:
    name: str
    n_mels: int
    d_model: int
    n_heads: int
    d_ffn: int
    n_enc_layers: int
    n_dec_layers: int
    n_vocab: int
    n_text_ctx: int          # rows of the learned decoder position table
    act: str                 # "bf16" or "f32": storage type of activations/weights on the GPU
    n_audio_ctx: int = 1500  # encoder frames per 30 s chunk
    head_dim: int = 64
    n_samples: int = 480000  # 30 s at 16 kHz
    n_frames: int = 3000     # STFT frames per chunk (hop 160)
    cfg_id: int = 0          # seed namespace

    def with_(self, **kw):
        return replace(self, **kw)


LARGE_V3 = dict(n_mels=128, d_model=1280, n_heads=20, d_ffn=5120, n_vocab=51866)

CONFIGS = {
    # whisper-tiny shape, fp32 end to end, 4+4 layers
    "tiny_f32": Dims("tiny_f32", n_mels=80, d_model=384, n_heads=6, d_ffn=1536,
                     n_enc_layers=4, n_dec_layers=4, n_vocab=51865, n_text_ctx=448,
                     act="f32", cfg_id=1),
    # one large-v3 encoder layer, bf16, batch 1, hidden states ~N(0,1)
    "v3_layer": Dims("v3_layer", **LARGE_V3, n_enc_layers=1, n_dec_layers=0,
                     n_text_ctx=448, act="bf16", cfg_id=2),
    # full 32-layer large-v3 encoder from 8 chunks of audio
    "v3_encoder": Dims("v3_encoder", **LARGE_V3, n_enc_layers=32, n_dec_layers=0,
                       n_text_ctx=448, act="bf16", cfg_id=3),
    # batched large-v3 decoder step over an fp8 self-KV cache; 448 prefill + 224 steps
    "v3_decode": Dims("v3_decode", **LARGE_V3, n_enc_layers=0, n_dec_layers=32,
                      n_text_ctx=672, act="bf16", cfg_id=4),
    # large-v3-turbo shape: 32 encoder + 4 decoder layers, 45 min long-form
    "turbo_longform": Dims("turbo_longform", **LARGE_V3, n_enc_layers=32, n_dec_layers=4,
                           n_text_ctx=448, act="bf16", cfg_id=5),
}

# Batch / step counts of each workload
RUN = {
    "tiny_f32": dict(batch=1, clip_s=10.0, steps=16),
    "v3_layer": dict(batch=1),
    "v3_encoder": dict(batch=8),
    "v3_decode": dict(batch=64, steps=224, prefill_max=448, cap=672),
    "turbo_longform": dict(batch=90, minutes=45, prompt=4, steps=224, cap=228),
}


def get_config(name: str) -> Dims:
    return CONFIGS[name]
