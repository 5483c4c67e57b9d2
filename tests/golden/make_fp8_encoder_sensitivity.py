"""Writes fp8_encoder_sensitivity.json: how far the oracle's own mixed_fp8
large-v3 encoder moves when the inputs of its fp8 sites are rounded to
bfloat16 first (act_transform=bf16_round), after 1, 4, 8, 16 and 32 layers,
and how far the whole fp8 encoder is from the plain one. Calls only the
oracle and the seeded input generators (weights and audio generated on the
CPU; chunk 0 of the tone audio, the oracle's own log-mel).

    python tests/golden/make_fp8_encoder_sensitivity.py   (about 10 minutes)
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import whisper_oracle as O  # noqa: E402
from workload import CONFIGS, gen_audio_tones, gen_weights  # noqa: E402


def rel(u, v):
    return float(np.abs(u - v).max() / np.abs(v).max())


def main():
    dims = CONFIGS["v3_encoder"]
    W = {k: v.double().numpy() for k, v in gen_weights("cpu", dims).items() if k.startswith("encoder.")}
    mel = O.log_mel(gen_audio_tones("cpu", dims.cfg_id, 1)[0].numpy(), dims.n_mels)
    x = O.conv_stem(mel, W)
    a, b, c = x, x, x
    out = {"config": "large-v3 encoder (d 1280, 20 heads), weights gen_weights('cpu'), chunk 0 of "
                     "gen_audio_tones('cpu', batch 1), oracle log-mel and conv stem",
           "measure": "max |y - y_ref| / max |y_ref| over the layer output (final LayerNorm after 32 layers)",
           "sensitivity": {}}
    for layer in range(dims.n_enc_layers):
        a = O.encoder_layer_mixed_fp8(a, W, layer, dims.n_heads)
        b = O.encoder_layer_mixed_fp8(b, W, layer, dims.n_heads, act_transform=O.bf16_round)
        c = O.encoder_layer(c, W, layer, dims.n_heads)
        n = layer + 1
        if n in (1, 4, 8, 16):
            out["sensitivity"][str(n)] = rel(b, a)
            print(n, out["sensitivity"][str(n)], flush=True)
    g, bt = W["encoder.ln_post.weight"], W["encoder.ln_post.bias"]
    ya, yb, yc = O.layer_norm(a, g, bt), O.layer_norm(b, g, bt), O.layer_norm(c, g, bt)
    out["sensitivity"]["32"] = rel(yb, ya)
    out["fp8_vs_plain_32"] = rel(ya, yc)
    print(out, flush=True)
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "fp8_encoder_sensitivity.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
