"""whisper_decode_step_noalloc (no workspace, library-held scratch) against
whisper_decode_step on the same inputs: bit-identical logits, argmax, cache
codes and lengths, on two calls in a row, the second with a smaller batch."""
import numpy as np
import pytest
import torch

from speech_recognition_amd import _lib as L
from speech_recognition_amd.runtime import DecodeState, Whisper, act_dtype
from tests.gpu_util import need_gpu, say
from workload import CONFIGS, gen_normal, gen_prefill_lengths, gen_tokens, gen_weights

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _pair(m, dims, B, cap, seed):
    """Two identical decode states over the same cross K/V and a random
    prefilled cache."""
    enc = gen_normal(DEV, (B, dims.n_audio_ctx, dims.d_model), dims.cfg_id, 5, seed,
                     bf16=dims.act == "bf16").to(act_dtype(dims))
    ckv = m.cross_kv(enc)
    lengths0 = gen_prefill_lengths(DEV, dims.cfg_id, B, cap // 2)
    sc = torch.full((dims.n_dec_layers, 2), 0.02)
    pre = torch.randint(0, 256, (dims.n_dec_layers, 2, B, dims.n_heads, cap, 64), dtype=torch.uint8,
                        generator=torch.Generator().manual_seed(seed)).to(DEV)
    pre[(pre & 0x7F) == 0x7F] = 0
    a = DecodeState(dims, B, cap, ckv, sc, lengths0)
    b = DecodeState(dims, B, cap, ckv, sc, lengths0)
    a.kv_cache.copy_(pre)
    b.kv_cache.copy_(pre)
    return a, b, ckv


def _compare(m, dims, B, cap, seed, steps=2):
    a, b, ckv = _pair(m, dims, B, cap, seed)
    toks = gen_tokens(DEV, dims.cfg_id, steps, B, dims.n_vocab)
    la = torch.empty(B, dims.n_vocab, dtype=torch.float32, device=DEV)
    lb = torch.full_like(la, float("nan"))
    for t in range(steps):
        m.decode_step(a, toks[t], la)
        L.whisper_decode_step_noalloc(dims, m.packed, B, cap, toks[t], b.lengths, b.kv_cache, b.kv_scales, ckv, lb,
                                      b.argmax, b.dev_error)
        torch.cuda.synchronize()
        assert torch.equal(la, lb), f"B={B} step {t}: logits differ"
        assert torch.equal(a.argmax, b.argmax) and torch.equal(a.lengths, b.lengths)
        assert torch.equal(a.kv_cache, b.kv_cache), f"B={B} step {t}: cache codes differ"
    assert int(b.dev_error[0].item()) == 0
    say(f"  B={B}: {steps} steps bit-identical to whisper_decode_step")


@pytest.mark.parametrize("name,layers,batches,cap", [
    ("v3_decode", 4, (64, 24), 96),   # bf16 fused step, split-K counters in the scratch
    ("tiny_f32", 4, (3, 1), 32),      # fp32 step
])
def test_decode_step_noalloc_matches_decode_step(name, layers, batches, cap):
    dims = CONFIGS[name].with_(n_dec_layers=layers, n_enc_layers=0)
    say(f"decode_step_noalloc vs decode_step: {name}, {layers} layers, batches {batches}")
    W = gen_weights(DEV, dims, ln_random=True)
    m = Whisper(dims, list(W.values()))
    for i, B in enumerate(batches):  # the second call reuses the scratch at a smaller batch
        _compare(m, dims, B, cap, 40 + i)


def test_decode_step_noalloc_rejects_oversized_batch():
    dims = CONFIGS["v3_decode"].with_(n_dec_layers=2)
    with pytest.raises(L.WhisperError) as e:
        L.whisper_decode_step_noalloc(dims, 16, 200, 672, 16, 16, 16, 16, 16, 16, 16, None)
    assert e.value.status == 5 and "scratch" in str(e.value)
