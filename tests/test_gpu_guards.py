"""Guards around caller buffers.

Each call runs twice on the same inputs: once with a zeroed workspace and once
with the workspace filled with 0xFF bytes (a NaN as fp32 and bf16, -1 as an
integer), so a kernel that reads workspace memory it did not write first shows
up as a difference. Every buffer the call writes sits inside canary bytes: the
workspace has PAD bytes past the exact size the library asked for, and the
logits and the KV cache are views into larger buffers. The outputs must be
bit-identical between the two runs and every canary must survive."""
import numpy as np
import pytest
import torch

from speech_recognition_amd import _lib as L
from speech_recognition_amd.runtime import Whisper
from tests.gpu_util import need_gpu, say
from workload import CONFIGS, gen_normal, gen_prefill_lengths, gen_tokens, gen_weights

pytestmark = pytest.mark.gpu
DEV = "cuda"
PAD = 4096


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def workspace(nbytes, byte):
    whole = torch.full((nbytes + PAD,), byte, dtype=torch.uint8, device=DEV)
    return whole, whole[:nbytes]


def inside(n, dtype, fill):
    whole = torch.full((n + 2 * PAD,), fill, dtype=dtype, device=DEV)
    return whole, whole[PAD:PAD + n]


def intact(whole, fill, lead=True):
    tail = bool(torch.all(whole[-PAD:] == fill))
    return tail and (bool(torch.all(whole[:PAD] == fill)) if lead else True)


@pytest.fixture(scope="module")
def decoder():
    dims = CONFIGS["v3_decode"].with_(n_dec_layers=2)
    W = gen_weights(DEV, dims)
    m = Whisper(dims, list(W.values()), mixed_fp8=True)
    del W
    return dims, m


@pytest.mark.parametrize("kind", ["step", "step_enc", "prefill_enc", "step_xq", "step_enc_fp8", "prefill_enc_fp8"])
def test_decode_poisoned_workspace_and_canaries(decoder, kind):
    dims, m = decoder
    B, cap, P = 37, 64, 3
    H, V, Ly = dims.n_heads, dims.n_vocab, dims.n_dec_layers
    enc = gen_normal(DEV, (B, dims.n_audio_ctx, dims.d_model), dims.cfg_id, 5, 3, bf16=True).to(torch.bfloat16)
    ckv = m.cross_kv(enc) if kind in ("step", "step_xq") else None
    xq = m.quantize_cross_kv(ckv) if kind == "step_xq" else None
    lengths0 = gen_prefill_lengths(DEV, dims.cfg_id, B, cap // 2)
    pre = torch.randint(0, 256, (Ly, 2, B, H, cap, 64), dtype=torch.uint8,
                        generator=torch.Generator().manual_seed(7)).to(DEV)
    pre[(pre & 0x7F) == 0x7F] = 0  # no NaN codes in the prefilled slots
    sc = torch.full((Ly, 2), 0.02, device=DEV)
    toks = gen_tokens(DEV, dims.cfg_id, P, B, V)
    rows = B * P if kind in ("prefill_enc", "prefill_enc_fp8") else B
    which = {"step_enc": L.WS_DECODE_ENC, "prefill_enc": L.WS_DECODE_ENC,
             "step_enc_fp8": L.WS_DECODE_ENC_FP8, "prefill_enc_fp8": L.WS_DECODE_ENC_FP8}.get(kind, L.WS_DECODE)
    nbytes = L.whisper_workspace_size(dims, rows, which)

    def run(byte):
        ws_whole, ws = workspace(nbytes, byte)
        lg_whole, lg = inside(B * V, torch.float32, 777.0)
        kv_whole, kv = inside(pre.numel(), torch.uint8, 0xA5)
        kv.copy_(pre.view(-1))
        kv = kv.view(pre.shape)
        lengths = lengths0.clone()
        am = torch.full((B,), -5, dtype=torch.int32, device=DEV)
        err = torch.zeros(4, dtype=torch.int32, device=DEV)
        outs = []
        if kind == "prefill_enc":
            L.whisper_decode_prefill_enc(dims, m.packed, B, P, cap, toks.t().contiguous(), lengths, kv, sc, enc, lg,
                                         am, err, ws, nbytes)
            outs.append((lg.clone(), am.clone()))
        elif kind == "prefill_enc_fp8":
            L.whisper_decode_prefill_enc_fp8(dims, m.packed, m.packed8, B, P, cap, toks.t().contiguous(), lengths, kv,
                                             sc, enc, lg, am, err, ws, nbytes)
            outs.append((lg.clone(), am.clone()))
        else:
            for t in range(2):
                if kind == "step":
                    L.whisper_decode_step(dims, m.packed, B, cap, toks[t], lengths, kv, sc, ckv, lg, am, err, ws, nbytes)
                elif kind == "step_enc":
                    L.whisper_decode_step_enc(dims, m.packed, B, cap, toks[t], lengths, kv, sc, enc, lg, am, err, ws,
                                              nbytes)
                elif kind == "step_enc_fp8":
                    L.whisper_decode_step_enc_fp8(dims, m.packed, m.packed8, B, cap, toks[t], lengths, kv, sc, enc,
                                                  lg, am, err, ws, nbytes)
                else:
                    L.whisper_decode_step_xq(dims, m.packed, B, cap, toks[t], lengths, kv, sc, xq[0], xq[1], lg, am,
                                             err, ws, nbytes)
                outs.append((lg.clone(), am.clone()))
        torch.cuda.synchronize()
        assert int(err[0].item()) == 0
        assert intact(ws_whole, byte, lead=False), f"{kind}: write past the workspace's {nbytes} bytes"
        assert intact(lg_whole, 777.0), f"{kind}: write outside the logits"
        assert intact(kv_whole, 0xA5), f"{kind}: write outside the KV cache"
        return outs, kv.clone(), lengths.clone()

    outs0, kv0, len0 = run(0x00)
    outs1, kv1, len1 = run(0xFF)
    for i, ((lg0, am0), (lg1, am1)) in enumerate(zip(outs0, outs1)):
        assert torch.isfinite(lg0).all()
        assert torch.equal(lg0, lg1), f"{kind} call {i}: logits depend on the workspace's prior contents"
        assert torch.equal(am0, am1)
    assert torch.equal(kv0, kv1) and torch.equal(len0, len1)
    say(f"  {kind}: B={B}, workspace {nbytes} B zeroed vs 0xFF bit-identical; canaries intact")


def test_encode_layers_poisoned_workspace_and_canaries():
    dims = CONFIGS["v3_encoder"].with_(n_enc_layers=2)
    W = gen_weights(DEV, dims)
    m = Whisper(dims, list(W.values()))
    del W
    B = 3
    h = gen_normal(DEV, (B, 1500, 1280), dims.cfg_id, 6, bf16=True).to(torch.bfloat16)
    nbytes = L.whisper_workspace_size(dims, B, L.WS_ENCODE)
    res = []
    for byte in (0x00, 0xFF):
        ws_whole, ws = workspace(nbytes, byte)
        o_whole, o = inside(h.numel(), torch.bfloat16, 3.0)
        L.whisper_encode_layers(dims, m.packed, h, B, 0, 2, True, o, ws, nbytes)
        torch.cuda.synchronize()
        assert intact(ws_whole, byte, lead=False), "write past the encoder workspace"
        assert intact(o_whole, 3.0), "write outside the encoder output"
        res.append(o.clone())
    assert torch.isfinite(res[0].float()).all()
    assert torch.equal(res[0], res[1]), "encoder output depends on the workspace's prior contents"
    say(f"  encode_layers B={B}: workspace {nbytes} B zeroed vs 0xFF bit-identical; canaries intact")
