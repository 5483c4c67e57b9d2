"""GPU parity of the composed hot path against the oracle (teacher forcing),
through the C ABI: encoder layer, full encoder from audio, the tiny fp32
model end to end, and the batched large-v3 decoder step over an fp8 KV cache.

Batch rows and chunks are independent, so at the large shapes the oracle runs
on a few rows/chunks only and those rows must match."""
import numpy as np
import pytest
import torch

from oracle import whisper_oracle as O
from speech_recognition_amd import _lib as L
from speech_recognition_amd.runtime import DecodeState, Whisper, act_dtype
from tests.gpu_util import TOL, host, need_gpu, rel_err, say
from workload import (CONFIGS, gen_audio_tones, gen_normal, gen_prefill_kv, gen_prefill_lengths, gen_tokens,
                      gen_weights)

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def model_for(dims, ln_random=False, fp8_encoder=False):
    W = gen_weights(DEV, dims, ln_random=ln_random)
    m = Whisper(dims, list(W.values()), fp8_encoder=fp8_encoder)
    torch.cuda.synchronize()
    return m, W


def host_weights(W, prefix=None):
    return {k: v.double().cpu().numpy() for k, v in W.items() if prefix is None or k.startswith(prefix)}


# ------------------------------------------------------------------ encoder
@pytest.mark.parametrize("ln_post", [False, True])
def test_encoder_layer_large_v3(ln_post):
    dims = CONFIGS["v3_layer"]
    say(f"encoder layer large-v3 B=1 ln_post={ln_post}")
    m, W = model_for(dims, ln_random=True)
    h = gen_normal(DEV, (1, 1500, 1280), dims.cfg_id, 6, bf16=True).to(torch.bfloat16)
    out = m.encode_layers(h, 0, 1, ln_post=ln_post)
    out2 = m.encode_layers(h, 0, 1, ln_post=ln_post)
    torch.cuda.synchronize()
    assert torch.equal(out, out2), "encoder layer is not deterministic"
    Wh = host_weights(W)
    ref = O.encoder_layers(host(h)[0], Wh, dims.n_heads, [0], ln_post=ln_post)
    e = rel_err(host(out)[0], ref)
    say(f"  rel err {e:.3e}")
    assert e < TOL


def test_encoder_layer_mixed_fp8_large_v3_two_chunks():
    """One large-v3 encoder layer with the mixed_fp8 sites (query, key, value,
    fc1, fc2 in E4M3; per-tensor weight scales, per-chunk activation scales)
    through whisper_encode_layers_fp8, two chunks (the 1500-row chunks cross
    256-row tiles), against the oracle's mixed_fp8 layer on each chunk. The
    two sides quantise activations that differ by bf16 rounding, so some codes
    differ by one step; the tolerance is the fp8 one of the decode tests."""
    dims = CONFIGS["v3_layer"]
    say("mixed_fp8 encoder layer large-v3 B=2")
    m, W = model_for(dims, ln_random=True, fp8_encoder=True)
    h = gen_normal(DEV, (2, 1500, 1280), dims.cfg_id, 7, bf16=True).to(torch.bfloat16)
    out = m.encode_layers_fp8(h, 0, 1)
    out2 = m.encode_layers_fp8(h, 0, 1)
    bf = m.encode_layers(h, 0, 1)
    torch.cuda.synchronize()
    assert torch.equal(out, out2), "fp8 encoder layer is not deterministic"
    Wh = host_weights(W)
    for b in range(2):
        x = host(h)[b]
        ref = O.encoder_layers_mixed_fp8(x, Wh, dims.n_heads, [0], ln_post=False)
        e = rel_err(host(out)[b], ref)
        # the fp8 result differs from the bf16 layer by the fp8 rounding, not more
        e_bf = rel_err(host(out)[b], host(bf)[b])
        say(f"  chunk {b}: rel err vs oracle {e:.3e}, vs bf16 path {e_bf:.3e}")
        assert e < TOL
        assert e_bf < 0.1


def test_encoder_layer_mixed_fp8_full_batch_sampled_chunks():
    """The mixed_fp8 layer at the bench's batch of 64 chunks (the per-chunk
    amax and quantisation grids at full size, 96000-row fp8 GEMMs), the first
    and last chunk against the oracle's mixed_fp8 layer."""
    dims = CONFIGS["v3_layer"]
    say("mixed_fp8 encoder layer large-v3 B=64, chunks 0 and 63")
    m, W = model_for(dims, ln_random=True, fp8_encoder=True)
    h = gen_normal(DEV, (64, 1500, 1280), dims.cfg_id, 8, bf16=True).to(torch.bfloat16)
    out = m.encode_layers_fp8(h, 0, 1)
    torch.cuda.synchronize()
    Wh = host_weights(W)
    for b in (0, 63):
        ref = O.encoder_layers_mixed_fp8(host(h[b]), Wh, dims.n_heads, [0], ln_post=False)
        e = rel_err(host(out[b]), ref)
        say(f"  chunk {b}: rel err vs oracle {e:.3e}")
        assert e < TOL


def _encoder_from_audio(dims, B, chunks):
    m, W = model_for(dims)
    audio = gen_audio_tones(DEV, dims.cfg_id, B)
    mel = m.logmel(audio)
    enc = m.encode(mel)
    enc2 = m.encode(mel)
    torch.cuda.synchronize()
    same = [bool(torch.equal(enc[b], enc2[b])) for b in range(B)]
    assert all(same), f"encoder is not deterministic: chunks equal across two runs {same}"
    Wh = host_weights(W, "encoder.")
    for b in chunks:
        mref = O.log_mel(audio[b].cpu().numpy(), dims.n_mels)
        em = rel_err(host(mel)[b], mref)
        ref = O.encoder(mref, Wh, dims.n_heads, dims.n_enc_layers)
        e = rel_err(host(enc)[b], ref)
        say(f"  chunk {b}: mel rel err {em:.2e}, encoder rel err {e:.3e}")
        assert em < 1e-3 and e < TOL


def test_encoder_layers_deterministic_ragged_tiles():
    """Repeated two-layer encodes at batch 3 (4500 rows: the last 256-row GEMM
    tile is ragged, and one workgroup's epilogue stores overlap the next tile's
    loads) must agree bit for bit with the first."""
    dims = CONFIGS["v3_encoder"].with_(n_enc_layers=2)
    say("encoder layers 0..2, B=3: five repeated runs bit-identical")
    m, _ = model_for(dims)
    h = gen_normal(DEV, (3, 1500, 1280), dims.cfg_id, 6, bf16=True).to(torch.bfloat16)
    ref = m.encode_layers(h, 0, 2)
    for i in range(4):
        o = m.encode_layers(h, 0, 2)
        torch.cuda.synchronize()
        same = [bool(torch.equal(o[b], ref[b])) for b in range(3)]
        assert all(same), f"run {i + 1}: chunks equal to the first run {same}"


def test_encoder_from_audio_two_layers():
    dims = CONFIGS["v3_encoder"].with_(n_enc_layers=2)
    say("encoder large-v3 shape, 2 layers, B=3 from audio")
    _encoder_from_audio(dims, 3, [0, 2])


def test_encoder_full_large_v3_from_audio():
    dims = CONFIGS["v3_encoder"]
    say("full 32-layer large-v3 encoder, B=8 from audio; oracle on chunks 0 and 7")
    _encoder_from_audio(dims, 8, [0, 7])


# ------------------------------------------------------------------ decoder helpers
def code_mismatch_ok(g, o, pre):
    """End-to-end fp8 codes (teacher forced): a GPU code equal to the oracle's
    passes; a differing one must be the e4m3 rounding of some value within
    delta = TOL * max|y| of the oracle's pre-quantisation value y, i.e. within
    the same tolerance the activations are held to (max over the layer's K or
    V row). pre: [H, 64] oracle pre-quantisation values.
    Returns (ok, n_differing)."""
    g = np.asarray(g, np.int64)
    o = np.asarray(o, np.int64)
    diff = g != o
    if not diff.any():
        return True, 0
    y = pre.astype(np.float64)
    delta = TOL * np.abs(y).max()
    vlo = O.e4m3_value(O.e4m3_encode((y - delta).astype(np.float32)))
    vhi = O.e4m3_value(O.e4m3_encode((y + delta).astype(np.float32)))
    vg = O.e4m3_value(g)
    ok = (~diff) | ((vg >= vlo) & (vg <= vhi))
    return bool(ok.all()), int(diff.sum())


def codec_on_oracle_values_bit_exact(pre, codes_ref):
    """The GPU codec fed the oracle's own pre-quantisation values (scale 1)
    must reproduce the oracle's codes bit for bit."""
    y = torch.from_numpy(np.ascontiguousarray(pre, dtype=np.float32)).to(DEV)
    one = torch.ones(4, dtype=torch.float32, device=DEV)
    c = torch.empty(y.numel(), dtype=torch.uint8, device=DEV)
    L.whisper_fp8_quantize(y, L.WHISPER_F32, y.numel(), one, c, None)
    torch.cuda.synchronize()
    return np.array_equal(c.cpu().numpy(), np.asarray(codes_ref).reshape(-1))


def check_logits_argmax(lg_gpu, am_gpu, lg_ref, rows, tag):
    n_tied = 0
    for b in rows:
        e = rel_err(lg_gpu[b], lg_ref[b])
        assert e < TOL, f"{tag} row {b}: logits rel err {e:.3e}"
        top2 = np.sort(lg_ref[b])[-2:]
        bound = 2 * np.abs(lg_gpu[b] - lg_ref[b]).max()
        if top2[1] - top2[0] <= bound:
            n_tied += 1
            continue
        assert am_gpu[b] == int(np.argmax(lg_ref[b])), f"{tag} row {b}: argmax differs"
    return n_tied


def run_decode_case(dims, B, cap, prefill_max, steps, rows, tag, cross_fp8_scale=None, cross_fmt="e4m3"):
    """Teacher-forced decode on the GPU from a prefilled fp8 cache vs the oracle on `rows`.
    cross_fp8_scale: when given, the cross-attention K/V are fp8 codes in
    cross_fmt ("e4m3" or "e5m2") with that scale for every (layer, K|V), on
    both sides (the GPU quantises its bf16 projections, the oracle its own
    fp64 ones)."""
    H, d, Lyr, T = dims.n_heads, dims.d_model, dims.n_dec_layers, dims.n_audio_ctx
    m, W = model_for(dims, ln_random=True)
    dt = act_dtype(dims)
    enc = gen_normal(DEV, (B, T, d), dims.cfg_id, 5, bf16=dims.act == "bf16").to(dt)
    ckv = m.cross_kv(enc)
    lengths0 = gen_prefill_lengths(DEV, dims.cfg_id, B, prefill_max) if prefill_max else torch.zeros(
        B, dtype=torch.int32, device=DEV)
    scales = torch.ones(Lyr, 2, dtype=torch.float32)
    prefill = {}
    if prefill_max:
        for l in range(Lyr):
            for kv in range(2):
                x = gen_prefill_kv(DEV, dims.cfg_id, l, kv, B, H, prefill_max)
                scales[l, kv] = float(O.e4m3_scale_from_amax(np.array([x.abs().max().item()], np.float32)))
                prefill[(l, kv)] = x
    xscales = None
    if cross_fp8_scale is not None:
        xscales = np.full((Lyr, 2), np.float32(cross_fp8_scale), np.float32)
        fmt = {"e4m3": L.WHISPER_FP8_E4M3, "e5m2": L.WHISPER_FP8_E5M2}[cross_fmt]
        xcodes, xsc = m.quantize_cross_kv(ckv, scales=torch.from_numpy(xscales), fmt=fmt)
        state = DecodeState(dims, B, cap, None, scales, lengths0, cross_codes=xcodes, cross_scales=xsc,
                            cross_format=fmt)
        del ckv
    else:
        state = DecodeState(dims, B, cap, ckv, scales, lengths0)
    for (l, kv), x in prefill.items():
        codes = torch.empty(x.shape, dtype=torch.uint8, device=DEV)
        L.whisper_fp8_quantize(x, L.WHISPER_F32, x.numel(), state.kv_scales[l, kv:kv + 1].contiguous().clone(),
                               codes, None)
        state.kv_cache[l, kv, :, :, :prefill_max, :] = codes
    tokens = gen_tokens(DEV, dims.cfg_id, steps, B, dims.n_vocab)
    logits = torch.empty(B, dims.n_vocab, dtype=torch.float32, device=DEV)
    gpu_steps = []
    for t in range(steps):
        pos = state.lengths.clone()
        m.decode_step(state, tokens[t], logits)
        torch.cuda.synchronize()
        gpu_steps.append((host(logits), state.argmax.cpu().numpy().copy(), pos.cpu().numpy()))
    assert int(state.dev_error[0].item()) == 0
    assert np.array_equal(state.lengths.cpu().numpy(), lengths0.cpu().numpy() + steps)
    cache_gpu = state.kv_cache.cpu().numpy()

    # ---- oracle on the chosen rows
    Wh = host_weights(W, "decoder.")
    sc = scales.numpy()
    enc_h = {b: host(enc[b]) for b in rows}
    cross_rows = {b: O.cross_kv(enc_h[b], Wh, H, Lyr) for b in rows}
    cross = [({b: cross_rows[b][l][0] for b in rows}, {b: cross_rows[b][l][1] for b in rows}) for l in range(Lyr)]
    if xscales is not None:
        cross = O.cross_kv_fp8(cross, xscales, fmt=cross_fmt)
    cache = [[{b: np.zeros((H, cap, 64), np.uint8) for b in rows} for kv in range(2)] for l in range(Lyr)]
    lengths = lengths0.cpu().numpy().copy()
    for (l, kv), x in prefill.items():
        xh = x.cpu().numpy()
        for b in rows:
            cache[l][kv][b][:, :prefill_max, :] = O.e4m3_quantize(xh[b], sc[l, kv])
            n0 = int(lengths[b])  # later slots were overwritten by the decode steps
            assert np.array_equal(cache[l][kv][b][:, :n0], cache_gpu[l, kv, b, :, :n0]), \
                "prefill codes differ between the GPU codec and the oracle codec"
    tok = tokens.cpu().numpy()
    n_flips = n_codes = n_tied = 0
    for t in range(steps):
        # the oracle continues from the GPU's codes for the new slot; they are
        # checked against the oracle's own codes right after
        forced = [[{b: cache_gpu[l, kv, b, :, int(lengths[b]), :] for b in rows} for kv in range(2)]
                  for l in range(Lyr)]
        lg_ref, tr = O.decode_step(Wh, H, tok[t], lengths, cache, sc, cross, rows=rows, forced_codes=forced)
        lg_g, am_g, pos = gpu_steps[t]
        n_tied += check_logits_argmax(lg_g, am_g, lg_ref, rows, f"{tag} step {t}")
        for b in rows:
            for l in range(Lyr):
                for kv in range(2):
                    own = tr["codes"][l, kv, b]
                    ok, nf = code_mismatch_ok(forced[l][kv][b], own, tr["pre_quant"][l, kv, b])
                    assert ok, f"{tag} step {t} row {b} layer {l} kv {kv}: {nf} fp8 codes differ beyond the band"
                    assert codec_on_oracle_values_bit_exact(tr["pre_quant"][l, kv, b], own)
                    n_flips += nf
                    n_codes += H * 64
        lengths = lengths + 1
    say(f"  {tag}: code flips {n_flips}/{n_codes} ({100.0 * n_flips / max(n_codes, 1):.3f}%), "
        f"tied argmax rows excluded {n_tied}/{steps * len(rows)}")
    assert n_flips <= 0.25 * n_codes


def test_decode_large_v3_shape_4_layers():
    dims = CONFIGS["v3_decode"].with_(n_dec_layers=4)
    say("decode large-v3 shape, 4 layers, B=64, cap 672, prefill U[1,448], 3 steps")
    lengths0 = gen_prefill_lengths("cpu", dims.cfg_id, 64, 448).numpy()
    rows = sorted({int(np.argmin(lengths0)), int(np.argmax(lengths0)), 5, 33})
    run_decode_case(dims, 64, 672, 448, 3, rows, "v3x4")


def test_decode_large_v3_full():
    dims = CONFIGS["v3_decode"]
    say("decode large-v3, 32 layers, B=64, cap 672, prefill U[1,448], 2 steps")
    lengths0 = gen_prefill_lengths("cpu", dims.cfg_id, 64, 448).numpy()
    rows = sorted({int(np.argmin(lengths0)), int(np.argmax(lengths0))})
    run_decode_case(dims, 64, 672, 448, 2, rows, "v3x32")


def test_decode_turbo_shape_batch90_empty_cache():
    dims = CONFIGS["turbo_longform"]
    say("decode turbo shape, 4 layers, B=90, empty cache s=1, 3 steps")
    run_decode_case(dims, 90, 228, 0, 3, [0, 89], "turbo")


def test_decode_fp8_cross_kv_large_v3_shape():
    """fp8 e4m3 cross-attention K/V (one scale per layer and K|V) through
    whisper_decode_step_xq, against the oracle attending over its own K/V
    quantised with the same scale. The scale 5/448 covers the K/V range of
    these inputs (std ~0.7)."""
    dims = CONFIGS["v3_decode"].with_(n_dec_layers=4)
    say("decode large-v3 shape, 4 layers, B=64, fp8 cross K/V, cap 672, prefill U[1,448], 3 steps")
    lengths0 = gen_prefill_lengths("cpu", dims.cfg_id, 64, 448).numpy()
    rows = sorted({int(np.argmin(lengths0)), int(np.argmax(lengths0)), 5, 33})
    run_decode_case(dims, 64, 672, 448, 3, rows, "v3x4 fp8 cross", cross_fp8_scale=5.0 / 448.0)


def test_decode_fp8_e5m2_cross_kv_large_v3_shape():
    """The E5M2 form of the fp8 cross-attention K/V (the aggressive preset's
    format, chosen for range) with unit scales: E5M2 spans these K/V values
    without per-tensor scaling. Against the oracle attending over its own K/V
    quantised to E5M2 with the same scales."""
    dims = CONFIGS["v3_decode"].with_(n_dec_layers=4)
    say("decode large-v3 shape, 4 layers, B=64, E5M2 cross K/V scale 1, cap 672, prefill U[1,448], 3 steps")
    lengths0 = gen_prefill_lengths("cpu", dims.cfg_id, 64, 448).numpy()
    rows = sorted({int(np.argmin(lengths0)), int(np.argmax(lengths0)), 7, 40})
    run_decode_case(dims, 64, 672, 448, 3, rows, "v3x4 e5m2 cross", cross_fp8_scale=1.0, cross_fmt="e5m2")


# ------------------------------------------------------------------ tiny fp32 end to end
def test_tiny_fp32_end_to_end():
    dims = CONFIGS["tiny_f32"]
    say("tiny fp32: 10 s clip -> log-mel -> 4-layer encoder -> cross K/V -> 16 decode steps")
    m, W = model_for(dims)
    audio = gen_audio_tones(DEV, dims.cfg_id, 1, seconds=10.0)
    mel = m.logmel(audio)
    enc = m.encode(mel)
    ckv = m.cross_kv(enc)
    steps = 16
    state = DecodeState(dims, 1, 448, ckv, torch.ones(dims.n_dec_layers, 2), torch.zeros(1, dtype=torch.int32))
    tokens = gen_tokens(DEV, dims.cfg_id, steps, 1, dims.n_vocab)
    logits = torch.empty(1, dims.n_vocab, dtype=torch.float32, device=DEV)
    gl, ga = [], []
    for t in range(steps):
        m.decode_step(state, tokens[t], logits)
        torch.cuda.synchronize()
        gl.append(host(logits))
        ga.append(state.argmax.cpu().numpy().copy())
    cache_gpu = state.kv_cache.cpu().numpy()
    Wh = host_weights(W)
    mref = O.log_mel(audio[0].cpu().numpy(), dims.n_mels)
    assert rel_err(host(mel)[0], mref) < 1e-3
    eref = O.encoder(mref, Wh, dims.n_heads, dims.n_enc_layers)
    e = rel_err(host(enc)[0], eref)
    say(f"  encoder rel err {e:.2e}")
    assert e < TOL
    cr = O.cross_kv(eref, Wh, dims.n_heads, dims.n_dec_layers)
    cross = [({0: k}, {0: v}) for k, v in cr]
    cache = [[{0: np.zeros((dims.n_heads, 448, 64), np.uint8)} for _ in range(2)] for _ in range(dims.n_dec_layers)]
    sc = np.ones((dims.n_dec_layers, 2), np.float32)
    tok = tokens.cpu().numpy()
    flips = 0
    for t in range(steps):
        forced = [[{0: cache_gpu[l, kv, 0, :, t]} for kv in range(2)] for l in range(dims.n_dec_layers)]
        lg, tr = O.decode_step(Wh, dims.n_heads, tok[t], np.array([t]), cache, sc, cross, forced_codes=forced)
        check_logits_argmax(gl[t], ga[t], lg, [0], f"tiny step {t}")
        for l in range(dims.n_dec_layers):
            for kv in range(2):
                own = tr["codes"][l, kv, 0]
                ok, nf = code_mismatch_ok(cache_gpu[l, kv, 0, :, t], own, tr["pre_quant"][l, kv, 0])
                assert ok, (t, l, kv, nf)
                assert codec_on_oracle_values_bit_exact(tr["pre_quant"][l, kv, 0], own)
                flips += nf
    say(f"  tiny: code flips {flips}")


# ------------------------------------------------------------------ decode-state semantics
def test_decode_resume_and_capacity():
    dims = CONFIGS["v3_decode"].with_(n_dec_layers=2)
    say("decode resume through host copy, and capacity error, large-v3 shape 2 layers B=8")
    B, cap = 8, 64
    m, W = model_for(dims)
    enc = gen_normal(DEV, (B, 1500, 1280), dims.cfg_id, 5, bf16=True).to(torch.bfloat16)
    ckv = m.cross_kv(enc)
    tokens = gen_tokens(DEV, dims.cfg_id, 6, B, dims.n_vocab)
    sc = torch.full((2, 2), 0.01)
    s1 = DecodeState(dims, B, cap, ckv, sc, torch.arange(B, dtype=torch.int32))
    for t in range(6):
        m.decode_step(s1, tokens[t])
    s2 = DecodeState(dims, B, cap, ckv, sc, torch.arange(B, dtype=torch.int32))
    for t in range(3):
        m.decode_step(s2, tokens[t])
    torch.cuda.synchronize()
    saved = (s2.kv_cache.cpu(), s2.lengths.cpu())
    s2.kv_cache.fill_(0x55)
    s2.lengths.fill_(0)
    s2.kv_cache.copy_(saved[0].to(DEV))
    s2.lengths.copy_(saved[1].to(DEV))
    for t in range(3, 6):
        m.decode_step(s2, tokens[t])
    torch.cuda.synchronize()
    assert torch.equal(s1.kv_cache, s2.kv_cache) and torch.equal(s1.argmax, s2.argmax)
    assert torch.equal(s1.lengths, s2.lengths)
    # a row whose slot is past the cache: the device error word is set, its write skipped
    s3 = DecodeState(dims, B, cap, ckv, sc, torch.tensor([0, 1, 2, 3, 4, 5, 6, cap], dtype=torch.int32))
    m.decode_step(s3, tokens[0])
    torch.cuda.synchronize()
    assert int(s3.dev_error[0].item()) == 6
    assert int(s3.kv_cache[:, :, 7].sum().item()) == 0


def test_decode_prefill_equals_successive_steps_and_oracle():
    """A causal prefill of P prompt tokens per row in one pass equals P
    successive decode steps bit for bit (cache codes, lengths, logits and
    argmax of the last token), and so does the step after it; its logits
    match the oracle's P teacher-forced steps on two rows."""
    dims = CONFIGS["v3_decode"].with_(n_dec_layers=2)
    B, P, cap, prefill_max = 24, 4, 96, 40
    say(f"decode prefill: large-v3 shape 2 layers, B={B}, {P} prompt tokens, prefill U[1,{prefill_max}]")
    m, W = model_for(dims, ln_random=True)
    H, Lyr = dims.n_heads, dims.n_dec_layers
    enc = gen_normal(DEV, (B, 1500, 1280), dims.cfg_id, 8, bf16=True).to(torch.bfloat16)
    ckv = m.cross_kv(enc)
    lengths0 = gen_prefill_lengths(DEV, dims.cfg_id, B, prefill_max)
    sc = torch.full((Lyr, 2), 0.02)
    toks = gen_tokens(DEV, dims.cfg_id, P + 1, B, dims.n_vocab)   # [P + 1, B]
    prefill = torch.randint(0, 256, (Lyr, 2, B, H, cap, 64), dtype=torch.uint8,
                            generator=torch.Generator().manual_seed(12)).to(DEV)
    prefill[(prefill & 0x7F) == 0x7F] = 0
    s1 = DecodeState(dims, B, cap, ckv, sc, lengths0)
    s2 = DecodeState(dims, B, cap, ckv, sc, lengths0)
    s1.kv_cache.copy_(prefill)
    s2.kv_cache.copy_(prefill)
    lg1 = torch.empty(B, dims.n_vocab, dtype=torch.float32, device=DEV)
    lg2 = torch.empty_like(lg1)
    m.decode_prefill(s1, toks[:P].t().contiguous(), lg1)
    for t in range(P):
        m.decode_step(s2, toks[t], lg2)
    torch.cuda.synchronize()
    assert int(s1.dev_error[0].item()) == 0 and int(s2.dev_error[0].item()) == 0
    assert torch.equal(s1.lengths, lengths0.to(DEV) + P) and torch.equal(s1.lengths, s2.lengths)
    assert torch.equal(s1.kv_cache, s2.kv_cache), "cache codes differ"
    assert torch.equal(lg1, lg2) and torch.equal(s1.argmax, s2.argmax), "last-token logits differ"
    m.decode_step(s1, toks[P], lg1)
    m.decode_step(s2, toks[P], lg2)
    torch.cuda.synchronize()
    assert torch.equal(lg1, lg2) and torch.equal(s1.kv_cache, s2.kv_cache)
    # oracle: P teacher-forced steps on two rows, continuing from the GPU's checked codes
    rows = [0, B - 1]
    Wh = host_weights(W, "decoder.")
    cross_rows = {b: O.cross_kv(host(enc[b]), Wh, H, Lyr) for b in rows}
    cross = [({b: cross_rows[b][l][0] for b in rows}, {b: cross_rows[b][l][1] for b in rows}) for l in range(Lyr)]
    cache_gpu = s2.kv_cache.cpu().numpy()
    pre = prefill.cpu().numpy()
    cache = [[{b: pre[l, kv, b].copy() for b in rows} for kv in range(2)] for l in range(Lyr)]
    lengths = lengths0.cpu().numpy().copy()
    tok = toks.cpu().numpy()
    scn = sc.numpy()
    for t in range(P):
        forced = [[{b: cache_gpu[l, kv, b, :, int(lengths[b]), :] for b in rows} for kv in range(2)]
                  for l in range(Lyr)]
        lg_ref, tr = O.decode_step(Wh, H, tok[t], lengths, cache, scn, cross, rows=rows, forced_codes=forced)
        for b in rows:
            for l in range(Lyr):
                for kv in range(2):
                    ok, _ = code_mismatch_ok(forced[l][kv][b], tr["codes"][l, kv, b], tr["pre_quant"][l, kv, b])
                    assert ok
        lengths = lengths + 1
    # the prefill's logits are those of token P - 1 (s1 has moved on one step: compare s2's copy taken above)
    m2 = DecodeState(dims, B, cap, ckv, sc, lengths0)
    m2.kv_cache.copy_(prefill)
    m.decode_prefill(m2, toks[:P].t().contiguous(), lg1)
    torch.cuda.synchronize()
    check_logits_argmax(host(lg1), m2.argmax.cpu().numpy(), lg_ref, rows, "prefill")


@pytest.mark.parametrize("cross_fp8", [False, True])
def test_plan_batch_pass_fits_its_budget(cross_fp8):
    """A batch sized by whisper_plan_batch runs the whole pass (log-mel,
    encoder, cross K/V, [fp8 quantisation], 4-token prefill, one decode step)
    with torch's peak device allocation inside the plan's total; the plan for
    one more chunk exceeds the budget. Turbo shape, 6 GiB budget."""
    dims = CONFIGS["turbo_longform"]
    budget, cap, P = 6 << 30, 228, 4
    m, W = model_for(dims)
    del W
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    plan = m.plan_batch(budget, cap, P, cross_fp8=cross_fp8, want_logits=True)
    B = plan["batch"]
    say(f"plan_batch turbo, 6 GiB, fp8 cross {cross_fp8}: B={B}, peak stage {plan['peak_stage']}, "
        f"total {plan['total'] / 2**30:.2f} GiB")
    assert B >= 2
    assert m.plan_batch(1 << 62, cap, P, cross_fp8=cross_fp8, want_logits=True, max_batch=B + 1)["total"] > budget
    base = torch.cuda.memory_allocated()
    assert base - plan["weights"] < (1 << 20), "only the packed weights should be live"
    torch.cuda.reset_peak_memory_stats()
    m.reserve_workspace(plan["workspace"])
    audio = gen_audio_tones("cpu", dims.cfg_id, B).to(DEV)  # no device temporaries beside the pass
    mel = m.logmel(audio)
    del audio
    enc = m.encode(mel)
    del mel
    ckv = m.cross_kv(enc)
    del enc
    kv_scales = torch.full((dims.n_dec_layers, 2), 0.05, dtype=torch.float32)
    lengths = torch.zeros(B, dtype=torch.int32)
    if cross_fp8:
        xcodes, xsc = m.quantize_cross_kv(ckv, scales=torch.full((dims.n_dec_layers, 2), 0.01))
        del ckv
        state = DecodeState(dims, B, cap, None, kv_scales, lengths, cross_codes=xcodes, cross_scales=xsc)
    else:
        state = DecodeState(dims, B, cap, ckv, kv_scales, lengths)
        del ckv
    prompt = gen_tokens("cpu", dims.cfg_id, P, B, dims.n_vocab).t().contiguous().to(DEV)
    logits = torch.empty(B, dims.n_vocab, dtype=torch.float32, device=DEV)
    if cross_fp8:  # the prefill takes bf16 cross K/V; fp8 feeds the prompt step by step
        for t in range(P):
            m.decode_step(state, prompt[:, t].contiguous(), logits)
    else:
        m.decode_prefill(state, prompt)
    tok = state.argmax.clone()
    m.decode_step(state, tok, logits)
    torch.cuda.synchronize()
    assert int(state.dev_error[0].item()) == 0
    assert np.array_equal(state.lengths.cpu().numpy(), np.full(B, P + 1))
    am = state.argmax.cpu().numpy()
    assert am.min() >= 0 and am.max() < dims.n_vocab
    peak = torch.cuda.max_memory_allocated() - base
    need = plan["total"] - plan["weights"]
    say(f"  peak {peak / 2**30:.3f} GiB of planned {need / 2**30:.3f} GiB beyond the weights")
    assert peak <= need + (16 << 20)
    assert peak >= 0.9 * need
