"""GPU parity of the individual kernels against the oracle, through the C ABI."""
import numpy as np
import pytest
import torch

from oracle import whisper_oracle as O
from speech_recognition_amd import _lib as L
from tests.gpu_util import TOL, bf16_bits, host, need_gpu, rel_err, say
from workload import CONFIGS, gen_normal

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


# ------------------------------------------------------------------ fp8 codec
FMTS = {"e4m3": L.WHISPER_FP8_E4M3, "e5m2": L.WHISPER_FP8_E5M2}


@pytest.mark.parametrize("fmt", list(FMTS))
def test_fp8_quantize_all_bf16_patterns_bit_exact(fmt):
    say(f"fp8 quantize {fmt}: all 65536 bf16 bit patterns, scale 1")
    quant = O.FP8_FORMATS[fmt][0]
    bits = torch.arange(-32768, 32768, dtype=torch.int32).to(torch.int16)
    x = bits.view(torch.bfloat16).to(DEV)
    scale = torch.ones(4, dtype=torch.float32, device=DEV)
    codes = torch.empty(65536, dtype=torch.uint8, device=DEV)
    L.whisper_fp8_quantize(x, L.WHISPER_BF16, 65536, scale, codes, None, fmt=FMTS[fmt])
    torch.cuda.synchronize()
    ref = quant(x.float().cpu().numpy(), 1.0)
    assert np.array_equal(codes.cpu().numpy(), ref)


@pytest.mark.parametrize("fmt", list(FMTS))
def test_fp8_quantize_fp32_scaled_bit_exact_and_amax_scale(fmt):
    say(f"fp8 quantize {fmt}: 1M fp32 values, device amax scale")
    quant, _, amax_scale = O.FP8_FORMATS[fmt]
    g = torch.Generator().manual_seed(3)
    x = (torch.randn(1 << 20, generator=g) * 3.7).to(DEV)
    codes = torch.empty(1 << 20, dtype=torch.uint8, device=DEV)
    scale = torch.zeros(4, dtype=torch.float32, device=DEV)
    ws = torch.empty(L.whisper_fp8_workspace_size(), dtype=torch.uint8, device=DEV)
    L.whisper_fp8_quantize(x, L.WHISPER_F32, x.numel(), None, codes, scale, ws, ws.numel(), fmt=FMTS[fmt])
    torch.cuda.synchronize()
    xs = x.cpu().numpy()
    s_ref = amax_scale(xs)
    assert scale[0].item() == float(s_ref)
    assert np.array_equal(codes.cpu().numpy(), quant(xs, s_ref))
    # a scale that is not a power of two and saturates part of the range
    s_fix = 0.0123 if fmt == "e4m3" else 0.0123 / 128
    s2 = torch.full((4,), s_fix, dtype=torch.float32, device=DEV)
    L.whisper_fp8_quantize(x, L.WHISPER_F32, x.numel(), s2, codes, None, fmt=FMTS[fmt])
    torch.cuda.synchronize()
    got = codes.cpu().numpy()
    assert np.array_equal(got, quant(xs, np.float32(s_fix)))
    top = 0x7E if fmt == "e4m3" else 0x7B
    assert np.count_nonzero((got & 0x7F) == top) > 0, "the fixed scale should saturate part of the range"


@pytest.mark.parametrize("fmt", list(FMTS))
def test_fp8_dequantize_all_codes(fmt):
    say(f"fp8 dequantize {fmt}: all 256 codes")
    dequant = O.FP8_FORMATS[fmt][1]
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).to(DEV)
    for s in (1.0, 0.0123):
        scale = torch.full((4,), s, dtype=torch.float32, device=DEV)
        y = torch.empty(256, dtype=torch.float32, device=DEV)
        L.whisper_fp8_dequantize(codes, 256, scale, y, L.WHISPER_F32, fmt=FMTS[fmt])
        torch.cuda.synchronize()
        ref = dequant(np.arange(256), np.float32(s)).astype(np.float32)
        got = y.cpu().numpy()
        assert np.array_equal(np.isnan(got), np.isnan(ref))
        ok = ~np.isnan(ref)
        assert np.array_equal(got[ok].view(np.uint32), ref[ok].view(np.uint32))


# ------------------------------------------------------------------ LayerNorm
@pytest.mark.parametrize("act,d,M", [("bf16", 1280, 1500), ("bf16", 1280, 37), ("f32", 384, 300)])
def test_layernorm_fused(act, d, M):
    say(f"layernorm act={act} d={d} M={M}")
    dims = CONFIGS["v3_layer"].with_(act=act, d_model=d, n_heads=d // 64)
    bf = act == "bf16"
    dt = torch.bfloat16 if bf else torch.float32
    h = gen_normal(DEV, (M, d), 9, 6, 1, bf16=bf).to(dt)
    r = gen_normal(DEV, (M, d), 9, 6, 2, std=2.0)          # fp32 residual stream
    gam = gen_normal(DEV, (d,), 9, 6, 3, std=0.5) + 1
    bet = gen_normal(DEV, (d,), 9, 6, 4, std=0.5)
    normed = torch.empty_like(h)
    total = torch.empty(M, d, dtype=torch.float32, device=DEV)
    L.whisper_layernorm_fused(dims, h, r, gam, bet, 1e-5, M, normed, total)
    normed0 = torch.empty_like(h)
    total0 = torch.empty(M, d, dtype=torch.float32, device=DEV)
    L.whisper_layernorm_fused(dims, h, None, gam, bet, 1e-5, M, normed0, total0)
    # in place on the residual stream, as the encoder and decoder use it
    r2 = r.clone()
    normed2 = torch.empty_like(h)
    L.whisper_layernorm_fused(dims, h, r2, gam, bet, 1e-5, M, normed2, r2)
    torch.cuda.synchronize()
    # total is the single fp32 rounding of h + r, bit for bit
    ref_total = (h.float().cpu() + r.cpu()).numpy()
    assert np.array_equal(total.cpu().numpy(), ref_total)
    assert np.array_equal(r2.cpu().numpy(), ref_total) and torch.equal(normed2, normed)
    assert np.array_equal(total0.cpu().numpy(), h.float().cpu().numpy())
    n_ref, _ = O.residual_layer_norm(host(h), host(r), host(gam), host(bet))
    for i in range(0, M, max(1, M // 7)):
        assert rel_err(host(normed)[i], n_ref[i]) < TOL
    assert rel_err(host(normed), n_ref) < TOL
    n0_ref = O.layer_norm(host(h), host(gam), host(bet))
    assert rel_err(host(normed0), n0_ref) < TOL


# ------------------------------------------------------------------ GEMM
@pytest.mark.parametrize("act,M,N,K,gelu,path", [
    ("bf16", 300, 200, 256, 0, 1), ("bf16", 300, 384, 1280, 1, 1), ("bf16", 129, 128, 64, 0, 1),
    ("bf16", 300, 200, 256, 0, 3), ("bf16", 530, 264, 320, 1, 4), ("bf16", 530, 264, 320, 1, 5),
    ("bf16", 1500, 1280, 1280, 0, 5), ("bf16", 3000, 640, 384, 1, 5),
    ("bf16", 530, 264, 320, 1, 6), ("bf16", 1500, 1280, 1280, 0, 6), ("bf16", 3000, 640, 384, 1, 6),
    ("bf16", 257, 2056, 64, 0, 6), ("bf16", 700, 520, 192, 1, 6),
    ("bf16", 1500, 1280, 1280, 0, 8), ("bf16", 3000, 640, 384, 1, 8),
    ("bf16", 700, 520, 256, 1, 8), ("bf16", 1024, 2560, 256, 0, 8),
    # persistent kernel: ragged M, more tiles than compute units (workgroups cross tile
    # boundaries), the smallest K it takes (8 k-steps), GELU, a grid with empty XCD ranges,
    # and a shape it does not take (falls back)
    ("bf16", 1500, 1280, 1280, 0, 9), ("bf16", 4100, 5120, 384, 1, 9), ("bf16", 4096, 4608, 256, 0, 9),
    ("bf16", 300, 256, 256, 1, 9), ("bf16", 3000, 1280, 5120, 0, 9), ("bf16", 700, 520, 256, 1, 9),
    ("bf16", 64, 1280, 1280, 0, 2), ("bf16", 90, 200, 5120, 1, 2), ("bf16", 1, 51, 128, 0, 2),
    ("f32", 77, 130, 240, 1, 1)])
def test_linear(act, M, N, K, gelu, path):
    _linear_case(act, M, N, K, gelu, path, True)


@pytest.mark.parametrize("path", [0, 9])
def test_linear_no_bias(path):
    _linear_case("bf16", 1000, 2560, 512, 1, path, False)


def _linear_case(act, M, N, K, gelu, path, with_bias):
    say(f"linear act={act} M={M} N={N} K={K} gelu={gelu} path={path} bias={with_bias}")
    bf = act == "bf16"
    dt = torch.bfloat16 if bf else torch.float32
    x = gen_normal(DEV, (M, K), 9, 6, 10, bf16=bf).to(dt)
    w = gen_normal(DEV, (N, K), 9, 6, 11, std=0.05, bf16=bf).to(dt)
    b = gen_normal(DEV, (N,), 9, 6, 12, std=0.5) if with_bias else None
    y = torch.empty(M, N, dtype=dt, device=DEV)
    L.whisper_linear(L.WHISPER_BF16 if bf else L.WHISPER_F32, x, K, w, b, M, N, K, gelu, y, path)
    torch.cuda.synchronize()
    ref = O.linear(host(x), host(w), host(b) if with_bias else np.zeros(N))
    if gelu:
        ref = O.gelu(ref)
    assert rel_err(host(y), ref) < TOL
    # per-row bound too (rows are the unit that later steps see)
    for i in (0, M // 2, M - 1):
        assert rel_err(host(y)[i], ref[i]) < TOL


# ------------------------------------------------------------------ attention
@pytest.mark.parametrize("act,B,T,H", [("bf16", 2, 300, 3), ("bf16", 1, 1500, 2), ("f32", 1, 200, 2)])
def test_attention_encoder(act, B, T, H):
    say(f"attention_encoder act={act} B={B} T={T} H={H}")
    bf = act == "bf16"
    dt = torch.bfloat16 if bf else torch.float32
    d = 64 * H
    qkv = gen_normal(DEV, (B, T, 3 * d), 9, 6, 20, std=1.5, bf16=bf).to(dt)
    out = torch.empty(B, T, d, dtype=dt, device=DEV)
    L.whisper_attention_encoder(L.WHISPER_BF16 if bf else L.WHISPER_F32, qkv, B, T, H, out)
    torch.cuda.synchronize()
    q = host(qkv)
    for b in range(B):
        ref = O.attention(q[b, :, :d], q[b, :, d:2 * d], q[b, :, 2 * d:], H)
        assert rel_err(host(out)[b], ref) < TOL


@pytest.mark.parametrize("cap,n_keys", [
    (100, [1, 17, 64, 99, 100]),
    # the kernel walks keys in batches of 512: one key, both sides of the batch
    # boundary, and the capacity of the batch-64 decode workload (448 + 224)
    (672, [1, 511, 512, 513, 671, 672]),
    # every frame of a 30 s chunk: the fp8 cross-attention form of the kernel
    (1500, [1500, 1024, 1499]),
])
def test_attention_decode_self_fp8(cap, n_keys):
    B, H = len(n_keys), 3
    say(f"attention_decode_self B={B} H={H} cap={cap} n_keys={n_keys}")
    g = torch.Generator().manual_seed(5 + cap)
    kc = torch.randint(0, 256, (B, H, cap, 64), generator=g, dtype=torch.int32)
    vc = torch.randint(0, 256, (B, H, cap, 64), generator=g, dtype=torch.int32)
    kc[(kc & 0x7F) == 0x7F] = 0x40   # no NaN codes among the keys
    vc[(vc & 0x7F) == 0x7F] = 0x41
    n_keys = torch.tensor(n_keys, dtype=torch.int32)
    # poison every slot past n_keys with NaN codes: causality means they are never read
    for b in range(B):
        kc[b, :, n_keys[b]:] = 0x7F
        vc[b, :, n_keys[b]:] = 0xFF
    kc, vc = kc.to(torch.uint8), vc.to(torch.uint8)
    q = gen_normal(DEV, (B, H * 64), 9, 6, 30, bf16=True).to(torch.bfloat16)
    scales = torch.tensor([0.004, 0.01, 0, 0], dtype=torch.float32, device=DEV)
    # canary bytes around the output: only the B x H*64 outputs are written
    buf = torch.full((B * H * 64 + 2 * 64,), -7.0, dtype=torch.bfloat16, device=DEV)
    out = buf[64:64 + B * H * 64].view(B, H * 64)
    L.whisper_attention_decode_self(L.WHISPER_BF16, q, B, H, cap, kc.to(DEV), vc.to(DEV), scales,
                                    n_keys.to(DEV), out)
    torch.cuda.synchronize()
    assert torch.all(buf[:64] == -7.0) and torch.all(buf[64 + B * H * 64:] == -7.0), "write outside the output"
    got = host(out)
    assert np.isfinite(got).all()
    qh = host(q)
    for b in range(B):
        n = int(n_keys[b])
        for h in range(H):
            kh = O.e4m3_dequantize(kc[b, h, :n].numpy(), np.float32(0.004))
            vh = O.e4m3_dequantize(vc[b, h, :n].numpy(), np.float32(0.01))
            ref = O.softmax(kh @ qh[b, h * 64:(h + 1) * 64] / 8.0) @ vh
            assert rel_err(got[b, h * 64:(h + 1) * 64], ref) < TOL, (b, h)


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_attention_decode_cross(act):
    B, H, T = 3, 2, 1500
    say(f"attention_decode_cross act={act} B={B} H={H} T={T}")
    bf = act == "bf16"
    dt = torch.bfloat16 if bf else torch.float32
    q = gen_normal(DEV, (B, H * 64), 9, 6, 40, std=0.5, bf16=bf).to(dt)
    k = gen_normal(DEV, (B, H, T, 64), 9, 6, 41, bf16=bf).to(dt)
    v = gen_normal(DEV, (B, H, T, 64), 9, 6, 42, bf16=bf).to(dt)
    out = torch.empty(B, H * 64, dtype=dt, device=DEV)
    nws = L.whisper_attention_decode_cross_workspace_size(B, H, T)
    ws = torch.empty(nws, dtype=torch.uint8, device=DEV)
    L.whisper_attention_decode_cross(L.WHISPER_BF16 if bf else L.WHISPER_F32, q, k, v, B, H, T, out, ws, nws)
    torch.cuda.synchronize()
    qh, kh, vh, got = host(q), host(k), host(v), host(out)
    for b in range(B):
        for h in range(H):
            ref = O.softmax(kh[b, h] @ qh[b, h * 64:(h + 1) * 64] / 8.0) @ vh[b, h]
            assert rel_err(got[b, h * 64:(h + 1) * 64], ref) < TOL


# ------------------------------------------------------------------ log-mel
@pytest.mark.parametrize("n_mels,n_samples", [(128, 480000), (80, 160000)])
def test_logmel(n_mels, n_samples):
    from workload import gen_audio_tones
    say(f"logmel n_mels={n_mels} n_samples={n_samples}")
    dims = CONFIGS["v3_encoder"] if n_mels == 128 else CONFIGS["tiny_f32"]
    B = 2
    audio = gen_audio_tones(DEV, 9, B, seconds=n_samples / 16000, total=n_samples)
    mel = torch.empty(B, n_mels, 3000, dtype=torch.float32, device=DEV)
    nws = L.whisper_workspace_size(dims, B, L.WS_LOGMEL)
    ws = torch.empty(nws, dtype=torch.uint8, device=DEV)
    L.whisper_logmel(dims, audio, B, n_samples, mel, ws, nws)
    torch.cuda.synchronize()
    for b in range(B):
        ref = O.log_mel(audio[b].cpu().numpy(), n_mels)
        e = rel_err(host(mel)[b], ref)
        say(f"  chunk {b}: rel err {e:.2e}")
        assert e < 1e-3


@pytest.mark.parametrize("stride", [400000, 480000])
def test_logmel_chunked_long_recording(stride):
    """Overlapping (25 s stride) and back-to-back chunks of one 75.5 s
    recording: each chunk's log-mel against the oracle's slice of the same
    recording (the last chunk zero-padded)."""
    from workload import gen_audio_longform
    dims = CONFIGS["v3_encoder"]
    n = 1_208_000
    rec = gen_audio_longform(DEV, 9, minutes=3.0)[:3].reshape(-1)[:n].contiguous()
    count, plan = L.whisper_chunk_plan(n, stride)
    say(f"logmel_chunked n={n} stride={stride}: {count} chunks")
    mel = torch.empty(count, 128, 3000, dtype=torch.float32, device=DEV)
    nws = L.whisper_workspace_size(dims, count, L.WS_LOGMEL)
    ws = torch.empty(nws, dtype=torch.uint8, device=DEV)
    L.whisper_logmel_chunked(dims, rec, n, stride, mel, ws, nws)
    torch.cuda.synchronize()
    ref = O.log_mel_chunked(rec.cpu().double().numpy(), stride, 128)
    assert ref.shape[0] == count
    for i in range(count):
        e = rel_err(host(mel)[i], ref[i])
        say(f"  chunk {i} (samples {plan[i][0]}..+{plan[i][1]}): rel err {e:.2e}")
        assert e < 1e-3


# ------------------------------------------------------------------ fp8 GEMM (mixed_fp8 sites)
@pytest.mark.parametrize("gelu", [False, True])
def test_gemm_fp8_codes_against_exact_products(gelu):
    """whisper_gemm_fp8 on seeded E4M3 codes: 700 rows (3 row tiles, ragged),
    512 columns (2 tiles), K = 1280, row scales in groups of 300 rows (groups
    cross tile edges), a weight scale and a bias, against the exact products
    of the codes' values (fp64), scaled, biased, GELU'd, then bf16."""
    say(f"fp8 GEMM 700x512x1280, gelu={gelu}")
    M, N, K, rps = 700, 512, 1280, 300
    g = torch.Generator().manual_seed(11)
    a = torch.randint(0, 256, (M, K), generator=g, dtype=torch.int32).to(torch.uint8)
    w = torch.randint(0, 256, (N, K), generator=g, dtype=torch.int32).to(torch.uint8)
    a[(a & 0x7F) == 0x7F] = 0  # no NaN codes
    w[(w & 0x7F) == 0x7F] = 0
    sa = (torch.rand(3, generator=g) * 0.01 + 0.001).float()
    sw = (torch.rand(1, generator=g) * 0.01 + 0.001).float()
    bias = torch.randn(N, generator=g).float()
    c = torch.full((M, N + 8), float("nan"), dtype=torch.bfloat16)
    dev = [t.to(DEV) for t in (a, w, sa, sw, bias, c)]
    L.whisper_gemm_fp8(dev[0], M, K, dev[2], rps, dev[1], N, dev[3], dev[4], gelu, dev[5], N + 8)
    torch.cuda.synchronize()
    got = dev[5].float().cpu().numpy()
    va, vw = O.e4m3_value(a.numpy()), O.e4m3_value(w.numpy())
    scale = np.float32(sa.numpy()[np.arange(M) // rps])[:, None].astype(np.float64) * float(sw[0])
    ref = (va @ vw.T) * scale + bias.numpy().astype(np.float64)
    if gelu:
        ref = O.gelu(ref)
    assert np.all(np.isnan(got[:, N:])), "columns past N must stay untouched"
    err = np.abs(got[:, :N] - ref)
    # fp32 summation of K exact products: |error| <= K 2^-24 sum |terms| (the
    # textbook bound for any order), doubled for the scale and bias roundings
    # and GELU's slope; then one bf16 rounding of the result
    terms = (np.abs(va) @ np.abs(vw).T) * scale
    bound = 2.0 ** -8 * np.abs(ref) + 2 * K * 2.0 ** -24 * (terms + np.abs(bias.numpy())) + 1e-6
    bad = np.argwhere(err > bound)
    assert bad.size == 0, (f"{len(bad)} outputs beyond the bound, first {bad[:3].tolist()}: "
                           f"got {got[tuple(bad[0])]}, ref {ref[tuple(bad[0])]}, bound {bound[tuple(bad[0])]}")
    # typical error is far inside the worst-case bound
    assert np.median(err / (np.abs(ref) + 1e-3)) < 2.0 ** -8



@pytest.mark.parametrize("N,K,gelu", [(5120, 1280, True), (1280, 5120, False)])
def test_gemm_fp8_full_encoder_shape_sampled_rows(N, K, gelu):
    """whisper_gemm_fp8 at the encoder's full batch-64 shapes (96000 rows:
    fc1 5120x1280 + GELU, fc2 1280x5120), one scale per 1500-row chunk as the
    encoder runs it; one sampled row per chunk checked against the exact
    products of its codes, inside the fp32 summation bound."""
    say(f"fp8 GEMM 96000x{N}x{K}, gelu={gelu}, sampled rows")
    M, rps = 96000, 1500
    g = torch.Generator().manual_seed(12)
    a = torch.randint(0, 256, (M, K), generator=g, dtype=torch.int32).to(torch.uint8)
    w = torch.randint(0, 256, (N, K), generator=g, dtype=torch.int32).to(torch.uint8)
    a[(a & 0x7F) == 0x7F] = 0
    w[(w & 0x7F) == 0x7F] = 0
    sa = (torch.rand(M // rps, generator=g) * 0.01 + 0.001).float()
    sw = (torch.rand(1, generator=g) * 0.01 + 0.001).float()
    bias = torch.randn(N, generator=g).float()
    dev = [t.to(DEV) for t in (a, w, sa, sw, bias)]
    c = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    L.whisper_gemm_fp8(dev[0], M, K, dev[2], rps, dev[1], N, dev[3], dev[4], gelu, c, N)
    torch.cuda.synchronize()
    rows = np.array([ch * rps + (ch * 37) % rps for ch in range(M // rps)] + [M - 1])
    got = c[torch.from_numpy(rows).to(DEV)].float().cpu().numpy()
    va, vw = O.e4m3_value(a.numpy()[rows]), O.e4m3_value(w.numpy())
    scale = np.float32(sa.numpy()[rows // rps])[:, None].astype(np.float64) * float(sw[0])
    ref = (va @ vw.T) * scale + bias.numpy().astype(np.float64)
    if gelu:
        ref = O.gelu(ref)
    terms = (np.abs(va) @ np.abs(vw).T) * scale
    bound = 2.0 ** -8 * np.abs(ref) + 2 * K * 2.0 ** -24 * (terms + np.abs(bias.numpy())) + 1e-6
    assert np.all(np.abs(got - ref) <= bound)
