"""Pins of the oracle's layers against independent library implementations
(torch CPU in float64), closed forms, brute force and invariants."""
import numpy as np
import pytest
import scipy.signal
import torch
import torch.nn.functional as F

from oracle import whisper_oracle as O



@pytest.fixture(autouse=True)
def _float64_default():
    """torch CPU references in float64, restored afterwards (the GPU tests
    collected in the same session build their inputs with torch defaults)."""
    prev = torch.get_default_dtype()
    torch.set_default_dtype(torch.float64)
    yield
    torch.set_default_dtype(prev)


def T(a):
    return torch.from_numpy(np.ascontiguousarray(a))


def test_gelu_identities_and_torch():
    x = np.linspace(-6, 6, 1001)
    assert np.allclose(O.gelu(x) - O.gelu(-x), x, atol=1e-15)
    assert O.gelu(np.array([0.0]))[0] == 0.0
    assert np.allclose(O.gelu(x), F.gelu(T(x)).numpy(), atol=1e-15)


def test_layer_norm_invariants_and_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 384)) * 3 + 1.5
    n = O.layer_norm(x, np.ones(384), np.zeros(384))
    var = x.var(axis=1)
    assert np.allclose(n.mean(axis=1), 0, atol=1e-12)
    assert np.allclose(n.var(axis=1), var / (var + 1e-5), atol=1e-12)
    g, b = rng.standard_normal(384), rng.standard_normal(384)
    ref = F.layer_norm(T(x), (384,), T(g), T(b), 1e-5).numpy()
    assert np.allclose(O.layer_norm(x, g, b), ref, atol=1e-12)


def test_residual_layer_norm_returns_sum_and_norm():
    rng = np.random.default_rng(1)
    h, r = rng.standard_normal((5, 64)), rng.standard_normal((5, 64))
    g, b = rng.standard_normal(64), rng.standard_normal(64)
    normed, total = O.residual_layer_norm(h, r, g, b)
    assert np.array_equal(total, h + r)
    assert np.allclose(normed, F.layer_norm(T(h + r), (64,), T(g), T(b), 1e-5).numpy(), atol=1e-12)
    normed0, total0 = O.residual_layer_norm(h, None, g, b)
    assert np.array_equal(total0, h)


def test_conv1d_against_scipy_and_torch():
    rng = np.random.default_rng(2)
    x, w, b = rng.standard_normal((5, 17)), rng.standard_normal((4, 5, 3)), rng.standard_normal(4)
    for stride in (1, 2):
        got = O.conv1d(x, w, b, stride, 1)
        ref = F.conv1d(T(x)[None], T(w), T(b), stride=stride, padding=1)[0].numpy()
        assert got.shape == ref.shape
        assert np.allclose(got, ref, atol=1e-12)
    # per channel pair with scipy's correlate on the zero-padded input
    got = O.conv1d(x, w, b, 1, 1)
    xp = np.pad(x, ((0, 0), (1, 1)))
    ref = np.stack([b[o] + sum(scipy.signal.correlate(xp[i], w[o, i], mode="valid") for i in range(5)) for o in range(4)])
    assert np.allclose(got, ref, atol=1e-12)
    # 3000 frames -> 1500 after the stride-2 conv
    assert O.conv1d(np.zeros((1, 3000)), np.zeros((1, 1, 3)), np.zeros(1), 2, 1).shape == (1, 1500)


def test_sinusoids_closed_form():
    pe = O.sinusoids(1500, 1280)
    assert np.all(pe[0, :640] == 0.0) and np.all(pe[0, 640:] == 1.0)
    t = np.arange(1500)
    assert np.allclose(pe[:, 0], np.sin(t)) and np.allclose(pe[:, 640], np.cos(t))
    assert np.allclose(pe[:, 639], np.sin(t / 10000.0))


def test_attention_invariants_brute_force_and_torch():
    rng = np.random.default_rng(3)
    q, k, v = rng.standard_normal((6, 128)), rng.standard_normal((9, 128)), rng.standard_normal((9, 128))
    got = O.attention(q, k, v, 2)
    # brute force loops
    bf = np.zeros_like(got)
    for h in range(2):
        for i in range(6):
            s = [sum(q[i, h * 64 + e] * k[j, h * 64 + e] for e in range(64)) / 8.0 for j in range(9)]
            m = max(s)
            p = [np.exp(x - m) for x in s]
            z = sum(p)
            for j in range(9):
                bf[i, h * 64:(h + 1) * 64] += p[j] / z * v[j, h * 64:(h + 1) * 64]
    assert np.allclose(got, bf, atol=1e-12)
    # torch scaled_dot_product_attention, heads split out
    tq, tk, tv = (T(a).view(-1, 2, 64).transpose(0, 1) for a in (q, k, v))
    ref = F.scaled_dot_product_attention(tq, tk, tv).transpose(0, 1).reshape(6, 128).numpy()
    assert np.allclose(got, ref, atol=1e-12)
    # Q = 0 -> every row is the mean of V
    assert np.allclose(O.attention(np.zeros_like(q), k, v, 2), np.tile(v.mean(axis=0), (6, 1)))
    # one key -> output equals V
    assert np.allclose(O.attention(q, k[:1], v[:1], 2), np.tile(v[0], (6, 1)))
    # joint permutation of keys and values leaves the output unchanged
    perm = rng.permutation(9)
    assert np.allclose(O.attention(q, k[perm], v[perm], 2), got)
    # softmax rows sum to one
    assert np.allclose(O.softmax(rng.standard_normal((4, 33)) * 10).sum(axis=1), 1.0)


def _tiny_weights(rng, d=64, f=256, n_mels=16, n_enc=2, n_dec=2, vocab=50, ctx=12):
    W = {}
    def n(*s, std=0.2):
        return rng.standard_normal(s) * std
    W["encoder.conv1.weight"], W["encoder.conv1.bias"] = n(d, n_mels, 3), n(d)
    W["encoder.conv2.weight"], W["encoder.conv2.bias"] = n(d, d, 3), n(d)
    for l in range(n_enc):
        p = f"encoder.blocks.{l}."
        for ln in ("attn_ln", "mlp_ln"):
            W[p + ln + ".weight"], W[p + ln + ".bias"] = 1 + n(d, std=0.1), n(d, std=0.1)
        for m in ("query", "key", "value", "out"):
            W[p + f"attn.{m}.weight"] = n(d, d)
            if m != "key":
                W[p + f"attn.{m}.bias"] = n(d)
        W[p + "mlp.0.weight"], W[p + "mlp.0.bias"] = n(f, d), n(f)
        W[p + "mlp.2.weight"], W[p + "mlp.2.bias"] = n(d, f), n(d)
    W["encoder.ln_post.weight"], W["encoder.ln_post.bias"] = 1 + n(d, std=0.1), n(d, std=0.1)
    W["decoder.token_embedding"], W["decoder.positional_embedding"] = n(vocab, d), n(ctx, d)
    for l in range(n_dec):
        p = f"decoder.blocks.{l}."
        for ln in ("attn_ln", "cross_attn_ln", "mlp_ln"):
            W[p + ln + ".weight"], W[p + ln + ".bias"] = 1 + n(d, std=0.1), n(d, std=0.1)
        for a in ("attn", "cross_attn"):
            for m in ("query", "key", "value", "out"):
                W[p + f"{a}.{m}.weight"] = n(d, d)
                if m != "key":
                    W[p + f"{a}.{m}.bias"] = n(d)
        W[p + "mlp.0.weight"], W[p + "mlp.0.bias"] = n(f, d), n(f)
        W[p + "mlp.2.weight"], W[p + "mlp.2.bias"] = n(d, f), n(d)
    W["decoder.ln.weight"], W["decoder.ln.bias"] = 1 + n(d, std=0.1), n(d, std=0.1)
    return W


def _load_mha(mha, W, p, d):
    with torch.no_grad():
        mha.in_proj_weight.copy_(T(np.concatenate([W[p + "query.weight"], W[p + "key.weight"], W[p + "value.weight"]])))
        mha.in_proj_bias.copy_(T(np.concatenate([W[p + "query.bias"], np.zeros(d), W[p + "value.bias"]])))
        mha.out_proj.weight.copy_(T(W[p + "out.weight"]))
        mha.out_proj.bias.copy_(T(W[p + "out.bias"]))


def _load_ln(ln, W, p):
    with torch.no_grad():
        ln.weight.copy_(T(W[p + ".weight"]))
        ln.bias.copy_(T(W[p + ".bias"]))


def _load_mlp(layer, W, p):
    with torch.no_grad():
        layer.linear1.weight.copy_(T(W[p + "mlp.0.weight"]))
        layer.linear1.bias.copy_(T(W[p + "mlp.0.bias"]))
        layer.linear2.weight.copy_(T(W[p + "mlp.2.weight"]))
        layer.linear2.bias.copy_(T(W[p + "mlp.2.bias"]))


def test_encoder_layer_matches_torch_transformer_encoder_layer():
    rng = np.random.default_rng(4)
    d, H = 64, 2
    W = _tiny_weights(rng, d=d)
    x = rng.standard_normal((23, d))
    ref_layer = torch.nn.TransformerEncoderLayer(d, H, 256, dropout=0.0, activation="gelu",
                                                 layer_norm_eps=1e-5, batch_first=True, norm_first=True)
    p = "encoder.blocks.0."
    _load_mha(ref_layer.self_attn, W, p + "attn.", d)
    _load_ln(ref_layer.norm1, W, p + "attn_ln")
    _load_ln(ref_layer.norm2, W, p + "mlp_ln")
    _load_mlp(ref_layer, W, p)
    ref_layer.eval()
    with torch.no_grad():
        ref = ref_layer(T(x)[None])[0].numpy()
    assert np.allclose(O.encoder_layer(x, W, 0, H), ref, atol=1e-10)


def test_encoder_from_mel_matches_torch_composition():
    rng = np.random.default_rng(5)
    d, H, n_mels = 64, 2, 16
    W = _tiny_weights(rng, d=d, n_mels=n_mels)
    mel = rng.standard_normal((n_mels, 40))
    got = O.encoder(mel, W, H, 2)
    x = F.gelu(F.conv1d(T(mel)[None], T(W["encoder.conv1.weight"]), T(W["encoder.conv1.bias"]), padding=1))
    x = F.gelu(F.conv1d(x, T(W["encoder.conv2.weight"]), T(W["encoder.conv2.bias"]), stride=2, padding=1))[0].T
    t = torch.arange(20.0)[:, None]
    inv = torch.exp(-np.log(10000.0) / 31 * torch.arange(32.0))[None]
    x = x + torch.cat([torch.sin(t * inv), torch.cos(t * inv)], dim=1)
    for l in range(2):
        layer = torch.nn.TransformerEncoderLayer(d, H, 256, dropout=0.0, activation="gelu",
                                                 batch_first=True, norm_first=True)
        p = f"encoder.blocks.{l}."
        _load_mha(layer.self_attn, W, p + "attn.", d)
        _load_ln(layer.norm1, W, p + "attn_ln")
        _load_ln(layer.norm2, W, p + "mlp_ln")
        _load_mlp(layer, W, p)
        layer.eval()
        with torch.no_grad():
            x = layer(x[None])[0]
    ref = F.layer_norm(x, (d,), T(W["encoder.ln_post.weight"]), T(W["encoder.ln_post.bias"]), 1e-5).detach().numpy()
    assert got.shape == (20, d)
    assert np.allclose(got, ref, atol=1e-10)


def test_decode_steps_match_torch_causal_decoder():
    """Exact-cache incremental decode == full causal torch decoder at every position."""
    rng = np.random.default_rng(6)
    d, H, L, V, ctx, Tenc, B, steps = 64, 2, 2, 50, 12, 7, 3, 6
    W = _tiny_weights(rng, d=d, n_dec=L, vocab=V, ctx=ctx)
    enc = rng.standard_normal((B, Tenc, d))
    toks = rng.integers(0, V, (steps, B))
    cross_b = [O.cross_kv(enc[b], W, H, L) for b in range(B)]
    cross = [(np.stack([cross_b[b][l][0] for b in range(B)]), np.stack([cross_b[b][l][1] for b in range(B)]))
             for l in range(L)]
    cache = np.zeros((L, 2, B, H, ctx, d // H))
    layers = []
    for l in range(L):
        layer = torch.nn.TransformerDecoderLayer(d, H, 256, dropout=0.0, activation="gelu",
                                                 batch_first=True, norm_first=True)
        p = f"decoder.blocks.{l}."
        _load_mha(layer.self_attn, W, p + "attn.", d)
        _load_mha(layer.multihead_attn, W, p + "cross_attn.", d)
        _load_ln(layer.norm1, W, p + "attn_ln")
        _load_ln(layer.norm2, W, p + "cross_attn_ln")
        _load_ln(layer.norm3, W, p + "mlp_ln")
        _load_mlp(layer, W, p)
        layer.eval()
        layers.append(layer)
    for t in range(steps):
        lengths = np.full(B, t)
        logits, _ = O.decode_step(W, H, toks[t], lengths, cache, None, cross)
        x = T(W["decoder.token_embedding"][toks[:t + 1].T] + W["decoder.positional_embedding"][:t + 1][None])
        mask = torch.nn.Transformer.generate_square_subsequent_mask(t + 1)
        with torch.no_grad():
            for layer in layers:
                x = layer(x, T(enc), tgt_mask=mask)
            y = F.layer_norm(x[:, -1], (d,), T(W["decoder.ln.weight"]), T(W["decoder.ln.bias"]), 1e-5)
            ref = (y @ T(W["decoder.token_embedding"]).T).numpy()
        assert np.allclose(logits, ref, atol=1e-9), t


def _fp8_setup(seed=7, B=3, steps=5):
    rng = np.random.default_rng(seed)
    d, H, L, V, ctx, Tenc = 64, 2, 2, 50, 12, 7
    W = _tiny_weights(rng, d=d, n_dec=L, vocab=V, ctx=ctx)
    enc = rng.standard_normal((B, Tenc, d))
    cross_b = [O.cross_kv(enc[b], W, H, L) for b in range(B)]
    cross = [(np.stack([cross_b[b][l][0] for b in range(B)]), np.stack([cross_b[b][l][1] for b in range(B)]))
             for l in range(L)]
    toks = rng.integers(0, V, (steps, B))
    scales = np.full((L, 2), np.float32(0.03), np.float32)
    return W, H, L, ctx, cross, toks, scales, d // H


def test_fp8_decode_properties():
    W, H, L, ctx, cross, toks, scales, dh = _fp8_setup()
    B = toks.shape[1]
    cache = np.zeros((L, 2, B, H, ctx, dh), np.uint8)
    cache_nan = np.full((L, 2, B, H, ctx, dh), 0x7F, np.uint8)   # NaN codes in every unwritten slot
    exact = np.zeros((L, 2, B, H, ctx, dh))
    for t in range(toks.shape[0]):
        lengths = np.full(B, t)
        lg, tr = O.decode_step(W, H, toks[t], lengths, cache, scales, cross)
        lg_nan, _ = O.decode_step(W, H, toks[t], lengths, cache_nan, scales, cross)
        lg_exact, _ = O.decode_step(W, H, toks[t], lengths, exact, None, cross)
        # causal: slots beyond the current position are never read
        assert np.array_equal(lg, lg_nan)
        # the stored codes are the codec applied to the new token's K / V, and
        # those K / V are the exact-cache step's
        for l in range(L):
            for kv in range(2):
                assert np.array_equal(cache[l, kv, :, :, t, :], O.e4m3_quantize(tr["kv"][l, kv], scales[l, kv]))
                assert np.array_equal(cache[l, kv, :, :, t, :], tr["codes"][l, kv])
        # quantisation noise is small next to the logits
        assert np.abs(lg - lg_exact).max() < 0.1 * np.abs(lg_exact).max()
    # rows are independent: computing a subset gives the same rows
    cache2 = np.zeros_like(cache)
    for t in range(toks.shape[0]):
        lg_sub, _ = O.decode_step(W, H, toks[t], np.full(B, t), cache2, scales, cross, rows=[1])
    assert np.array_equal(lg_sub[1], lg[1])
    assert np.array_equal(cache2[:, :, 1], cache[:, :, 1])


def test_fp8_decode_position_zero_reads_its_own_value():
    """At position 0 the self-attention softmax has one key, so the attention
    output equals the dequantised V just written; check through a layer whose
    out-projection is the identity and whose later sublayers are zeroed."""
    W, H, L, ctx, cross, toks, scales, dh = _fp8_setup(seed=8, B=2, steps=1)
    d = H * dh
    W = dict(W)
    p = "decoder.blocks.0."
    W[p + "attn.out.weight"] = np.eye(d)
    W[p + "attn.out.bias"] = np.zeros(d)
    for k in ("cross_attn.out.weight", "cross_attn.out.bias", "mlp.2.weight", "mlp.2.bias"):
        W[p + k] = np.zeros_like(W[p + k])
    cross1 = cross[:1]
    cache = np.zeros((1, 2, 2, H, ctx, dh), np.uint8)
    _, tr = O.decode_step(W, H, toks[0], np.zeros(2, int), cache, scales[:1], cross1)
    x0 = W["decoder.token_embedding"][toks[0]] + W["decoder.positional_embedding"][0]
    v_hat = O.e4m3_dequantize(cache[0, 1, :, :, 0, :], scales[0, 1]).reshape(2, d)
    assert np.allclose(tr["x"], x0 + v_hat, atol=1e-12)


def test_prefill_matches_torch_causal_decoder():
    """A causal prefill of P tokens per row from an exact cache gives the last
    position's logits of the full causal torch decoder over those P tokens, and
    with an fp8 cache it equals P single steps code for code."""
    rng = np.random.default_rng(10)
    d, H, L, V, ctx, Tenc, B, P = 64, 2, 2, 50, 12, 7, 2, 5
    W = _tiny_weights(rng, d=d, n_dec=L, vocab=V, ctx=ctx)
    enc = rng.standard_normal((B, Tenc, d))
    toks = rng.integers(0, V, (B, P))
    cross_b = [O.cross_kv(enc[b], W, H, L) for b in range(B)]
    cross = [(np.stack([cross_b[b][l][0] for b in range(B)]), np.stack([cross_b[b][l][1] for b in range(B)]))
             for l in range(L)]
    exact = np.zeros((L, 2, B, H, ctx, d // H))
    logits, traces = O.decode_prefill(W, H, toks, np.zeros(B, int), exact, None, cross)
    assert len(traces) == P
    x = T(W["decoder.token_embedding"][toks] + W["decoder.positional_embedding"][:P][None])
    mask = torch.nn.Transformer.generate_square_subsequent_mask(P)
    with torch.no_grad():
        for l in range(L):
            layer = torch.nn.TransformerDecoderLayer(d, H, 256, dropout=0.0, activation="gelu",
                                                     batch_first=True, norm_first=True)
            p = f"decoder.blocks.{l}."
            _load_mha(layer.self_attn, W, p + "attn.", d)
            _load_mha(layer.multihead_attn, W, p + "cross_attn.", d)
            _load_ln(layer.norm1, W, p + "attn_ln")
            _load_ln(layer.norm2, W, p + "cross_attn_ln")
            _load_ln(layer.norm3, W, p + "mlp_ln")
            _load_mlp(layer, W, p)
            layer.eval()
            x = layer(x, T(enc), tgt_mask=mask)
        y = F.layer_norm(x[:, -1], (d,), T(W["decoder.ln.weight"]), T(W["decoder.ln.bias"]), 1e-5)
        ref = (y @ T(W["decoder.token_embedding"]).T).numpy()
    assert np.allclose(logits, ref, atol=1e-9)
    # fp8 cache: the prefill is P steps in a row, code for code
    scales = np.full((L, 2), np.float32(0.03), np.float32)
    c1 = np.zeros((L, 2, B, H, ctx, d // H), np.uint8)
    c2 = np.zeros_like(c1)
    lg1, _ = O.decode_prefill(W, H, toks, np.array([0, 3]), c1, scales, cross)
    lengths = np.array([0, 3])
    for p in range(P):
        lg2, _ = O.decode_step(W, H, toks[:, p], lengths, c2, scales, cross)
        lengths = lengths + 1
    assert np.array_equal(lg1, lg2) and np.array_equal(c1, c2)


def test_top2_gap_and_greedy_token():
    lg = np.array([[0.0, 3.0, 1.0, 3.0], [5.0, -1.0, 2.5, 0.0]])
    assert list(O.greedy_token(lg)) == [1, 0]  # lowest index among equal maxima
    assert np.allclose(O.top2_gap(lg), [0.0, 2.5])


def test_fp8_cross_kv_grid_values_exact_and_error_bound():
    """fp8 cross K/V: with power-of-two scales, values already on the scaled
    e4m3 grid pass unchanged (so a decode step over such K/V equals the
    unquantised step exactly);
    others move by at most half an e4m3 step: 2^-4 of the value in the
    normal range, 2^-10 * scale in the subnormal range; magnitudes past
    448 * scale saturate. Dict and array forms agree. With kv_transform =
    bf16_round the bf16 rounding (2^-9) adds to the bound, and the result is
    the quantisation of the rounded values."""
    W, H, L, ctx, cross, toks, scales, dh = _fp8_setup()
    scales = np.array([[2.0 ** -5, 2.0 ** -4], [2.0 ** -6, 2.0 ** -3]], np.float32)  # exact in fp32 both ways
    rng = np.random.default_rng(5)
    # snap every K/V onto the scaled grid (finite codes only, within range)
    grid = []
    for layer, (k, v) in enumerate(cross):
        pair = []
        for kv, x in ((0, k), (1, v)):
            codes = rng.integers(0, 256, x.shape).astype(np.uint8)
            codes[(codes & 0x7F) == 0x7F] = 0
            pair.append(O.e4m3_value(codes).astype(np.float64) * np.float64(np.float32(scales[layer][kv])))
        grid.append(tuple(pair))
    q = O.cross_kv_fp8(grid, scales)
    for layer in range(L):
        for kv in range(2):
            assert np.array_equal(q[layer][kv], grid[layer][kv])
    qd = O.cross_kv_fp8([({b: k[b] for b in range(k.shape[0])}, {b: v[b] for b in range(v.shape[0])})
                         for k, v in grid], scales)
    assert all(np.array_equal(qd[l][kv][b], q[l][kv][b]) for l in range(L) for kv in range(2) for b in range(2))
    B = toks.shape[1]
    c1 = np.zeros((L, 2, B, H, ctx, dh), np.uint8)
    c2 = np.zeros_like(c1)
    lg1, _ = O.decode_step(W, H, toks[0], np.zeros(B, int), c1, scales, grid)
    lg2, _ = O.decode_step(W, H, toks[0], np.zeros(B, int), c2, scales, q)
    assert np.array_equal(lg1, lg2)
    # error bound on general values, with saturation past the range
    s = np.float32(0.01)
    x = rng.standard_normal(20000) * 1.5
    x[:10] = [5.0, -5.0, 4.48, -4.48, 1e-6, -1e-6, 0.0, 3e-5, 100.0, -100.0]
    y = O.cross_kv_fp8([(x, x)], np.array([[s, s]], np.float32))[0][0]
    inr = np.abs(x) <= 448 * float(s)
    normal = inr & (np.abs(x) >= 2.0 ** -6 * float(s))
    # half an e4m3 step: 2^-4 of the value in the normal range, 2^-10 * scale below
    assert np.all(np.abs(y - x)[normal] <= 2.0 ** -4 * np.abs(x[normal]) * (1 + 1e-6))
    sub = inr & ~normal
    assert np.all(np.abs(y - x)[sub] <= 2.0 ** -10 * float(s) * (1 + 1e-6))
    assert np.all(np.abs(y[~inr]) == np.float64(np.float32(448.0) * s))
    # with the values rounded to bf16 first: that rounding (2^-9) on top
    yb = O.cross_kv_fp8([(x, x)], np.array([[s, s]], np.float32), kv_transform=O.bf16_round)[0][0]
    bf = 2.0 ** -9
    assert np.all(np.abs(yb - x)[normal] <= (2.0 ** -4 * (1 + bf) + bf) * np.abs(x[normal]) * (1 + 1e-6))
    assert np.array_equal(yb, O.cross_kv_fp8([(O.bf16_round(x), x)], np.array([[s, s]], np.float32))[0][0])


def test_fp8_cross_kv_e5m2_grid_values_exact_and_error_bound():
    """fp8 cross K/V in E5M2 (the aggressive preset's cross-attention format):
    with power-of-two scales, values on the scaled e5m2 grid pass unchanged,
    so a decode step over them equals the unquantised step exactly; others
    move by at most half an e5m2 step (2^-3 of the value in the normal
    range, 2^-17 * scale below it); past 57344 * scale they saturate."""
    W, H, L, ctx, cross, toks, scales, dh = _fp8_setup()
    scales = np.array([[2.0 ** -12, 2.0 ** -11], [2.0 ** -13, 2.0 ** -10]], np.float32)
    rng = np.random.default_rng(6)
    grid = []
    for layer, (k, v) in enumerate(cross):
        pair = []
        for kv, x in ((0, k), (1, v)):
            codes = rng.integers(0, 256, x.shape).astype(np.uint8)
            codes[(codes & 0x7F) >= 0x7C] = 0
            pair.append(O.e5m2_value(codes).astype(np.float64) * np.float64(np.float32(scales[layer][kv])))
        grid.append(tuple(pair))
    q = O.cross_kv_fp8(grid, scales, fmt="e5m2")
    for layer in range(L):
        for kv in range(2):
            assert np.array_equal(q[layer][kv], grid[layer][kv])
    # the E4M3 form of the same values is not exact (E5M2's exponent range)
    q4 = O.cross_kv_fp8(grid, scales, fmt="e4m3")
    assert not all(np.array_equal(q4[l][kv], grid[l][kv]) for l in range(L) for kv in range(2))
    B = toks.shape[1]
    c1 = np.zeros((L, 2, B, H, ctx, dh), np.uint8)
    c2 = np.zeros_like(c1)
    lg1, _ = O.decode_step(W, H, toks[0], np.zeros(B, int), c1, scales, grid)
    lg2, _ = O.decode_step(W, H, toks[0], np.zeros(B, int), c2, scales, q)
    assert np.array_equal(lg1, lg2)
    s = np.float32(0.01)
    x = rng.standard_normal(20000) * 50.0
    x[:8] = [600.0, -600.0, 573.44, -573.44, 1e-9, 0.0, 1e4, -1e4]
    y = O.cross_kv_fp8([(x, x)], np.array([[s, s]], np.float32), fmt="e5m2")[0][0]
    inr = np.abs(x) <= 57344 * float(s)
    normal = inr & (np.abs(x) >= 2.0 ** -14 * float(s))
    assert np.all(np.abs(y - x)[normal] <= 2.0 ** -3 * np.abs(x[normal]) * (1 + 1e-6))
    sub = inr & ~normal
    assert np.all(np.abs(y - x)[sub] <= 2.0 ** -17 * float(s) * (1 + 1e-6))
    assert np.all(np.abs(y[~inr]) == np.float64(np.float32(57344.0) * s))
