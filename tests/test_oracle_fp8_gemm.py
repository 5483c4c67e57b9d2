"""Pins of the oracle's mixed_fp8 encoder sites (fp8 E4M3 weights and
activations with per-tensor amax scales at the query/key/value and FFN
matmuls): grid values pass exactly, an independent library quantiser
(torch.float8_e4m3fn) gives the same product, the error stays inside the
half-step bound, and with fp8 off the layer is the plain encoder layer."""
import numpy as np
import torch

from oracle import whisper_oracle as O
from tests.test_oracle_layers import _tiny_weights


def _grid(rng, shape, s):
    codes = rng.integers(0, 256, shape).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0
    return O.e4m3_value(codes) * s


def test_fp8_linear_exact_on_scaled_grid():
    rng = np.random.default_rng(0)
    sx, sw = 2.0 ** -5, 2.0 ** -7
    x, w, b = _grid(rng, (37, 96), sx), _grid(rng, (40, 96), sw), rng.standard_normal(40)
    assert np.array_equal(O.fp8_linear(x, w, b, sx, sw), O.linear(x, w, b))
    assert np.array_equal(O.fp8_linear(x, w, None, sx, sw), O.linear(x, w))


def test_fp8_linear_matches_torch_quantiser():
    rng = np.random.default_rng(1)
    x, w, b = rng.standard_normal((33, 128)) * 2.0, rng.standard_normal((24, 128)) * 0.05, rng.standard_normal(24)
    sx, sw = O.e4m3_scale_from_amax(x), O.e4m3_scale_from_amax(w)

    def tq(a, s):  # fl32(a * fl32(1/s)) rounded by torch's float8_e4m3fn conversion
        y = torch.from_numpy(a.astype(np.float32)) * torch.tensor(np.float32(1.0) / np.float32(s))
        return y.to(torch.float8_e4m3fn).to(torch.float64).numpy()

    ref = (tq(x, sx) @ tq(w, sw).T) * (float(sx) * float(sw)) + b
    assert np.allclose(O.fp8_linear(x, w, b, sx, sw), ref, rtol=1e-13, atol=1e-13)


def test_fp8_linear_error_within_half_step_bound():
    rng = np.random.default_rng(2)
    x, w = rng.standard_normal((50, 64)), rng.standard_normal((30, 64)) * 0.1
    sx, sw = O.e4m3_scale_from_amax(x), O.e4m3_scale_from_amax(w)

    def half_step(a, s):  # 2^-4 relative in the normal range, 2^-10 * s below it
        return np.maximum(np.abs(a) * 2.0 ** -4, 2.0 ** -10 * float(s)) * (1 + 1e-6)

    dx, dw = half_step(x, sx), half_step(w, sw)
    bound = np.abs(x) @ dw.T + dx @ np.abs(w).T + dx @ dw.T
    err = np.abs(O.fp8_linear(x, w, None, sx, sw) - O.linear(x, w))
    assert np.all(err <= bound)
    assert err.max() > 0


def test_mixed_fp8_layer_off_is_the_plain_layer_and_on_stays_close():
    rng = np.random.default_rng(3)
    W = _tiny_weights(rng, d=64, f=256)
    x = rng.standard_normal((40, 64))
    assert np.array_equal(O.encoder_layer_mixed_fp8(x, W, 0, 2, fp8=False), O.encoder_layer(x, W, 0, 2))
    assert np.array_equal(O.encoder_layers_mixed_fp8(x, W, 2, [0, 1], fp8=False),
                          O.encoder_layers(x, W, 2, [0, 1]))
    y8 = O.encoder_layer_mixed_fp8(x, W, 0, 2)
    y = O.encoder_layer(x, W, 0, 2)
    # e4m3 keeps 3 mantissa bits (a rounding error of up to 2^-4 per operand),
    # so the layer moves by some per cent, not by its own size
    rel = np.linalg.norm(y8 - y) / np.linalg.norm(y)
    assert 0 < rel < 0.15


def test_mixed_fp8_sites_use_per_tensor_amax_scales():
    """The layer's fp8 sites equal fp8_linear with amax scales of exactly the
    site's input (one chunk, the oracle's own values, no rounding) and
    weight: recompute the layer from its parts. With act_transform the same
    holds for the transformed inputs (bf16_round: the sensitivity runs)."""
    rng = np.random.default_rng(4)
    W = _tiny_weights(rng, d=64, f=256)
    x = rng.standard_normal((30, 64))
    p = "encoder.blocks.1."
    s = O.e4m3_scale_from_amax
    for tr in (lambda a: a, O.bf16_round):
        a = tr(O.layer_norm(x, W[p + "attn_ln.weight"], W[p + "attn_ln.bias"]))
        q = O.fp8_linear(a, W[p + "attn.query.weight"], W[p + "attn.query.bias"], s(a), s(W[p + "attn.query.weight"]))
        k = O.fp8_linear(a, W[p + "attn.key.weight"], None, s(a), s(W[p + "attn.key.weight"]))
        v = O.fp8_linear(a, W[p + "attn.value.weight"], W[p + "attn.value.bias"], s(a),
                         s(W[p + "attn.value.weight"]))
        h = x + O.linear(O.attention(q, k, v, 2), W[p + "attn.out.weight"], W[p + "attn.out.bias"])
        m = tr(O.layer_norm(h, W[p + "mlp_ln.weight"], W[p + "mlp_ln.bias"]))
        g = tr(O.gelu(O.fp8_linear(m, W[p + "mlp.0.weight"], W[p + "mlp.0.bias"], s(m), s(W[p + "mlp.0.weight"]))))
        out = h + O.fp8_linear(g, W[p + "mlp.2.weight"], W[p + "mlp.2.bias"], s(g), s(W[p + "mlp.2.weight"]))
        got = O.encoder_layer_mixed_fp8(x, W, 1, 2, act_transform=None if tr is not O.bf16_round else O.bf16_round)
        assert np.array_equal(got, out)
    # the rounding moves some codes, so the layer differs
    y0 = O.encoder_layer_mixed_fp8(x, W, 1, 2)
    y1 = O.encoder_layer_mixed_fp8(x, W, 1, 2, act_transform=O.bf16_round)
    assert np.abs(y1 - y0).max() > 0


def test_mixed_fp8_encoder_from_mel_is_stem_then_layers():
    rng = np.random.default_rng(5)
    W = _tiny_weights(rng, d=64, f=256)
    mel = rng.standard_normal((16, 3000)) * 0.3
    want = O.encoder_layers_mixed_fp8(O.conv_stem(mel, W), W, 2, [0, 1], ln_post=True)
    assert np.array_equal(O.encoder_mixed_fp8(mel, W, 2, 2), want)


def test_bf16_round_matches_torch_and_keeps_grid_values():
    rng = np.random.default_rng(9)
    x = np.concatenate([rng.standard_normal(100000) * sc for sc in (1e-3, 1.0, 300.0)])
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.bf16_round(x), ref)
    g = O.e4m3_value(np.arange(127))  # every e4m3 value is a bf16 value
    assert np.array_equal(O.bf16_round(g), g)



def test_fp8_linear_rows_per_row_scales_match_torch_quantiser():
    """The decoder FFN site: each row quantised with its own amax scale
    (fl32(amax) / 448), the weight with its tensor's, against torch's
    float8_e4m3fn conversion of fl32(v * fl32(1/s)); rows are independent."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((6, 96)) * np.array([0.01, 1.0, 30.0, 0.5, 2.0, 200.0])[:, None]
    w, b = rng.standard_normal((40, 96)) * 0.05, rng.standard_normal(40)

    def tq(a, s):
        y = torch.from_numpy(np.asarray(a, np.float32)) * torch.tensor(np.float32(1.0) / np.float32(s))
        return y.to(torch.float8_e4m3fn).to(torch.float64).numpy()

    sw = O.e4m3_scale_from_amax(w)
    got = O.fp8_linear_rows(x, w, b)
    for r in range(x.shape[0]):
        sx = np.float32(np.float32(np.abs(x[r]).max()) / np.float32(448.0))
        ref = (tq(x[r], sx) @ tq(w, sw).T) * (float(sx) * float(sw)) + b
        assert np.allclose(got[r], ref, rtol=1e-13, atol=1e-13), r
    part = O.fp8_linear_rows(x, w, b, rows=[1, 4])
    assert np.array_equal(part[[1, 4]], got[[1, 4]]) and not part[[0, 2, 3, 5]].any()


def test_decode_step_mixed_fp8_ffn_site():
    """decode_step with the decoder FFN in fp8: off is the plain step; on, the
    logits move by the fp8 rounding (some per cent), and rows are
    independent (a subset gives exactly those rows)."""
    from tests.test_oracle_layers import _fp8_setup
    W, H, L, ctx, cross, toks, scales, dh = _fp8_setup()
    B = toks.shape[1]
    c0 = np.zeros((L, 2, B, H, ctx, dh), np.uint8)
    lg, _ = O.decode_step(W, H, toks[0], np.zeros(B, int), c0.copy(), scales, cross)
    lg8, _ = O.decode_step(W, H, toks[0], np.zeros(B, int), c0.copy(), scales, cross, mixed_fp8=True)
    lg8r, _ = O.decode_step(W, H, toks[0], np.zeros(B, int), c0.copy(), scales, cross, rows=[1], mixed_fp8=True)
    rel = np.abs(lg8 - lg).max() / np.abs(lg).max()
    assert 0 < rel < 0.15
    assert np.array_equal(lg8r[1], lg8[1])


def test_decode_step_mixed_fp8_mlp_recomputed_with_torch_quantiser():
    """One decoder layer: the mixed_fp8 step's residual output equals the
    residual entering its MLP (the same step with the MLP weights zeroed)
    plus fc2(GELU(fc1(LN(x)))) recomputed with torch's float8_e4m3fn
    quantiser, each row with its own activation scales and each weight with
    its tensor's (fp64 products of the code values)."""
    from tests.test_oracle_layers import _tiny_weights
    rng = np.random.default_rng(17)
    d, H, V, ctx, Tenc, B = 64, 2, 50, 8, 7, 3
    W = _tiny_weights(rng, d=d, n_dec=1, vocab=V, ctx=ctx)
    p = "decoder.blocks.0."
    W[p + "mlp.0.bias"] = rng.standard_normal(W[p + "mlp.0.bias"].shape) * 0.1
    W[p + "mlp.2.bias"] = rng.standard_normal(W[p + "mlp.2.bias"].shape) * 0.1
    enc = rng.standard_normal((B, Tenc, d))
    cross_b = [O.cross_kv(enc[b], W, H, 1) for b in range(B)]
    cross = [(np.stack([c[0][0] for c in cross_b]), np.stack([c[0][1] for c in cross_b]))]
    toks = rng.integers(0, V, B)
    scales = np.full((1, 2), np.float32(0.03), np.float32)
    W0 = dict(W)
    for k in ("mlp.0.weight", "mlp.0.bias", "mlp.2.weight", "mlp.2.bias"):
        W0[p + k] = np.zeros_like(W[p + k])
    cache = lambda: np.zeros((1, 2, B, H, ctx, d // H), np.uint8)  # noqa: E731
    _, tr0 = O.decode_step(W0, H, toks, np.zeros(B, int), cache(), scales, cross)
    _, tr8 = O.decode_step(W, H, toks, np.zeros(B, int), cache(), scales, cross, mixed_fp8=True)
    x_pre = tr0["x"]

    def tq(a, s):
        y = torch.from_numpy(np.asarray(a, np.float32)) * torch.tensor(np.float32(1.0) / np.float32(s))
        return y.to(torch.float8_e4m3fn).to(torch.float64).numpy()

    def site(a, w, b):
        sw = np.float32(np.float32(np.abs(w).max()) / np.float32(448.0))
        sa = np.float32(np.float32(np.abs(a).max()) / np.float32(448.0))
        return (tq(a, sa) @ tq(w, sw).T) * (float(sa) * float(sw)) + b

    for r in range(B):
        m = O.layer_norm(x_pre[r], W[p + "mlp_ln.weight"], W[p + "mlp_ln.bias"])
        h = O.gelu(site(m, W[p + "mlp.0.weight"], W[p + "mlp.0.bias"]))
        want = x_pre[r] + site(h, W[p + "mlp.2.weight"], W[p + "mlp.2.bias"])
        assert np.allclose(tr8["x"][r], want, rtol=1e-12, atol=1e-12), r
