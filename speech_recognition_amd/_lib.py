"""ctypes binding of libwhisper_mi355x.so: same names and arguments as the C
ABI in include/whisper_mi355x.h; only marshalling happens here.

Pointers may be passed as torch tensors (their data_ptr() is used), plain
ints or None (NULL). `stream` defaults to torch's current stream on the
current device. A non-OK status raises WhisperError with the library's own
message. Loading fails loudly if the library has not been built: there is no
fallback path.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# WHISPER_MI355X_LIB selects another build of the same library (the host
# AddressSanitizer build the CPU tests use)
LIB_PATH = os.environ.get("WHISPER_MI355X_LIB") or os.path.join(_HERE, "libwhisper_mi355x.so")

WHISPER_F32, WHISPER_BF16 = 0, 1
WHISPER_FP8_E4M3, WHISPER_FP8_E5M2 = 0, 1
WS_LOGMEL, WS_ENCODE, WS_CROSS_KV, WS_DECODE, WS_ENCODE_FP8, WS_DECODE_ENC, WS_DECODE_ENC_FP8 = 0, 1, 2, 3, 4, 5, 6

EXPORTS = [
    "whisper_weight_count", "whisper_packed_weights_size", "whisper_pack_weights", "whisper_workspace_size",
    "whisper_logmel", "whisper_encode", "whisper_encode_layers", "whisper_cross_kv", "whisper_decode_step",
    "whisper_decode_step_xq", "whisper_decode_prefill",
    "whisper_fp8_workspace_size", "whisper_fp8_quantize", "whisper_fp8_dequantize", "whisper_layernorm_fused",
    "whisper_linear", "whisper_attention_encoder", "whisper_attention_decode_self",
    "whisper_attention_decode_cross_workspace_size", "whisper_attention_decode_cross",
    "whisper_profile_arm", "whisper_profile_disarm", "whisper_status_string", "whisper_last_error",
    "whisper_peak_mfma", "whisper_peak_mfma_flop", "whisper_peak_read", "whisper_chunk_plan", "whisper_plan_batch",
    "whisper_packed_weights_fp8_size", "whisper_pack_weights_fp8", "whisper_encode_fp8", "whisper_encode_layers_fp8",
    "whisper_gemm_fp8",
    "whisper_logmel_chunked",
    "whisper_decode_linear_workspace_size", "whisper_decode_linear", "whisper_debug_kv_arm",
    "whisper_debug_kv_disarm", "whisper_decode_step_noalloc", "whisper_decode_step_enc", "whisper_decode_prefill_enc",
    "whisper_decode_step_enc_fp8", "whisper_decode_mlp_fp8_workspace_size", "whisper_decode_mlp_fp8",
    "whisper_e4m3_round_host", "whisper_decode_prefill_enc_fp8",
]

DEC_LN_STORE, DEC_LN_GELU, DEC_LN_F32, DEC_LN_QKV, DEC_RESID, DEC_RESID_SPLITK = 0, 1, 2, 3, 4, 5
PROF_DECODE_CROSS_ATTENTION, PROF_DECODE_SELF_ATTENTION, PROF_ENCODER_ATTENTION = 1, 2, 3
PROF_ENCODER_FFN1, PROF_ENCODER_LAYERNORM = 4, 5


class WhisperError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"whisper status {status}: {msg}")
        self.status = status


class WhisperDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in (
        "n_mels", "n_audio_ctx", "d_model", "n_heads", "head_dim", "d_ffn",
        "n_enc_layers", "n_dec_layers", "n_vocab", "n_text_ctx", "act")]


class WhisperBatchPlan(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int), ("peak_stage", ctypes.c_int)] + [
        (n, ctypes.c_size_t) for n in ("weights", "workspace", "audio", "mel", "encoder_out", "cross_kv",
                                       "cross_codes", "kv_cache", "decode_state", "logits")] + [
        ("stage", ctypes.c_size_t * 5), ("total", ctypes.c_size_t)]


PLAN_STAGES = ("logmel", "encode", "cross_kv", "quantise", "decode")


def make_dims(d):
    """WhisperDims from a workload Dims-like object (or pass a WhisperDims)."""
    if isinstance(d, WhisperDims):
        return d
    return WhisperDims(d.n_mels, d.n_audio_ctx, d.d_model, d.n_heads, d.head_dim, d.d_ffn,
                       d.n_enc_layers, d.n_dec_layers, d.n_vocab, d.n_text_ctx,
                       WHISPER_BF16 if d.act == "bf16" else WHISPER_F32)


_lib = None
P, I, Z, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
_SIG = {
    "whisper_weight_count": (I, [P]),
    "whisper_packed_weights_size": (Z, [P]),
    "whisper_pack_weights": (I, [P, P, P, P]),
    "whisper_workspace_size": (Z, [P, I, I]),
    "whisper_logmel": (I, [P, P, I, I, P, P, Z, P]),
    "whisper_encode": (I, [P, P, P, I, P, P, Z, P]),
    "whisper_encode_layers": (I, [P, P, P, I, I, I, I, P, P, Z, P]),
    "whisper_cross_kv": (I, [P, P, P, I, P, P, Z, P]),
    "whisper_decode_step": (I, [P, P, I, I, P, P, P, P, P, P, P, P, P, Z, P]),
    "whisper_decode_step_xq": (I, [P, P, I, I, P, P, P, P, P, P, I, P, P, P, P, Z, P]),
    "whisper_decode_step_noalloc": (I, [P, P, I, I, P, P, P, P, P, P, P, P, P]),
    "whisper_decode_step_enc": (I, [P, P, I, I, P, P, P, P, P, P, P, P, P, Z, P]),
    "whisper_decode_step_enc_fp8": (I, [P, P, P, I, I, P, P, P, P, P, P, P, P, P, Z, P]),
    "whisper_decode_prefill_enc": (I, [P, P, I, I, I, P, P, P, P, P, P, P, P, P, Z, P]),
    "whisper_decode_prefill": (I, [P, P, I, I, I, P, P, P, P, P, P, P, P, P, Z, P]),
    "whisper_fp8_workspace_size": (Z, []),
    "whisper_fp8_quantize": (I, [P, I, I, Z, P, P, P, P, Z, P]),
    "whisper_fp8_dequantize": (I, [P, I, Z, P, P, I, P]),
    "whisper_layernorm_fused": (I, [P, P, P, P, P, F, I, P, P, P]),
    "whisper_linear": (I, [I, P, I, P, P, I, I, I, I, P, I, P]),
    "whisper_attention_encoder": (I, [I, P, I, I, I, P, P]),
    "whisper_attention_decode_self": (I, [I, P, I, I, I, P, P, P, P, P, P]),
    "whisper_attention_decode_cross_workspace_size": (Z, [I, I, I]),
    "whisper_attention_decode_cross": (I, [I, P, P, P, I, I, I, P, P, Z, P]),
    "whisper_chunk_plan": (I, [ctypes.c_int64, I, P, I]),
    "whisper_plan_batch": (I, [P, Z, I, I, I, I, I, P]),
    "whisper_packed_weights_fp8_size": (Z, [P]),
    "whisper_pack_weights_fp8": (I, [P, P, P, P, Z, P]),
    "whisper_encode_fp8": (I, [P, P, P, P, I, P, P, Z, P]),
    "whisper_encode_layers_fp8": (I, [P, P, P, P, I, I, I, I, P, P, Z, P]),
    "whisper_gemm_fp8": (I, [P, I, I, P, I, P, I, P, P, I, P, ctypes.c_long, P]),
    "whisper_logmel_chunked": (I, [P, P, ctypes.c_int64, I, P, P, Z, P]),
    "whisper_peak_mfma": (I, [I, I, P, P]),
    "whisper_peak_mfma_flop": (ctypes.c_double, [I, I]),
    "whisper_peak_read": (I, [P, Z, I, P, P]),
    "whisper_decode_linear_workspace_size": (Z, [I, I, I, I]),
    "whisper_decode_linear": (I, [I, I, I, I, P, P, P, P, P, P, P, P, P, P, I, P, P, Z, P]),
    "whisper_decode_mlp_fp8_workspace_size": (Z, [I, I, I]),
    "whisper_decode_mlp_fp8": (I, [I, I, I, P, P, P, P, P, P, P, P, P, P, Z, P]),
    "whisper_e4m3_round_host": (I, [P, P, Z]),
    "whisper_decode_prefill_enc_fp8": (I, [P, P, P, I, I, I, P, P, P, P, P, P, P, P, P, Z, P]),
    "whisper_debug_kv_arm": (I, [P, P, Z]),
    "whisper_debug_kv_disarm": (None, []),
    "whisper_profile_arm": (I, [I, P, P, I]),
    "whisper_profile_disarm": (I, []),
    "whisper_status_string": (ctypes.c_char_p, [I]),
    "whisper_last_error": (ctypes.c_char_p, []),
}


def lib():
    """Load the library (once). Raises if it is missing: build it first."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run speech_recognition_amd/build.py "
                              "(or __graft_entry__.build()) first")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIG.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _p(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _dtype_check(name, t, dt):
    """A torch tensor passed where the call's whisper_dtype fixes the element
    type must have that type (a silent mismatch reinterprets the bytes)."""
    if t is None or isinstance(t, int) or not hasattr(t, "dtype"):
        return
    import torch
    want = {WHISPER_F32: torch.float32, WHISPER_BF16: torch.bfloat16}.get(dt)
    if want is not None and t.dtype != want:
        raise WhisperError(3, f"{name}: tensor dtype {t.dtype} does not match whisper dtype {want}")


def _stream(s):
    if s is not None:
        return s if isinstance(s, int) else s.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(status):
    if status != 0:
        raise WhisperError(status, lib().whisper_last_error().decode())


def _dims_ptr(d):
    dd = make_dims(d)
    return dd, ctypes.byref(dd)


# ------------------------------------------------------------------ size queries
def whisper_weight_count(dims):
    dd, dp = _dims_ptr(dims)
    return lib().whisper_weight_count(dp)


def whisper_packed_weights_size(dims):
    dd, dp = _dims_ptr(dims)
    return lib().whisper_packed_weights_size(dp)


def whisper_workspace_size(dims, batch, which):
    dd, dp = _dims_ptr(dims)
    return lib().whisper_workspace_size(dp, batch, which)


def whisper_fp8_workspace_size():
    return lib().whisper_fp8_workspace_size()


def whisper_attention_decode_cross_workspace_size(batch, n_heads, T):
    return lib().whisper_attention_decode_cross_workspace_size(batch, n_heads, T)


# ------------------------------------------------------------------ calls
def whisper_pack_weights(dims, logical, packed, stream=None):
    """logical: sequence of fp32 device tensors (or pointers) in the ABI's order."""
    dd, dp = _dims_ptr(dims)
    arr = (ctypes.c_void_p * len(logical))(*[_p(t) for t in logical])
    _check(lib().whisper_pack_weights(dp, arr, _p(packed), _stream(stream)))


def whisper_logmel(dims, audio, batch, n_samples, mel_out, ws, ws_bytes, stream=None):
    dd, dp = _dims_ptr(dims)
    _check(lib().whisper_logmel(dp, _p(audio), batch, n_samples, _p(mel_out), _p(ws), ws_bytes, _stream(stream)))


def whisper_encode(dims, packed, mel, batch, enc_out, ws, ws_bytes, stream=None):
    dd, dp = _dims_ptr(dims)
    _check(lib().whisper_encode(dp, _p(packed), _p(mel), batch, _p(enc_out), _p(ws), ws_bytes, _stream(stream)))


def whisper_encode_layers(dims, packed, h_in, batch, layer_begin, layer_end, apply_ln_post, h_out, ws, ws_bytes,
                          stream=None):
    dd, dp = _dims_ptr(dims)
    _check(lib().whisper_encode_layers(dp, _p(packed), _p(h_in), batch, layer_begin, layer_end, int(apply_ln_post),
                                       _p(h_out), _p(ws), ws_bytes, _stream(stream)))


def whisper_cross_kv(dims, packed, enc_out, batch, cross_kv, ws=None, ws_bytes=0, stream=None):
    dd, dp = _dims_ptr(dims)
    _check(lib().whisper_cross_kv(dp, _p(packed), _p(enc_out), batch, _p(cross_kv), _p(ws), ws_bytes,
                                  _stream(stream)))


def whisper_decode_step(dims, packed, batch, kv_cap, tokens, lengths, kv_cache, kv_scales, cross_kv, logits, argmax,
                        dev_error, ws, ws_bytes, stream=None):
    dd, dp = _dims_ptr(dims)
    _check(lib().whisper_decode_step(dp, _p(packed), batch, kv_cap, _p(tokens), _p(lengths), _p(kv_cache),
                                     _p(kv_scales), _p(cross_kv), _p(logits), _p(argmax), _p(dev_error), _p(ws),
                                     ws_bytes, _stream(stream)))


def whisper_decode_step_noalloc(dims, packed, batch, kv_cap, tokens, lengths, kv_cache, kv_scales, cross_kv, logits,
                                argmax, dev_error, stream=None):
    dd, dp = _dims_ptr(dims)
    _check(lib().whisper_decode_step_noalloc(dp, _p(packed), batch, kv_cap, _p(tokens), _p(lengths), _p(kv_cache),
                                             _p(kv_scales), _p(cross_kv), _p(logits), _p(argmax), _p(dev_error),
                                             _stream(stream)))


def whisper_decode_step_enc(dims, packed, batch, kv_cap, tokens, lengths, kv_cache, kv_scales, enc_out, logits, argmax,
                            dev_error, ws, ws_bytes, stream=None):
    dd, dp = _dims_ptr(dims)
    _check(lib().whisper_decode_step_enc(dp, _p(packed), batch, kv_cap, _p(tokens), _p(lengths), _p(kv_cache),
                                         _p(kv_scales), _p(enc_out), _p(logits), _p(argmax), _p(dev_error), _p(ws),
                                         ws_bytes, _stream(stream)))


def whisper_decode_step_enc_fp8(dims, packed, packed8, batch, kv_cap, tokens, lengths, kv_cache, kv_scales, enc_out,
                                logits, argmax, dev_error, ws, ws_bytes, stream=None):
    dd, dp = _dims_ptr(dims)
    _check(lib().whisper_decode_step_enc_fp8(dp, _p(packed), _p(packed8), batch, kv_cap, _p(tokens), _p(lengths),
                                             _p(kv_cache), _p(kv_scales), _p(enc_out), _p(logits), _p(argmax),
                                             _p(dev_error), _p(ws), ws_bytes, _stream(stream)))


def whisper_decode_prefill_enc(dims, packed, batch, n_tokens, kv_cap, tokens, lengths, kv_cache, kv_scales, enc_out,
                               logits, argmax, dev_error, ws, ws_bytes, stream=None):
    dd, dp = _dims_ptr(dims)
    _check(lib().whisper_decode_prefill_enc(dp, _p(packed), batch, n_tokens, kv_cap, _p(tokens), _p(lengths),
                                            _p(kv_cache), _p(kv_scales), _p(enc_out), _p(logits), _p(argmax),
                                            _p(dev_error), _p(ws), ws_bytes, _stream(stream)))


def whisper_decode_prefill_enc_fp8(dims, packed, packed8, batch, n_tokens, kv_cap, tokens, lengths, kv_cache,
                                   kv_scales, enc_out, logits, argmax, dev_error, ws, ws_bytes, stream=None):
    dd, dp = _dims_ptr(dims)
    _check(lib().whisper_decode_prefill_enc_fp8(dp, _p(packed), _p(packed8), batch, n_tokens, kv_cap, _p(tokens),
                                                _p(lengths), _p(kv_cache), _p(kv_scales), _p(enc_out), _p(logits),
                                                _p(argmax), _p(dev_error), _p(ws), ws_bytes, _stream(stream)))


def whisper_decode_prefill(dims, packed, batch, n_tokens, kv_cap, tokens, lengths, kv_cache, kv_scales, cross_kv,
                           logits, argmax, dev_error, ws, ws_bytes, stream=None):
    dd, dp = _dims_ptr(dims)
    _check(lib().whisper_decode_prefill(dp, _p(packed), batch, n_tokens, kv_cap, _p(tokens), _p(lengths),
                                        _p(kv_cache), _p(kv_scales), _p(cross_kv), _p(logits), _p(argmax),
                                        _p(dev_error), _p(ws), ws_bytes, _stream(stream)))


def whisper_decode_step_xq(dims, packed, batch, kv_cap, tokens, lengths, kv_cache, kv_scales, cross_codes,
                           cross_scales, logits, argmax, dev_error, ws, ws_bytes, stream=None,
                           cross_format=WHISPER_FP8_E4M3):
    dd, dp = _dims_ptr(dims)
    _check(lib().whisper_decode_step_xq(dp, _p(packed), batch, kv_cap, _p(tokens), _p(lengths), _p(kv_cache),
                                        _p(kv_scales), _p(cross_codes), _p(cross_scales), cross_format,
                                        _p(logits), _p(argmax), _p(dev_error), _p(ws), ws_bytes, _stream(stream)))


def whisper_fp8_quantize(x, dt, n, scale_in, codes, scale_out, ws=None, ws_bytes=0, stream=None,
                         fmt=WHISPER_FP8_E4M3):
    _dtype_check("whisper_fp8_quantize x", x, dt)
    _check(lib().whisper_fp8_quantize(_p(x), dt, fmt, n, _p(scale_in), _p(codes), _p(scale_out), _p(ws), ws_bytes,
                                      _stream(stream)))


def whisper_fp8_dequantize(codes, n, scale, y, dt, stream=None, fmt=WHISPER_FP8_E4M3):
    _dtype_check("whisper_fp8_dequantize y", y, dt)
    _check(lib().whisper_fp8_dequantize(_p(codes), fmt, n, _p(scale), _p(y), dt, _stream(stream)))


def whisper_layernorm_fused(dims, h, residual, gamma, beta, eps, M, normed, total, stream=None):
    dd, dp = _dims_ptr(dims)
    _check(lib().whisper_layernorm_fused(dp, _p(h), _p(residual), _p(gamma), _p(beta), eps, M, _p(normed),
                                         _p(total), _stream(stream)))


def whisper_linear(dt, x, lda, w, bias, M, N, K, act, y, path=0, stream=None):
    for nm, t in (("x", x), ("w", w), ("y", y)):
        _dtype_check("whisper_linear " + nm, t, dt)
    _check(lib().whisper_linear(dt, _p(x), lda, _p(w), _p(bias), M, N, K, act, _p(y), path, _stream(stream)))


def whisper_attention_encoder(dt, qkv, batch, T, n_heads, out, stream=None):
    _dtype_check("whisper_attention_encoder qkv", qkv, dt)
    _dtype_check("whisper_attention_encoder out", out, dt)
    _check(lib().whisper_attention_encoder(dt, _p(qkv), batch, T, n_heads, _p(out), _stream(stream)))


def whisper_attention_decode_self(dt, q, batch, n_heads, cap, k_codes, v_codes, scales, n_keys, out, stream=None):
    _dtype_check("whisper_attention_decode_self q", q, dt)
    _dtype_check("whisper_attention_decode_self out", out, dt)
    _check(lib().whisper_attention_decode_self(dt, _p(q), batch, n_heads, cap, _p(k_codes), _p(v_codes),
                                               _p(scales), _p(n_keys), _p(out), _stream(stream)))


def whisper_attention_decode_cross(dt, q, k, v, batch, n_heads, T, out, ws, ws_bytes, stream=None):
    for nm, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        _dtype_check("whisper_attention_decode_cross " + nm, t, dt)
    _check(lib().whisper_attention_decode_cross(dt, _p(q), _p(k), _p(v), batch, n_heads, T, _p(out), _p(ws),
                                                ws_bytes, _stream(stream)))


def whisper_profile_arm(kind, start_events, stop_events):
    """start_events / stop_events: sequences of torch.cuda.Event (recorded once
    beforehand so the handles exist) or raw hipEvent_t ints; kept alive by
    the caller until disarm."""
    n = len(start_events)
    h = lambda e: e if isinstance(e, int) else e.cuda_event  # noqa: E731
    starts = (ctypes.c_void_p * n)(*[h(e) for e in start_events])
    stops = (ctypes.c_void_p * n)(*[h(e) for e in stop_events])
    whisper_profile_arm._keep = (starts, stops)
    _check(lib().whisper_profile_arm(kind, starts, stops, n))


def whisper_profile_disarm():
    n = lib().whisper_profile_disarm()
    whisper_profile_arm._keep = None
    return n


def whisper_decode_linear_workspace_size(mode, M, N, K):
    return lib().whisper_decode_linear_workspace_size(mode, M, N, K)


def whisper_decode_linear(mode, M, N, K, x, a, w, bias, gamma, beta, y, kv_cache=None, kv_scales=None,
                          lengths=None, kv_cap=0, dev_error=None, ws=None, ws_bytes=0, stream=None):
    _check(lib().whisper_decode_linear(mode, M, N, K, _p(x), _p(a), _p(w), _p(bias), _p(gamma), _p(beta), _p(y),
                                       _p(kv_cache), _p(kv_scales), _p(lengths), kv_cap, _p(dev_error), _p(ws),
                                       ws_bytes, _stream(stream)))


def whisper_decode_mlp_fp8_workspace_size(M, d, f):
    return lib().whisper_decode_mlp_fp8_workspace_size(M, d, f)


def whisper_decode_mlp_fp8(M, d, f, x, gamma, beta, w1, b1, w2, b2, hidden=None, hidden_amax=None, ws=None,
                           ws_bytes=0, stream=None):
    _check(lib().whisper_decode_mlp_fp8(M, d, f, _p(x), _p(gamma), _p(beta), _p(w1), _p(b1), _p(w2), _p(b2),
                                        _p(hidden), _p(hidden_amax), _p(ws), ws_bytes, _stream(stream)))


def whisper_e4m3_round_host(x):
    """x: a C-contiguous float32 numpy array; returns the rounded values."""
    import numpy as np
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty_like(x)
    _check(lib().whisper_e4m3_round_host(x.ctypes.data, y.ctypes.data, x.size))
    return y


def whisper_debug_kv_arm(kv_pre, kv_force, n_elems):
    """kv_pre (fp32) and kv_force (int16): device tensors or None, kept alive
    by the caller until disarm."""
    _check(lib().whisper_debug_kv_arm(_p(kv_pre), _p(kv_force), n_elems))


def whisper_debug_kv_disarm():
    lib().whisper_debug_kv_disarm()


def whisper_status_string(status):
    return lib().whisper_status_string(status).decode()


def whisper_last_error():
    return lib().whisper_last_error().decode()


# ------------------------------------------------------------------ measured ceilings
def whisper_peak_mfma(n_wg, iters, out, stream=None):
    _check(lib().whisper_peak_mfma(n_wg, iters, _p(out), _stream(stream)))


def whisper_peak_mfma_flop(n_wg, iters):
    return lib().whisper_peak_mfma_flop(n_wg, iters)


def whisper_peak_read(buf, nbytes, n_wg, out, stream=None):
    _check(lib().whisper_peak_read(_p(buf), nbytes, n_wg, _p(out), _stream(stream)))


# ------------------------------------------------------------------ overlapping chunks of a long recording
def whisper_chunk_plan(n_samples, stride):
    """(count, plan) with plan a list of (first sample, valid samples, first owned frame, end of owned frames)."""
    n = lib().whisper_chunk_plan(n_samples, stride, None, 0)
    if n <= 0:
        raise WhisperError(1, "chunk_plan: need n_samples > 0 and stride in 160..480000, a multiple of 160")
    buf = (ctypes.c_int32 * (4 * n))()
    lib().whisper_chunk_plan(n_samples, stride, buf, n)
    return n, [tuple(buf[4 * i:4 * i + 4]) for i in range(n)]


def whisper_packed_weights_fp8_size(dims):
    dd, dp = _dims_ptr(dims)
    return lib().whisper_packed_weights_fp8_size(dp)


def whisper_pack_weights_fp8(dims, logical, packed8, ws, ws_bytes, stream=None):
    dd, dp = _dims_ptr(dims)
    arr = (ctypes.c_void_p * len(logical))(*[_p(t) for t in logical])
    _check(lib().whisper_pack_weights_fp8(dp, arr, _p(packed8), _p(ws), ws_bytes, _stream(stream)))


def whisper_encode_fp8(dims, packed, packed8, mel, batch, enc_out, ws, ws_bytes, stream=None):
    dd, dp = _dims_ptr(dims)
    _check(lib().whisper_encode_fp8(dp, _p(packed), _p(packed8), _p(mel), batch, _p(enc_out), _p(ws), ws_bytes,
                                    _stream(stream)))


def whisper_encode_layers_fp8(dims, packed, packed8, h_in, batch, l0, l1, ln_post, h_out, ws, ws_bytes,
                              stream=None):
    dd, dp = _dims_ptr(dims)
    _check(lib().whisper_encode_layers_fp8(dp, _p(packed), _p(packed8), _p(h_in), batch, l0, l1, int(bool(ln_post)),
                                           _p(h_out), _p(ws), ws_bytes, _stream(stream)))


def whisper_gemm_fp8(a, M, K, a_scales, rows_per_scale, w, N, w_scale, bias, gelu, c, ldc, stream=None):
    _check(lib().whisper_gemm_fp8(_p(a), M, K, _p(a_scales), rows_per_scale, _p(w), N, _p(w_scale), _p(bias),
                                  int(bool(gelu)), _p(c), ldc, _stream(stream)))


def whisper_plan_batch(dims, budget_bytes, kv_cap, prompt_tokens=0, cross_fp8=False, want_logits=False,
                       max_batch=4096):
    """Largest batch whose one-pass footprint fits budget_bytes, with the
    footprint breakdown, as a dict (raises WhisperError with status 6 when one
    chunk does not fit)."""
    dd, dp = _dims_ptr(dims)
    plan = WhisperBatchPlan()
    _check(lib().whisper_plan_batch(dp, budget_bytes, kv_cap, prompt_tokens, int(bool(cross_fp8)),
                                    int(bool(want_logits)), max_batch, ctypes.byref(plan)))
    out = {n: getattr(plan, n) for n, _ in WhisperBatchPlan._fields_ if n != "stage"}
    out["stage"] = dict(zip(PLAN_STAGES, list(plan.stage)))
    out["peak_stage"] = PLAN_STAGES[plan.peak_stage]
    return out


def whisper_logmel_chunked(dims, audio, n_samples, stride, mel_out, ws, ws_bytes, stream=None):
    dd, dp = _dims_ptr(dims)
    _check(lib().whisper_logmel_chunked(dp, _p(audio), n_samples, stride, _p(mel_out), _p(ws), ws_bytes,
                                        _stream(stream)))
