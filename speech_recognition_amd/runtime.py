"""Device-buffer plumbing around the C ABI.

torch provides device memory and the stream; every step of the hot path runs
in the library's HIP kernels through the ctypes binding. The helpers here
only size and allocate buffers and pass pointers.
"""
import torch

from . import _lib as L

__all__ = ["Whisper", "DecodeState", "act_dtype"]


def act_dtype(dims):
    return torch.bfloat16 if dims.act == "bf16" else torch.float32


def _empty_bytes(n, device):
    return torch.empty(max(int(n), 256), dtype=torch.uint8, device=device)


class Whisper:
    """Packed weights plus per-call workspaces for one model shape."""

    def __init__(self, dims, logical_weights, device="cuda", mixed_fp8=False):
        """logical_weights: fp32 device tensors in the ABI's canonical order.
        mixed_fp8: also pack the E4M3 weights of the mixed_fp8 sites (encoder
        query/key/value and MLP: encode_fp8 / encode_layers_fp8; decoder MLP:
        decode_step with a DecodeState made with ffn_fp8=True)."""
        self.dims = dims
        self.device = torch.device(device)
        n = L.whisper_weight_count(dims)
        if n != len(logical_weights):
            raise ValueError(f"expected {n} weight tensors, got {len(logical_weights)}")
        for t in logical_weights:
            if t.dtype != torch.float32 or not t.is_contiguous() or t.device.type != "cuda":
                raise ValueError("logical weights must be contiguous fp32 device tensors")
        self.packed = _empty_bytes(L.whisper_packed_weights_size(dims), self.device)
        L.whisper_pack_weights(dims, logical_weights, self.packed)
        self.packed8 = None
        if mixed_fp8:
            self.packed8 = _empty_bytes(L.whisper_packed_weights_fp8_size(dims), self.device)
            ws = torch.empty(L.whisper_fp8_workspace_size(), dtype=torch.uint8, device=self.device)
            L.whisper_pack_weights_fp8(dims, logical_weights, self.packed8, ws, ws.numel())
        self._ws = None

    def workspace(self, batch, which):
        """The model's one workspace, grown to the largest size asked so far.
        Calls are ordered on one stream, so every stage reuses the same
        buffer (the schedule whisper_plan_batch sizes)."""
        nbytes = L.whisper_workspace_size(self.dims, batch, which)
        if self._ws is None or self._ws.numel() < nbytes:
            self._ws = None
            self._ws = _empty_bytes(nbytes, self.device)
        return self._ws, nbytes

    def reserve_workspace(self, nbytes):
        """Allocate the shared workspace up front (e.g. a plan's workspace size)."""
        if self._ws is None or self._ws.numel() < nbytes:
            self._ws = None
            self._ws = _empty_bytes(nbytes, self.device)

    def plan_batch(self, budget_bytes, kv_cap, prompt_tokens=0, cross_fp8=False, want_logits=False,
                   max_batch=4096):
        """Largest batch of 30 s chunks whose pass fits budget_bytes (whisper_plan_batch)."""
        return L.whisper_plan_batch(self.dims, budget_bytes, kv_cap, prompt_tokens, cross_fp8, want_logits,
                                    max_batch)

    # ---------------------------------------------------------------- stages
    def logmel(self, audio, out=None):
        B, n = audio.shape
        mel = out if out is not None else torch.empty(B, self.dims.n_mels, 3000, dtype=torch.float32,
                                                      device=self.device)
        ws, nb = self.workspace(B, L.WS_LOGMEL)
        L.whisper_logmel(self.dims, audio, B, n, mel, ws, nb)
        return mel

    def encode(self, mel, out=None):
        B = mel.shape[0]
        enc = out if out is not None else torch.empty(B, self.dims.n_audio_ctx, self.dims.d_model,
                                                      dtype=act_dtype(self.dims), device=self.device)
        ws, nb = self.workspace(B, L.WS_ENCODE)
        L.whisper_encode(self.dims, self.packed, mel, B, enc, ws, nb)
        return enc

    def encode_fp8(self, mel, out=None):
        """encode with the mixed_fp8 sites in E4M3 (needs mixed_fp8=True)."""
        B = mel.shape[0]
        enc = out if out is not None else torch.empty(B, self.dims.n_audio_ctx, self.dims.d_model,
                                                      dtype=act_dtype(self.dims), device=self.device)
        ws, nb = self.workspace(B, L.WS_ENCODE_FP8)
        L.whisper_encode_fp8(self.dims, self.packed, self.packed8, mel, B, enc, ws, nb)
        return enc

    def encode_layers_fp8(self, h, layer_begin, layer_end, ln_post=False, out=None):
        B = h.shape[0]
        o = out if out is not None else torch.empty_like(h)
        ws, nb = self.workspace(B, L.WS_ENCODE_FP8)
        L.whisper_encode_layers_fp8(self.dims, self.packed, self.packed8, h, B, layer_begin, layer_end, ln_post, o,
                                    ws, nb)
        return o

    def encode_layers(self, h, layer_begin, layer_end, ln_post=False, out=None):
        B = h.shape[0]
        o = out if out is not None else torch.empty_like(h)
        ws, nb = self.workspace(B, L.WS_ENCODE)
        L.whisper_encode_layers(self.dims, self.packed, h, B, layer_begin, layer_end, ln_post, o, ws, nb)
        return o

    def cross_kv(self, enc, out=None):
        B = enc.shape[0]
        d = self.dims
        ckv = out if out is not None else torch.empty(d.n_dec_layers, 2, B, d.n_heads, d.n_audio_ctx, 64,
                                                      dtype=act_dtype(d), device=self.device)
        L.whisper_cross_kv(d, self.packed, enc, B, ckv)
        return ckv

    def quantize_cross_kv(self, ckv, scales=None, codes=None, fmt=L.WHISPER_FP8_E4M3):
        """fp8 codes (fmt: WHISPER_FP8_E4M3 or WHISPER_FP8_E5M2) of bf16 cross K/V
        [L, 2, B, H, T, 64], one scale per (layer, K|V) slab: the given scales
        [L, 2], or amax / (448 or 57344) of each slab when None.
        Returns (codes uint8 of the same shape, scales fp32 [L, 2] on the device)."""
        n_l = ckv.shape[0]
        codes = codes if codes is not None else torch.empty(ckv.shape, dtype=torch.uint8, device=ckv.device)
        sc = torch.zeros(n_l, 2, dtype=torch.float32, device=ckv.device)
        if scales is not None:
            sc.copy_(torch.as_tensor(scales, dtype=torch.float32))
        ws = None if scales is not None else torch.empty(L.whisper_fp8_workspace_size(), dtype=torch.uint8,
                                                         device=ckv.device)
        n = ckv[0, 0].numel()
        for l in range(n_l):
            for kv in range(2):
                if scales is not None:
                    L.whisper_fp8_quantize(ckv[l, kv], L.WHISPER_BF16, n, sc[l, kv:kv + 1], codes[l, kv], None,
                                           fmt=fmt)
                else:
                    L.whisper_fp8_quantize(ckv[l, kv], L.WHISPER_BF16, n, None, codes[l, kv], sc[l, kv:kv + 1],
                                           ws, ws.numel(), fmt=fmt)
        return codes, sc

    def decode_prefill(self, state, tokens, logits=None):
        """tokens [B, P]: P prompt tokens per row in one pass (equal to P decode steps)."""
        B, n_tok = tokens.shape
        assert B == state.batch and state.cross_codes is None
        if state.ffn_fp8:
            if self.packed8 is None or state.enc is None:
                raise ValueError("the fp8 MLP sites need mixed_fp8=True and a state over the encoder output")
            ws, nb = self.workspace(B * n_tok, L.WS_DECODE_ENC_FP8)
            L.whisper_decode_prefill_enc_fp8(self.dims, self.packed, self.packed8, B, n_tok, state.cap,
                                             tokens.contiguous(), state.lengths, state.kv_cache, state.kv_scales,
                                             state.enc, logits, state.argmax, state.dev_error, ws, nb)
            return state.argmax
        if state.enc is not None:
            ws, nb = self.workspace(B * n_tok, L.WS_DECODE_ENC)
            L.whisper_decode_prefill_enc(self.dims, self.packed, B, n_tok, state.cap, tokens.contiguous(),
                                         state.lengths, state.kv_cache, state.kv_scales, state.enc, logits,
                                         state.argmax, state.dev_error, ws, nb)
            return state.argmax
        ws, nb = self.workspace(B * n_tok, L.WS_DECODE)
        L.whisper_decode_prefill(self.dims, self.packed, B, n_tok, state.cap, tokens.contiguous(), state.lengths,
                                 state.kv_cache, state.kv_scales, state.cross_kv, logits, state.argmax,
                                 state.dev_error, ws, nb)
        return state.argmax

    def decode_step(self, state, tokens, logits=None):
        B = state.batch
        if state.ffn_fp8:
            if self.packed8 is None or state.enc is None:
                raise ValueError("the fp8 MLP sites need mixed_fp8=True and a state over the encoder output")
            ws, nb = self.workspace(B, L.WS_DECODE_ENC_FP8)
            L.whisper_decode_step_enc_fp8(self.dims, self.packed, self.packed8, B, state.cap, tokens, state.lengths,
                                          state.kv_cache, state.kv_scales, state.enc, logits, state.argmax,
                                          state.dev_error, ws, nb)
            return state.argmax
        if state.enc is not None:
            ws, nb = self.workspace(B, L.WS_DECODE_ENC)
            L.whisper_decode_step_enc(self.dims, self.packed, B, state.cap, tokens, state.lengths, state.kv_cache,
                                      state.kv_scales, state.enc, logits, state.argmax, state.dev_error, ws, nb)
            return state.argmax
        ws, nb = self.workspace(B, L.WS_DECODE)
        if state.cross_codes is not None:
            L.whisper_decode_step_xq(self.dims, self.packed, B, state.cap, tokens, state.lengths, state.kv_cache,
                                     state.kv_scales, state.cross_codes, state.cross_scales, logits, state.argmax,
                                     state.dev_error, ws, nb, cross_format=state.cross_format)
        else:
            L.whisper_decode_step(self.dims, self.packed, B, state.cap, tokens, state.lengths, state.kv_cache,
                                  state.kv_scales, state.cross_kv, logits, state.argmax, state.dev_error, ws, nb)
        return state.argmax


class DecodeState:
    """Caller-owned decode state: fp8 self-KV cache, scales, lengths, and the
    cross-attention source: cross K/V (bf16, or fp8 codes in cross_format
    with per-(layer, K|V) scales from quantize_cross_kv), or the encoder
    output itself (enc, [B, 1500, d] bf16: decode_step_enc). ffn_fp8: the
    decoder MLP as mixed_fp8 sites (decode_step_enc_fp8; needs enc)."""

    def __init__(self, dims, batch, cap, cross_kv, kv_scales, lengths, device="cuda", cross_codes=None,
                 cross_scales=None, cross_format=L.WHISPER_FP8_E4M3, enc=None, ffn_fp8=False):
        self.batch, self.cap = batch, cap
        self.kv_cache = torch.zeros(dims.n_dec_layers, 2, batch, dims.n_heads, cap, 64, dtype=torch.uint8,
                                    device=device)
        self.kv_scales = kv_scales.to(device=device, dtype=torch.float32).contiguous()
        self.lengths = lengths.to(device=device, dtype=torch.int32).contiguous().clone()
        self.cross_kv = cross_kv
        self.enc = enc
        self.ffn_fp8 = ffn_fp8
        self.cross_codes, self.cross_scales = cross_codes, cross_scales
        self.cross_format = cross_format
        self.argmax = torch.zeros(batch, dtype=torch.int32, device=device)
        self.dev_error = torch.zeros(4, dtype=torch.int32, device=device)
