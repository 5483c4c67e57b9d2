/*
 * whisper_mi355x.h — C ABI of the Whisper large-v3 inference hot path on
 * MI355X (gfx950): log-mel front end, encoder, cross-attention K/V, and the
 * batched decoder step over a caller-owned fp8 (OCP E4M3) self-attention KV
 * cache.
 *
 * Sources. The calls follow the problem as the pages state it:
 *  - whisper_blaze showcase page ("Hopper-Native CUDA Kernels for Whisper"),
 *    "The Solution": the five kernels (GEMM, flash attention for encoder self /
 *    decoder causal self / decoder cross attention, GPU mel spectrogram,
 *    fused residual+LayerNorm, fp8 quantise with per-tensor scales), and the
 *    "Using it" direct kernel calls (quantise_e4m3, layernorm_fused,
 *    decoder_self_attn, mel_spectrogram);
 *  - whisper-blaze project page, "Direct Kernel API": quantise_e4m3 returns
 *    codes and a per-tensor scale, dequantise_e4m3 takes codes, scale, shape;
 *    layernorm_fused_residual returns (normed, total);
 *  - "Blazingly fast whisper transcriptions with Inference Endpoints",
 *    "Inference Stack": compute in bfloat16, KV cache stored as float8 (one
 *    byte per element), quantised on the way in.
 *
 * Conventions (all entry points):
 *  - Every pointer argument is device memory owned by the caller unless
 *    stated otherwise; the library never allocates, frees or retains caller
 *    memory and keeps no state between calls apart from thread-local error
 *    text and the optional measurement and K/V debug hooks below.
 *  - `stream` is a hipStream_t passed as void* (NULL = default stream). Work
 *    is enqueued asynchronously; no call synchronises.
 *  - Argument, shape, dtype, alignment (16 bytes for tensors and workspaces;
 *    4 bytes for the int32 token / length / argmax / key-count arrays, the
 *    fp32 scale arrays and the device error word) and workspace-size checks
 *    run before any launch; a failing check returns a
 *    status and launches nothing. Launch failures return WHISPER_ERR_HIP.
 *    Nothing throws or aborts across the ABI. whisper_last_error() returns
 *    text for the last failure on the calling thread.
 *  - Activations that feed a GEMM or attention are stored in `dims->act`
 *    (bf16 or fp32); the residual stream between blocks, accumulation,
 *    softmax and LayerNorm statistics are fp32; logits are fp32.
 *  - Concurrent calls that share a workspace or output buffer race; calls on
 *    distinct buffers may run on distinct streams.
 */
#ifndef WHISPER_MI355X_H
#define WHISPER_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  WHISPER_OK = 0,
  WHISPER_ERR_INVALID_ARG = 1, /* NULL pointer, non-positive size, bad enum */
  WHISPER_ERR_SHAPE = 2,       /* dims inconsistent or unsupported */
  WHISPER_ERR_DTYPE = 3,       /* dtype not supported by this call */
  WHISPER_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned */
  WHISPER_ERR_WORKSPACE = 5,   /* workspace smaller than the size query returns */
  WHISPER_ERR_CAPACITY = 6,    /* KV cache slot out of range (also written to the device error word) */
  WHISPER_ERR_HIP = 7          /* a HIP launch failed */
} whisper_status;

/* fp8 code formats (OCP 8-bit floats; whisper_blaze showcase page,
 * fp8_quantize.cu card: E4M3 for precision, E5M2 for range). Encoding rounds
 * to nearest even and saturates at the largest finite magnitude (448 or
 * 57344; infinities too); NaN maps to a NaN code of the input's sign. */
typedef enum {
  WHISPER_FP8_E4M3 = 0, /* E4M3FN: bias 7, no infinities, S.1111.111 is NaN */
  WHISPER_FP8_E5M2 = 1  /* E5M2: bias 15, binary16's top byte (inf and NaN as IEEE) */
} whisper_fp8_format;

typedef enum { WHISPER_F32 = 0, WHISPER_BF16 = 1 } whisper_dtype;

/* Model shape. head_dim must be 64 and n_heads*64 == d_model; n_audio_ctx is
 * the number of encoder frames per 30 s chunk (1500); n_text_ctx the number of
 * learned decoder positions. */
typedef struct {
  int n_mels, n_audio_ctx, d_model, n_heads, head_dim, d_ffn;
  int n_enc_layers, n_dec_layers, n_vocab, n_text_ctx;
  whisper_dtype act;
} whisper_dims;

enum { WHISPER_WS_LOGMEL = 0, WHISPER_WS_ENCODE = 1, WHISPER_WS_CROSS_KV = 2, WHISPER_WS_DECODE = 3,
       WHISPER_WS_ENCODE_FP8 = 4 /* whisper_encode_fp8 / whisper_encode_layers_fp8 */,
       WHISPER_WS_DECODE_ENC = 5 /* whisper_decode_step_enc / whisper_decode_prefill_enc, batch = query rows */,
       WHISPER_WS_DECODE_ENC_FP8 = 6 /* whisper_decode_step_enc_fp8 / whisper_decode_prefill_enc_fp8 */ };

/* ------------------------------------------------------------------ weights
 * Logical weights are fp32 device tensors in PyTorch layout, passed as an
 * array of whisper_weight_count() pointers in this order:
 *   encoder (only if n_enc_layers > 0):
 *     conv1.weight [d, n_mels, 3], conv1.bias [d], conv2.weight [d, d, 3], conv2.bias [d],
 *     per layer: attn_ln.{weight,bias} [d], attn.query.{weight [d,d], bias [d]},
 *                attn.key.weight [d,d] (no bias), attn.value.{weight,bias},
 *                attn.out.{weight,bias}, mlp_ln.{weight,bias},
 *                mlp.0.{weight [f,d], bias [f]}, mlp.2.{weight [d,f], bias [d]}   (15 tensors)
 *     ln_post.{weight,bias}
 *   decoder (only if n_dec_layers > 0):
 *     token_embedding [n_vocab, d] (also the tied output projection),
 *     positional_embedding [n_text_ctx, d],
 *     per layer: attn_ln.{w,b}, attn.query.{w,b}, attn.key.w, attn.value.{w,b}, attn.out.{w,b},
 *                cross_attn_ln.{w,b}, cross_attn.query.{w,b}, cross_attn.key.w,
 *                cross_attn.value.{w,b}, cross_attn.out.{w,b},
 *                mlp_ln.{w,b}, mlp.0.{w,b}, mlp.2.{w,b}                          (24 tensors)
 *     ln.{weight,bias}
 * whisper_pack_weights converts them once into the library's packed buffer
 * (activation dtype for matrices, fp32 for biases and LayerNorm parameters;
 * fused QKV, tap-major conv filters, all decoder layers' cross K/V stacked,
 * encoder sinusoidal positions precomputed; in bf16 the decoder's
 * LayerNorm-consumer matrices are LayerNorm-folded and all decoder GEMM
 * matrices are stored in MFMA fragment order). The packed buffer is caller
 * memory of whisper_packed_weights_size() bytes; the logical tensors may be
 * freed once the pack has completed on `stream`. */
int whisper_weight_count(const whisper_dims* dims);
size_t whisper_packed_weights_size(const whisper_dims* dims);
whisper_status whisper_pack_weights(const whisper_dims* dims, const float* const* logical, void* packed,
                                    void* stream);

/* Workspace bytes for a call (`which` is one of WHISPER_WS_*) at `batch`
 * chunks (LOGMEL, ENCODE, CROSS_KV) or rows (DECODE). 0 on invalid input. */
size_t whisper_workspace_size(const whisper_dims* dims, int batch, int which);

/* Batch sizing under a device-memory budget (whisper_blaze showcase page,
 * "VRAM capping": a VRAM limit on a shared card sizes each GPU batch to fit;
 * the project page's batcher caps the batch to the budget). Host arithmetic
 * only, from the size queries above; nothing is allocated or launched.
 * Fills *plan for the largest batch B in 1..max_batch (and B * max(1,
 * prompt_tokens) <= 4096) whose peak footprint fits in budget_bytes, for one
 * pass of B 30 s chunks: log-mel, encoder, cross K/V, an optional fp8
 * quantisation of the cross K/V (cross_fp8 != 0), then decoding with a
 * kv_cap-slot fp8 KV cache (prompt_tokens > 1: one causal prefill first).
 * Every buffer is rounded up to 256 bytes. The schedule keeps the packed
 * weights and ONE workspace of the largest size any call of the pass needs
 * alive throughout, and each stage's buffers only while a stage reads or
 * writes them:
 *   logmel:   audio [B, 480000] fp32 + mel [B, n_mels, 3000] fp32
 *   encode:   mel + encoder output [B, 1500, d] (act dtype)
 *   cross_kv: encoder output + cross K/V [L, 2, B, H, 1500, 64] (act dtype)
 *   quantise: cross K/V + codes (1 byte each) + scales [L, 2] fp32 (fp8 only)
 *   decode:   cross K/V (or codes + scales) + KV cache [L, 2, B, H, kv_cap, 64]
 *             uint8 + its scales + tokens, lengths, argmax [B] int32 + prompt
 *             [B, prompt_tokens] int32 + error word + logits [B, n_vocab] fp32
 *             when want_logits;
 * total = weights + workspace + the largest stage. Returns WHISPER_OK, or
 * WHISPER_ERR_CAPACITY when even B = 1 does not fit (plan then describes
 * B = 1 with plan->batch = 0), WHISPER_ERR_SHAPE for dims without both
 * encoder and decoder or kv_cap outside 1..4096, WHISPER_ERR_INVALID_ARG for
 * a NULL plan or max_batch < 1. */
typedef struct {
  int batch;                 /* planned batch (0: one chunk does not fit) */
  int peak_stage;            /* 0 logmel, 1 encode, 2 cross_kv, 3 quantise, 4 decode */
  size_t weights, workspace; /* packed weights; the one shared workspace */
  size_t audio, mel, encoder_out, cross_kv, cross_codes, kv_cache, decode_state, logits;
  size_t stage[5];           /* live stage buffers of each stage (without weights, workspace) */
  size_t total;              /* weights + workspace + max(stage) */
} whisper_batch_plan;
whisper_status whisper_plan_batch(const whisper_dims* dims, size_t budget_bytes, int kv_cap, int prompt_tokens,
                                  int cross_fp8, int want_logits, int max_batch, whisper_batch_plan* plan);

/* ------------------------------------------------------------------ front end
 * Log-mel features of `batch` chunks (showcase page, mel_spectrogram.cu card;
 * direct kernel call mel_spectrogram(audio) -> [1, 128, T]).
 * audio:   [batch, n_samples] fp32, 16 kHz, n_samples <= 480000 (zero-padded to
 *          30 s; framing reflects at the 480000-sample edges).
 * mel_out: [batch, n_mels, 3000] fp32 (row stride 3000).
 * Reading: 400-point periodic-Hann frames, hop 160, centre reflect padding,
 * 201-bin power spectrum, Slaney mel 0-8 kHz, log10 floor 1e-10, clamp to
 * chunk max - 8, (x + 4) / 4. */
whisper_status whisper_logmel(const whisper_dims* dims, const float* audio, int batch, int n_samples,
                              float* mel_out, void* ws, size_t ws_bytes, void* stream);

/* Overlapping-chunk log-mel for long recordings (showcase page,
 * mel_spectrogram.cu card: overlapping-chunk support for long audio).
 * Chunk i covers samples [i*stride, i*stride + 480000) of the one recording
 * `audio` [n_samples] fp32, zero past its end, and is framed, clamped and
 * scaled as a standalone 30 s clip (whisper_logmel). stride: 160..480000 and
 * a multiple of the 160-sample hop (480000 = no overlap).
 * whisper_chunk_plan (host only) returns the chunk count, and with `plan`
 * non-NULL and max_chunks >= that count fills plan[4 i + 0..3] = {first
 * sample, valid samples, first owned frame, end of owned frames}: owned
 * frames (chunk-local, 10 ms each) split every overlap at its midpoint so
 * each frame of the recording belongs to exactly one chunk, and end at the
 * last frame centred on real audio in the final chunk. Returns 0 on invalid
 * input (or too small a plan), and for recordings of more than 2^31 - 1
 * samples (about 37 h at 16 kHz), whose chunk starts would not fit the int32
 * plan entries. mel_out: [count, n_mels, 3000] fp32; ws:
 * whisper_workspace_size(dims, count, WHISPER_WS_LOGMEL) bytes. */
int whisper_chunk_plan(int64_t n_samples, int stride, int32_t* plan, int max_chunks);
whisper_status whisper_logmel_chunked(const whisper_dims* dims, const float* audio, int64_t n_samples, int stride,
                                      float* mel_out, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------ encoder
 * The encoder transformer of the showcase page ("The Approach": the encoder's
 * attention and its FFN matmuls; "The Solution": gemm_hopper.cu for the
 * projections, flash_attn_hopper.cu for encoder self-attention,
 * layernorm_fused.cu for every residual + LayerNorm; the project page's
 * fused-kernel list counts 162 LayerNorms in large-v3, i.e. pre-LN blocks plus
 * a final LayerNorm per stack).
 * mel [batch, n_mels, 3000] fp32 -> enc_out [batch, n_audio_ctx, d] (act dtype):
 * conv k3 s1 + GELU, conv k3 s2 + GELU, + sinusoidal positions, n_enc_layers
 * pre-LN blocks (fused residual+LayerNorm, bidirectional attention, GELU MLP),
 * final LayerNorm. packed: whisper_pack_weights output; ws:
 * whisper_workspace_size(dims, batch, WHISPER_WS_ENCODE) bytes (16-byte
 * aligned). Errors: INVALID_ARG (batch <= 0, NULL), SHAPE (no encoder layers),
 * ALIGN, WORKSPACE, HIP; nothing is launched unless all checks pass. */
whisper_status whisper_encode(const whisper_dims* dims, const void* packed, const float* mel, int batch,
                              void* enc_out, void* ws, size_t ws_bytes, void* stream);

/* Encoder blocks [layer_begin, layer_end) on hidden states h_in [batch,
 * n_audio_ctx, d] (act dtype, read only) -> h_out (same shape); with
 * apply_ln_post != 0 the final LayerNorm is applied. Uses the ENCODE workspace. */
whisper_status whisper_encode_layers(const whisper_dims* dims, const void* packed, const void* h_in, int batch,
                                     int layer_begin, int layer_end, int apply_ln_post, void* h_out, void* ws,
                                     size_t ws_bytes, void* stream);

/* Cross-attention keys/values of every decoder layer, once per chunk batch
 * (the decoder cross-attention over the encoder output of the showcase page's
 * flash_attn_hopper.cu card; the keys and values depend only on the encoder
 * output, so they are projected once for all decode steps):
 * K = enc W_k^T, V = enc W_v^T + b_v, written head-major as
 * cross_kv [n_dec_layers][2][batch][n_heads][n_audio_ctx][64] (act dtype),
 * caller-owned. enc_out: [batch, n_audio_ctx, d] from whisper_encode. ws and
 * ws_bytes are not used (NULL is fine). Errors: INVALID_ARG, SHAPE (no
 * decoder layers), ALIGN, HIP; nothing is launched unless all checks pass. */
whisper_status whisper_cross_kv(const whisper_dims* dims, const void* packed, const void* enc_out, int batch,
                                void* cross_kv, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------ decoder step
 * One batched decoder step with given tokens (teacher forcing or greedy): the
 * autoregressive decoder of the showcase page (flash_attn_hopper.cu card:
 * causal self-attention and cross-attention) over the KV cache of the
 * Endpoints post's inference stack ("Inference Stack": compute in bfloat16,
 * keys and values stored as float8, one byte per element, quantised on the
 * way in). Errors: INVALID_ARG, SHAPE (no decoder layers, kv_cap outside
 * 1..4096), ALIGN, WORKSPACE (ws smaller than whisper_workspace_size(dims,
 * batch, WHISPER_WS_DECODE), or an armed K/V debug buffer too small), HIP;
 * nothing is launched unless all checks pass.
 * tokens:    [batch] int32 token ids.
 * lengths:   [batch] int32, in/out. lengths[b] is the cache slot the new token's
 *            K/V go to and its position; +1 on return.
 * kv_cache:  [n_dec_layers][2][batch][n_heads][kv_cap][64] uint8 OCP-E4M3 codes
 *            (K then V), caller-owned. Per layer the new token's K and V are
 *            quantised from the fp32 projection output as
 *            code = e4m3_rne_saturate(fl32(x * fl32(1/scale))) into slot
 *            lengths[b], then attention reads slots 0..lengths[b] dequantised.
 * kv_scales: [n_dec_layers][2] fp32 (K, V), constant while codes are live.
 * cross_kv:  from whisper_cross_kv for the same batch.
 * logits:    [batch, n_vocab] fp32 or NULL (then kept in the workspace).
 * argmax:    [batch] int32 greedy token (lowest index on ties).
 * dev_error: device int32 or NULL; set to WHISPER_ERR_CAPACITY when a slot is
 *            >= kv_cap or >= n_text_ctx (that row's write is skipped), or
 *            WHISPER_ERR_INVALID_ARG for a token id out of range. */
whisper_status whisper_decode_step(const whisper_dims* dims, const void* packed, int batch, int kv_cap,
                                   const int32_t* tokens, int32_t* lengths, uint8_t* kv_cache,
                                   const float* kv_scales, const void* cross_kv, float* logits, int32_t* argmax,
                                   int32_t* dev_error, void* ws, size_t ws_bytes, void* stream);

/* whisper_decode_step for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. It takes no
 * workspace: the step's activations, split-K partials and tile counters live
 * in a library-owned static device array of WHISPER_NOALLOC_SCRATCH_BYTES
 * (8 MiB) per GPU, set up on the first call on that device and held until the
 * process ends; the call itself allocates nothing. Arguments and results are
 * those of whisper_decode_step, except that logits must be given (non-NULL).
 * A batch whose workspace without logits (whisper_workspace_size(dims, batch,
 * WHISPER_WS_DECODE) less batch * n_vocab * 4 bytes, about 81 KB per row at
 * the large-v3 shape: up to 100 rows) exceeds the array returns
 * WHISPER_ERR_WORKSPACE before launching anything. Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (other
 * streams, other threads) race and must be serialised by the caller; the
 * split-K tile counters are cleared at the start of every call. */
#define WHISPER_NOALLOC_SCRATCH_BYTES (8u << 20)
whisper_status whisper_decode_step_noalloc(const whisper_dims* dims, const void* packed, int batch, int kv_cap,
                                           const int32_t* tokens, int32_t* lengths, uint8_t* kv_cache,
                                           const float* kv_scales, const void* cross_kv, float* logits,
                                           int32_t* argmax, int32_t* dev_error, void* stream);

/* Causal prefill of n_tokens prompt tokens per row in one pass (the pages'
 * decoder self-attention with multiple queries; showcase page,
 * flash_attn_hopper.cu card: causal mask). bf16 models only. tokens:
 * [batch, n_tokens] int32; row b's token p goes to cache slot and position
 * lengths[b] + p and attends over slots 0 .. lengths[b] + p. The result
 * equals n_tokens successive whisper_decode_step calls with those tokens:
 * the same codes in kv_cache, and logits / argmax of each row's last
 * token ([batch, n_vocab] / [batch]); lengths[b] += n_tokens. Requires
 * batch * n_tokens <= 4096; ws: whisper_workspace_size(dims, batch *
 * n_tokens, WHISPER_WS_DECODE) bytes. Other arguments as whisper_decode_step. */
whisper_status whisper_decode_prefill(const whisper_dims* dims, const void* packed, int batch, int n_tokens,
                                      int kv_cap, const int32_t* tokens, int32_t* lengths, uint8_t* kv_cache,
                                      const float* kv_scales, const void* cross_kv, float* logits, int32_t* argmax,
                                      int32_t* dev_error, void* ws, size_t ws_bytes, void* stream);

/* Decoder step and causal prefill with the cross-attention read straight
 * from the encoder output (the decoder cross-attention over the encoder
 * output of the showcase page's flash_attn_hopper.cu card). As
 * whisper_decode_step / whisper_decode_prefill, bf16 models with d_model in
 * {512, 768, 1024, 1280}, except that enc_out [batch][n_audio_ctx][d] bf16
 * (whisper_encode's output) replaces cross_kv. Since K = E W_k^T and
 * V = E W_v^T + b_v are linear in E and the softmax weights sum to one, each
 * head computes softmax((W_k,h^T q_h) . E^T / 8) over the frames, u_h =
 * sum_t p_t E_t, and W_v,h u_h + b_v,h: the same attention, reading E once per
 * layer (half the bytes of K and V) and never forming K or V, so no
 * whisper_cross_kv pass is needed. The frames are shared among workgroups
 * according to the number of activation rows, so a prefill here agrees with
 * successive steps to rounding, not bit for bit. ws: whisper_workspace_size(dims, batch *
 * n_tokens, WHISPER_WS_DECODE_ENC) bytes. Errors as whisper_decode_prefill. */
whisper_status whisper_decode_step_enc(const whisper_dims* dims, const void* packed, int batch, int kv_cap,
                                       const int32_t* tokens, int32_t* lengths, uint8_t* kv_cache,
                                       const float* kv_scales, const void* enc_out, float* logits, int32_t* argmax,
                                       int32_t* dev_error, void* ws, size_t ws_bytes, void* stream);

/* whisper_decode_step_enc with the decoder MLP as mixed_fp8 sites (the
 * showcase page's precision.py card: in the mixed_fp8 preset the decoder FFN
 * runs in fp8 E4M3, weights and activations). packed8: whisper_pack_weights_fp8
 * output, which holds E4M3 codes of each decoder layer's fc1 and fc2 with one
 * amax scale per tensor (fl32(amax) / 448). Per layer: each row's
 * a = bf16(LayerNorm(x)) (fp32 statistics; rounded to bf16 like every
 * activation of the step) is quantised with its own scale (fl32(amax |a|) /
 * 448, code = e4m3(fl32(a * fl32(1 / s)))); fc1 sums code values times weight
 * code values in fp32, times the two scales, + bias, GELU, stored bf16; each
 * stored hidden row is quantised the same way with its own scale; fc2
 * likewise, + bias, added to the residual stream (whisper_decode_mlp_fp8 runs
 * this sublayer alone). The rest of the step is whisper_decode_step_enc. Requires d_model and d_ffn multiples of 256 (and of
 * 80), d_ffn a multiple of 1024. ws: whisper_workspace_size(dims, batch,
 * WHISPER_WS_DECODE_ENC_FP8) bytes. Errors as whisper_decode_step_enc. */
whisper_status whisper_decode_step_enc_fp8(const whisper_dims* dims, const void* packed, const void* packed8,
                                           int batch, int kv_cap, const int32_t* tokens, int32_t* lengths,
                                           uint8_t* kv_cache, const float* kv_scales, const void* enc_out,
                                           float* logits, int32_t* argmax, int32_t* dev_error, void* ws,
                                           size_t ws_bytes, void* stream);
whisper_status whisper_decode_prefill_enc(const whisper_dims* dims, const void* packed, int batch, int n_tokens,
                                          int kv_cap, const int32_t* tokens, int32_t* lengths, uint8_t* kv_cache,
                                          const float* kv_scales, const void* enc_out, float* logits,
                                          int32_t* argmax, int32_t* dev_error, void* ws, size_t ws_bytes,
                                          void* stream);
/* whisper_decode_prefill_enc with the decoder MLP as mixed_fp8 sites, as
 * whisper_decode_step_enc_fp8 (each of the batch * n_tokens activation rows
 * takes its own activation scales): the computation of n_tokens successive
 * whisper_decode_step_enc_fp8 calls. ws: whisper_workspace_size(dims,
 * batch * n_tokens, WHISPER_WS_DECODE_ENC_FP8) bytes. */
whisper_status whisper_decode_prefill_enc_fp8(const whisper_dims* dims, const void* packed, const void* packed8,
                                              int batch, int n_tokens, int kv_cap, const int32_t* tokens,
                                              int32_t* lengths, uint8_t* kv_cache, const float* kv_scales,
                                              const void* enc_out, float* logits, int32_t* argmax,
                                              int32_t* dev_error, void* ws, size_t ws_bytes, void* stream);

/* Decoder step with fp8 cross-attention K/V (the fp8 cross-attention site of
 * the showcase page's precision presets, whose aggressive preset takes E5M2
 * there for range; project page, "Direct Kernel API": quantise_e4m3 with a
 * per-tensor scale). As whisper_decode_step, bf16 models only, except that
 * the cross-attention keys and values are fp8 codes:
 * cross_codes:  [n_dec_layers][2][batch][n_heads][n_audio_ctx][64] uint8, the
 *               bf16 whisper_cross_kv output of each (layer, K|V) slab
 *               quantised with whisper_fp8_quantize in cross_format
 *               (code = fp8_rne_saturate(fl32(x * fl32(1/scale)))),
 *               caller-owned;
 * cross_scales: [n_dec_layers][2] fp32 device scales, K then V;
 * cross_format: WHISPER_FP8_E4M3 or WHISPER_FP8_E5M2 (else INVALID_ARG).
 * The KV cache stays E4M3 either way. The cross-attention reads half the
 * bytes of the bf16 form and dequantises on read: score =
 * (q . value(codes_k)) * scale_k / 8, output = sum p * value(codes_v) * scale_v. */
whisper_status whisper_decode_step_xq(const whisper_dims* dims, const void* packed, int batch, int kv_cap,
                                      const int32_t* tokens, int32_t* lengths, uint8_t* kv_cache,
                                      const float* kv_scales, const uint8_t* cross_codes, const float* cross_scales,
                                      whisper_fp8_format cross_format, float* logits, int32_t* argmax,
                                      int32_t* dev_error, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------ mixed_fp8 encoder
 * The showcase page's mixed_fp8 precision preset (precision.py card, its
 * table of layer sites): the encoder FFN (fc1, fc2) and the attention's
 * query/key/value projections take fp8 E4M3 weights and activations, and so
 * does the decoder FFN (whisper_decode_step_enc_fp8, one activation scale per
 * row there: a row is one token of one chunk); the attention, its output
 * projection, the conv stem and the rest of the decoder keep bf16. Scales (fp8_quantize.cu card; "Learnings": per-tensor
 * scales from activation maxima): one per weight tensor, fl32(amax) / 448,
 * computed at pack time; one per activation tensor at each site and chunk
 * (the 1500 x d or 1500 x d_ffn activation of one 30 s clip, so a chunk's
 * output does not depend on its batch), fl32(amax) / 448, computed on the
 * device before each site. A site computes
 *   y = fl32(sum value(code_x) value(code_w)) * s_x * s_w + bias
 * with fp32 accumulation, then its epilogue (GELU for fc1) in bf16.
 * Only for bf16 models with d_model and d_ffn multiples of 256.
 *
 * whisper_pack_weights_fp8 quantises the encoder's query, key, value, fc1 and
 * fc2 weights and the decoder's fc1 and fc2 weights from the same logical
 * fp32 tensors whisper_pack_weights takes (16-byte aligned) into caller
 * memory `packed8` of whisper_packed_weights_fp8_size() bytes (0 for a model
 * with no layers); ws: whisper_fp8_workspace_size() bytes. The bf16 `packed` buffer is still needed (biases, LayerNorms, stem,
 * out-projection). whisper_encode_fp8 and whisper_encode_layers_fp8 are
 * whisper_encode and whisper_encode_layers with the fp8 sites; ws:
 * whisper_workspace_size(dims, batch, WHISPER_WS_ENCODE_FP8) bytes. */
size_t whisper_packed_weights_fp8_size(const whisper_dims* dims);
whisper_status whisper_pack_weights_fp8(const whisper_dims* dims, const float* const* logical, void* packed8,
                                        void* ws, size_t ws_bytes, void* stream);
whisper_status whisper_encode_fp8(const whisper_dims* dims, const void* packed, const void* packed8,
                                  const float* mel, int batch, void* enc_out, void* ws, size_t ws_bytes,
                                  void* stream);
whisper_status whisper_encode_layers_fp8(const whisper_dims* dims, const void* packed, const void* packed8,
                                         const void* h_in, int batch, int layer_begin, int layer_end,
                                         int apply_ln_post, void* h_out, void* ws, size_t ws_bytes, void* stream);

/* One fp8 site as a kernel call (showcase page, gemm_hopper.cu card: FP8
 * E4M3 GEMM). a: E4M3 codes [M, K] row-major; w: E4M3 codes [N, K] (PyTorch
 * weight layout); a_scales: one fp32 scale per group of rows_per_scale rows
 * (row m uses a_scales[m / rows_per_scale]); w_scale: one fp32 scale; bias:
 * [N] fp32 or NULL; gelu != 0 applies exact GELU. c: bf16 [M, ldc], columns
 * 0..N-1 written: c[m][n] = bf16(epi(acc * a_scales[m / rows_per_scale] *
 * w_scale[0] + bias[n])), acc the fp32 sum of value(a[m][k]) * value(w[n][k]).
 * Requires K % 256 == 0, K >= 512, N % 256 == 0, ldc % 8 == 0, ldc >= N,
 * rows_per_scale >= 256, every operand under 2 GB (else WHISPER_ERR_SHAPE). */
whisper_status whisper_gemm_fp8(const uint8_t* a, int M, int K, const float* a_scales, int rows_per_scale,
                                const uint8_t* w, int N, const float* w_scale, const float* bias, int gelu, void* c,
                                long ldc, void* stream);

/* ------------------------------------------------------------------ kernel-level calls
 * fp8 codec with a per-tensor scale (project page quantise_e4m3 /
 * dequantise_e4m3; showcase page fp8_quantize.cu card: E4M3 and E5M2).
 * x: n values of dtype `dt`; fmt: WHISPER_FP8_E4M3 or WHISPER_FP8_E5M2 (else
 * INVALID_ARG). With scale_in == NULL the scale is computed on the device as
 * fl32(amax) / fmax (fmax = 448 for E4M3, 57344 for E5M2; 1.0 if amax is 0)
 * and written to scale_out; this needs a workspace of
 * whisper_fp8_workspace_size() bytes.
 * codes[i] = fp8_rne_saturate(fl32(x[i] * fl32(1/scale))). */
size_t whisper_fp8_workspace_size(void);
whisper_status whisper_fp8_quantize(const void* x, whisper_dtype dt, whisper_fp8_format fmt, size_t n,
                                    const float* scale_in, uint8_t* codes, float* scale_out, void* ws,
                                    size_t ws_bytes, void* stream);
/* y[i] = fl32(value(codes[i]) * scale[0]) in format fmt, stored in dtype dt
 * (E5M2 infinity codes give +-inf, NaN codes NaN). */
whisper_status whisper_fp8_dequantize(const uint8_t* codes, whisper_fp8_format fmt, size_t n, const float* scale,
                                      void* y, whisper_dtype dt, void* stream);

/* Fused residual + LayerNorm (showcase page, layernorm_fused.cu card; project
 * page layernorm_fused_residual): total = fl32(h + residual) (h alone if
 * residual is NULL), normed = (total - mean) / sqrt(var + eps) * gamma + beta,
 * biased variance over d_model, fp32 statistics. h and normed: [M, d_model] in
 * dims->act; residual and total: [M, d_model] fp32 (the residual stream is
 * kept in fp32 between blocks); gamma, beta: [d_model] fp32. normed or total
 * may be NULL (not written). total may alias residual. */
whisper_status whisper_layernorm_fused(const whisper_dims* dims, const void* h, const float* residual,
                                       const float* gamma, const float* beta, float eps, int M, void* normed,
                                       float* total, void* stream);

/* Projection GEMM (showcase page, gemm_hopper.cu card): y = act(x . w^T + bias)
 * with x [M, K] (row stride lda elements), w [N, K], bias [N] fp32 or NULL,
 * y [M, N]; act 0 = none, 1 = exact GELU. dt = WHISPER_BF16 needs K % 64 == 0
 * and lda % 8 == 0. path: 0 auto, 1 tiled MFMA (automatic tile), 2 skinny
 * (M <= 128, K % 128 == 0); 3, 4, 5, 6 force the 128x128, 256x256 8-wave,
 * 256x256 4-wave and 256x256 LDS-DMA-pipelined 8-wave tiled kernels; 8 is
 * the 8-wave LDS-DMA kernel with the plain tile order (6 uses the
 * weight-panel-grouped order), and 7 (once a 4-wave LDS-DMA kernel, retired:
 * its accumulators did not fit the register file) runs 8's kernel; 9 is the
 * persistent 8-wave LDS-DMA kernel
 * (one workgroup per compute unit, the ring running on across tiles), which
 * the automatic choice takes for large bf16 GEMMs without activation or with
 * GELU when N % 256 == 0, K % 128 == 0, K >= 256 and y is under 2 GB. 5-9
 * are for measurement; 5-8 need N % 8 == 0 and the DMA kernels K % 128 == 0,
 * and fall back to 128x128 otherwise; 9 falls back to 6. */
whisper_status whisper_linear(whisper_dtype dt, const void* x, int lda, const void* w, const float* bias, int M,
                              int N, int K, int act, void* y, int path, void* stream);

/* Encoder bidirectional self-attention (flash_attn_hopper.cu card): qkv
 * [batch, T, 3*n_heads*64] (Q | K | V, heads contiguous) -> out [batch, T,
 * n_heads*64], per head softmax(q k^T / 8) v; no score matrix is stored. */
whisper_status whisper_attention_encoder(whisper_dtype dt, const void* qkv, int batch, int T, int n_heads,
                                         void* out, void* stream);

/* Decoder self-attention over an e4m3 cache (direct kernel call
 * decoder_self_attn): q [batch, n_heads*64]; k_codes, v_codes [batch][n_heads]
 * [cap][64]; scales [2] fp32 (K, V); n_keys [batch] int32 keys 0..n_keys-1
 * are attended (clamped to cap). out [batch, n_heads*64]. */
whisper_status whisper_attention_decode_self(whisper_dtype dt, const void* q, int batch, int n_heads, int cap,
                                             const uint8_t* k_codes, const uint8_t* v_codes, const float* scales,
                                             const int32_t* n_keys, void* out, void* stream);

/* Decoder cross-attention: q [batch, n_heads*64], k and v head-major
 * [batch][n_heads][T][64] -> out [batch, n_heads*64], one pass per (row,
 * head). whisper_attention_decode_cross_workspace_size() returns 0: ws and
 * ws_bytes are accepted for interface stability and not used (NULL is fine). */
size_t whisper_attention_decode_cross_workspace_size(int batch, int n_heads, int T);
whisper_status whisper_attention_decode_cross(whisper_dtype dt, const void* q, const void* k, const void* v,
                                              int batch, int n_heads, int T, void* out, void* ws, size_t ws_bytes,
                                              void* stream);

/* One projection of the batched decoder step, as the fused step runs it
 * (kernel-level call for tests and measurement; the decoder GEMMs of the
 * showcase page's gemm_hopper.cu card with the residual + LayerNorm of its
 * layernorm_fused.cu card folded in). bf16 weights, fp32 accumulation,
 * M <= 4096 rows, K % 32 == 0. The LN modes compute LN(x) . W^T + bias with
 * LN(x) = (x - mean) / sqrt(var + 1e-5) * gamma + beta over the K values of a
 * row (biased variance), folded into the weights: y = r (x . W'^T - mean c1) +
 * b2, W' = bf16(gamma * W), c1 = sum_k W'[., k], b2 = bias + W . beta,
 * r = 1 / sqrt(var + 1e-5), with x entering the MFMA as bf16 hi + lo parts.
 *   WHISPER_DEC_LN_STORE  y [M, N] bf16                           (cross-attention query)
 *   WHISPER_DEC_LN_GELU   y [M, N] bf16 = gelu(.)                 (MLP up-projection)
 *   WHISPER_DEC_LN_F32    y [M, N] fp32, unrounded                (vocabulary projection)
 *   WHISPER_DEC_LN_QKV    N == 3 K, K % 64 == 0: columns [0, K) -> y [M, K] bf16
 *                         (query); key and value columns appended as e4m3 codes
 *                         code = e4m3_rne_saturate(fl32(v * fl32(1/scale))) to
 *                         kv_cache [2][M][K/64][kv_cap][64] at slot lengths[m]
 *                         (scales kv_scales[2], K then V; a slot outside
 *                         0..kv_cap-1 skips the write and sets *dev_error = 6)
 *   WHISPER_DEC_RESID     x [M, N] fp32 += a . bf16(W)^T + bias, a [M, K] bf16 (N % 32 == 0)
 *   WHISPER_DEC_RESID_SPLITK  the same with K split over 4 workgroups per
 *                         16 x 80 tile (N % 80 == 0, K % 1024 == 0), as the
 *                         step's MLP down-projection
 * x: LN modes [M, K] fp32 (read); residual modes [M, N] fp32 (read and
 * written). w: [N, K] fp32 logical weight and bias [N] fp32 or NULL; each
 * call rounds and re-lays them out into ws (whisper_decode_linear_workspace_size
 * bytes, 0 for invalid arguments). gamma, beta: [K] fp32 (LN modes).
 * Errors: INVALID_ARG (mode, sizes, NULL), SHAPE, ALIGN, WORKSPACE, HIP;
 * nothing is launched unless all checks pass. */
enum {
  WHISPER_DEC_LN_STORE = 0, WHISPER_DEC_LN_GELU = 1, WHISPER_DEC_LN_F32 = 2, WHISPER_DEC_LN_QKV = 3,
  WHISPER_DEC_RESID = 4, WHISPER_DEC_RESID_SPLITK = 5
};
size_t whisper_decode_linear_workspace_size(int mode, int M, int N, int K);
whisper_status whisper_decode_linear(int mode, int M, int N, int K, float* x, const void* a, const float* w,
                                     const float* bias, const float* gamma, const float* beta, void* y,
                                     uint8_t* kv_cache, const float* kv_scales, const int32_t* lengths, int kv_cap,
                                     int32_t* dev_error, void* ws, size_t ws_bytes, void* stream);

/* One decoder MLP sublayer with the mixed_fp8 sites (the showcase page's
 * precision.py card: decoder FFN in fp8 E4M3), as whisper_decode_step_enc_fp8
 * runs it (kernel-level call for tests and measurement):
 *   a   = bf16(LN(x))                     LN as in whisper_decode_linear
 *   h   = bf16(gelu(site(a, w1) + b1))    (the hidden rows, bf16)
 *   x  += site(h, w2) + b2
 * where site(a, w) = e4m3(a / s_a) . e4m3(w / s_w)^T * s_a * s_w with one
 * activation scale per row, s_a = fl32(amax |a_row|) / 448 (1 for a zero
 * row), and a per-tensor weight scale s_w = fl32(amax |w|) / 448; codes are
 * e4m3_rne_saturate(fl32(v * fl32(1 / s))), products exact, fp32
 * accumulation. x: [M, d] fp32 row-major, read and written. gamma, beta,
 * b2: [d] fp32; w1 [f, d], b1 [f], w2 [d, f] fp32 logical weights, which
 * each call quantises into ws (whisper_decode_mlp_fp8_workspace_size bytes,
 * 0 for invalid sizes). hidden: optional [M, f] bf16 output, the GELU rows
 * as stored (the second site's input). hidden_amax: optional [M] fp32
 * output, amax |h_row| (the second site's s_a is hidden_amax / 448).
 * Sizes: 1 <= M <= 4096, d % 80 == 0, d <= 2048, f % 80 == 0, f % 1024 == 0.
 * Errors: SHAPE, INVALID_ARG (NULL), ALIGN, WORKSPACE, HIP; nothing is
 * launched unless all checks pass. */
size_t whisper_decode_mlp_fp8_workspace_size(int M, int d, int f);
/* Host evaluation (no GPU) of the rounding the second site applies to its
 * bf16 input in registers: y[i] = the value of e4m3_rne_saturate(x[i]) for
 * finite x[i] (the code is not formed; host and device run the same fp32
 * arithmetic). x, y: n host floats. Errors: INVALID_ARG (NULL with n > 0). */
whisper_status whisper_e4m3_round_host(const float* x, float* y, size_t n);
whisper_status whisper_decode_mlp_fp8(int M, int d, int f, float* x, const float* gamma, const float* beta,
                                      const float* w1, const float* b1, const float* w2, const float* b2,
                                      void* hidden, float* hidden_amax, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------ K/V append debug hooks
 * For parity tests of the fp8 KV append (quantise on write, Endpoints post,
 * "Inference Stack"). While armed, every whisper_decode_step,
 * whisper_decode_step_xq, whisper_decode_prefill and WHISPER_DEC_LN_QKV call
 * uses two optional caller buffers of [n_layers][2][rows][d_model] elements
 * (rows = batch * n_tokens; one layer for whisper_decode_linear), indexed by
 * (layer, K|V, activation row, channel):
 *   kv_pre   (fp32, may be NULL): receives the key and value of each appended
 *            token as the projection computes them, the value the codec
 *            multiplies by fl32(1/scale) and rounds;
 *   kv_force (int16, may be NULL): an entry >= 0 is the code written to the
 *            cache for that value instead of the kernel's own (so a test can
 *            give the GPU another implementation's codes, and the GPU's later
 *            reads see them); a negative entry keeps the kernel's code.
 * A call whose rows would not fit in n_elems returns WHISPER_ERR_WORKSPACE
 * before launching anything. The buffers are caller device memory that must
 * stay valid until disarm. Process-wide, not thread-safe (like the
 * measurement hook below); disarmed, the hooks cost one pointer test per
 * appended value. */
whisper_status whisper_debug_kv_arm(float* kv_pre, const int16_t* kv_force, size_t n_elems);
void whisper_debug_kv_disarm(void);

/* ------------------------------------------------------------------ measured ceilings
 * The rates this part sustains, for rooflines reported against measured as
 * well as vendor peaks. whisper_peak_mfma runs n_wg workgroups of 4 waves,
 * each `iters` rounds of 16 independent MFMA 16x16x32 bf16 on register
 * operands, and writes n_wg * 4 floats to `out` (device, 4-byte aligned);
 * its FLOP count is whisper_peak_mfma_flop(n_wg, iters). whisper_peak_read
 * streams `bytes` (a positive multiple of 16) of the 16-byte-aligned device
 * buffer `buf` with 16-byte loads over n_wg workgroups of 256 threads and
 * writes n_wg floats to `out`. Time them with events on `stream`. */
whisper_status whisper_peak_mfma(int n_wg, int iters, float* out, void* stream);
double whisper_peak_mfma_flop(int n_wg, int iters);
whisper_status whisper_peak_read(const void* buf, size_t bytes, int n_wg, float* out, void* stream);

/* ------------------------------------------------------------------ measurement hook
 * For measurement harnesses that need one kernel's own launch duration inside
 * the composite calls, on the stream it runs on. While armed, every launch of
 * the chosen kernel family is bracketed by hipEventRecord(start_events[i]) and
 * hipEventRecord(stop_events[i]) on the call's stream, for the first
 * `capacity` launches; events are hipEvent_t (passed as void*) created and
 * owned by the caller. Process-wide, not thread-safe; the only state the
 * library keeps besides error text. whisper_profile_disarm returns the number
 * of event pairs recorded and clears the hook. Disarmed, the hook costs one
 * flag test per launch of the measured kernels, nothing on the device. */
enum {
  WHISPER_PROF_DECODE_CROSS_ATTENTION = 1, /* split-T partial kernel of the decoder cross-attention */
  WHISPER_PROF_DECODE_SELF_ATTENTION = 2,  /* decoder self-attention over the fp8 cache */
  WHISPER_PROF_ENCODER_ATTENTION = 3,      /* encoder flash attention */
  WHISPER_PROF_ENCODER_FFN1 = 4,           /* encoder MLP up-projection GEMM (+GELU) */
  WHISPER_PROF_ENCODER_LAYERNORM = 5       /* encoder fused residual + LayerNorm before the MLP */
};
whisper_status whisper_profile_arm(int kind, void* const* start_events, void* const* stop_events, int capacity);
int whisper_profile_disarm(void);

const char* whisper_status_string(whisper_status status);
const char* whisper_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* WHISPER_MI355X_H */
