// Launch-level interface between the C-ABI host layer (api.cpp) and the
// kernel translation units. Everything here enqueues on a stream and returns
// the launch status; argument checks happen in api.cpp before any launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace wh {

enum ActType { ACT_F32 = 0, ACT_BF16 = 1 };
// fp8 code formats (values match the public whisper_fp8_format enum)
enum Fp8Fmt { FP8_E4M3 = 0, FP8_E5M2 = 1 };
typedef uint16_t u16_t;

// ------------------------------------------------------------------ GEMM
// C = epilogue(A[M,K] . B[N,K]^T + bias); A rows may overlap (lda < K) for
// the implicit-GEMM convolutions. Batched over blockIdx.z with element strides.
enum Epi {
  EPI_STORE = 0,    // C = acc + bias (act type)
  EPI_GELU = 1,     // C = gelu(acc + bias)
  EPI_GELU_PE = 2,  // C (fp32 residual stream) = gelu(acc + bias) + pe[row, col]
  EPI_F32 = 3,      // C (fp32) = acc + bias
  EPI_CROSSKV = 4,  // scatter acc + bias head-major into [L][2][B][H][T][64]
  EPI_DEC_QKV = 5,  // q -> q_out; k, v -> e4m3 codes at cache slot lengths[row]
};

struct GemmParams {
  const void* A; long lda; long strideA;
  const void* B; long ldb;
  int M, N, K, batch;
  const float* bias;
  void* C; long ldc; long strideC;
  const float* pe;
  // EPI_CROSSKV
  int ckv_T, ckv_B, ckv_H, ckv_d;
  // EPI_DEC_QKV
  uint8_t* kv_cache; const float* kv_scales; const int32_t* lengths; int32_t* dev_error;
  int kv_cap, kv_B, kv_H, kv_layer, d_model;
  // EPI_DEC_QKV debug hooks (NULL: off): kv_pre receives the fp32 K / V values
  // the codec is applied to; a non-negative kv_force entry is written to the
  // cache instead of the kernel's own code. Both [n_layers][2][M][d_model].
  float* kv_pre;
  const int16_t* kv_force;
  // tiled-kernel choice for measurement: 0 automatic, 1 128x128, 2 256x256/8 waves, 3 256x256/4 waves,
  // 4 256x256 with the LDS DMA pipeline
  int variant;
  // fp8 GEMM (launch_gemm_fp8): C = epi(acc * a_scale[m / a_rows_per_scale] * b_scale[0] + bias)
  const float* a_scale; int a_rows_per_scale; const float* b_scale;
};

hipError_t launch_gemm(ActType t, Epi epi, const GemmParams& p, hipStream_t s);
// fp8 E4M3 A [M, K] and B [N, K] codes (K, lda, ldb in bytes), bf16 C;
// EPI_STORE or EPI_GELU.
hipError_t launch_gemm_fp8(Epi epi, const GemmParams& p, hipStream_t s);
// Skinny path for decode (M <= 128): weights streamed once, K split over waves.
hipError_t launch_gemm_skinny(ActType t, Epi epi, const GemmParams& p, hipStream_t s);

// ------------------------------------------------------------------ decoder-step GEMMs (bf16, M <= 128)
// PRO_A: A is a bf16 activation block. PRO_X: A = LayerNorm(X) of the fp32
// residual stream, folded into W (gamma), c1 and the bias (beta).
enum DecPro { PRO_A = 0, PRO_X = 1 };
enum DecEpi { DEPI_STORE = 0, DEPI_GELU = 1, DEPI_RESID = 2, DEPI_QKV = 3, DEPI_F32 = 4 };
struct DecGemmParams {
  int M, N, K;
  const u16_t* W;            // [N, K] bf16 in fragment order (PRO_X: gamma-folded)
  const float* bias;         // [N] or NULL (PRO_X: folded bias b + W beta)
  const float* c1;           // PRO_X: [N] row sums of the folded W
  const u16_t* A; long lda;  // PRO_A: [M, K] bf16, row stride lda
  float* X;                  // residual stream [M, d] fp32 in 16-row tiles (dec_x_index): PRO_X input, DEPI_RESID in/out
  u16_t* out;                // DEPI_STORE / GELU: [M, N] bf16; DEPI_QKV: q [M, d]
  float* out_f32;            // DEPI_F32: [M, N]
  // DEPI_QKV: k, v appended as e4m3 codes at slot lengths[m]
  uint8_t* kv_cache; const float* kv_scales; const int32_t* lengths; int32_t* dev_error;
  int kv_cap, kv_B, kv_H, kv_layer, d_model;
  // DEPI_QKV debug hooks (NULL: off): kv_pre receives the fp32 K / V values
  // the codec is applied to; a non-negative kv_force entry is written to the
  // cache instead of the kernel's own code. Both [n_layers][2][M][d_model].
  float* kv_pre;
  const int16_t* kv_force;
  // split-K over ks workgroups per output tile (PRO_A only; ks <= 1: none):
  // partial blocks [tiles][ks][MB*CB][64 lanes] f32x4 and one counter per tile,
  // zero on entry (each launch leaves them zero)
  int ks; float* part; int32_t* cnt;
  // rows per batch row (prefill of R tokens per row: row m is batch row m / R
  // at position lengths[m / R] + m % R); 0 or 1 for one token per row
  int rows_per_b;
  // PRO_A with one A row per group of a_group output columns (0: off): the A
  // row of output column n starts a_group_stride elements further per group
  // (A + m * lda + (n / a_group) * a_group_stride); a_group must be a
  // multiple of the workgroup's column tile
  int a_group; long a_group_stride;
  // fp8 weights (launch_gemm_dec_fp8): W8 E4M3 codes [N, K] in fragment order
  // with the per-tensor scale w_scale8[0]; the products are the codes' values,
  // and the epilogue multiplies by (row scale) * w_scale8[0] before the bias.
  // Row scale: row_scale[m] (A already holds code values), or, with aq_part,
  // fl32(amax) / 448 (1 for 0) where amax is the largest of the row's
  // amax_nblk partials aq_part[m][0 .. amax_nblk) (amax_nblk % 4 == 0, aq_part
  // 16-byte aligned), the A row being quantised
  // in registers as e4m3(fl32(a * fl32(1 / s))). amax_out (DEPI_GELU, NULL:
  // off; amax_nblk == N / 16): amax_out[m][j] = max |stored bf16 output| of
  // row m over columns 16 j .. 16 j + 15, every entry of rows < M written.
  const uint8_t* W8; const float* w_scale8; const float* row_scale; const float* aq_part; float* amax_out;
  int amax_nblk;
  // DEPI_F32 (NULL: off): per row, the largest value of each 16-column block
  // and its column (lowest on ties; NaN never chosen), [M][ceil(N / 16)] as
  // (float bits, column); argmax_part reduces them
  int2* amax_part;
};
void dec_gemm_tiles(int M, int N, int& mb, int& cb);
hipError_t launch_gemm_dec(DecPro pro, DecEpi epi, const DecGemmParams& p, int mb, int cb, hipStream_t s);
// The decoder MLP as mixed_fp8 sites (bf16 activations A, fp8 weights W8):
// DEPI_GELU (up-projection, 80-column tiles) or DEPI_RESID with split-K over
// DEC_KSPLIT workgroups (down-projection).
hipError_t launch_gemm_dec_fp8(DecEpi epi, const DecGemmParams& p, hipStream_t s);
hipError_t launch_pack_dec_weight_fp8(const float* W, int N, int K, const float* scale, void* Wf, hipStream_t s);
void e4m3_round_host(const float* x, float* y, size_t n);
hipError_t launch_rows_max(const float* part, int M, int nblk, float* out, hipStream_t s);
hipError_t launch_ln_quant_rows(const float* X, const float* g, const float* b, int M, int K, void* A, float* srow,
                                hipStream_t s);
hipError_t launch_fold_ln(const float* W, const float* gamma, const float* beta, const float* bias, int N, int K,
                          void* Wf, float* c1, float* b2, hipStream_t s);
hipError_t launch_pack_dec_weight(const float* W, int N, int K, void* Wf, hipStream_t s);

// ------------------------------------------------------------------ cross-attention over the encoder output (cross_enc.hip)
// W_kT[h][n][j] = bf16(W_k[h * 64 + j][n]) from the fp32 [d, d] key weight
hipError_t launch_pack_kt(const float* wk, int d, void* wkt, hipStream_t s);
// q'[m][h][:] = W_k,h^T q[m][h*64 : h*64+64] (bf16 in and out)
hipError_t launch_absorb_q(const void* q, const void* wkt, int M, int H, int d, void* qp, hipStream_t s);
// Work split of the attention over E: the M rows' frames as one sequence of
// G = M * nsub sub-tiles of 16 frames, cut into n_wg even shares (one per
// workgroup); a share touches at most kmax rows and leaves one partial per row
// segment, in slot w * kmax + (row - the share's first row).
struct XePlan { int nsub; long G; int n_wg, kmax; };
void cross_enc_plan(int M, int T, int n_cu, XePlan& p);
// unnormalised U [n_wg * kmax][H][d] bf16 and (max, sum) [n_wg * kmax][H][2];
// query row m reads encoder row m / rows_per_b of E [B][T][d]; reverse != 0:
// each share is walked last sub-tile first
hipError_t launch_attn_cross_enc(const void* qp, const void* E, int M, int H, int T, int d, int rows_per_b,
                                 const XePlan& plan, int reverse, void* upart, float* ml, hipStream_t s);
// u [M][H][d] bf16 = each row's segments combined with their softmax weights
hipError_t launch_absorb_combine(const void* upart, const float* ml, int M, int H, int d, const XePlan& plan, void* u,
                                 hipStream_t s);

// ------------------------------------------------------------------ LayerNorm
// h is in the activation type (or fp32 when h_f32); residual and total are the
// fp32 residual stream; normed is in the activation type.
// row_amax (optional, needs normed): per row, max |normed| as stored
hipError_t launch_layernorm(ActType t, bool h_f32, const void* h, const float* res, const float* g, const float* b,
                            float eps, int M, int d, void* normed, float* total, hipStream_t s,
                            float* row_amax = nullptr);

// ------------------------------------------------------------------ fp8 codec
// fmt: FP8_E4M3 or FP8_E5M2 (common.hpp); the amax scale divides by that
// format's largest finite magnitude (448 or 57344).
hipError_t launch_amax(ActType t, int fmt, const void* x, size_t n, float* partial, int n_partial, float* scale_out,
                       hipStream_t s);
hipError_t launch_fp8_quantize(ActType t, int fmt, const void* x, size_t n, const float* scale, uint8_t* codes,
                               hipStream_t s);
hipError_t launch_fp8_dequantize(ActType t, int fmt, const uint8_t* codes, size_t n, const float* scale, void* y,
                                 hipStream_t s);
// bf16 x [rows, K] -> E4M3 codes with one amax scale per chunk of
// rows_per_chunk rows; partial: 64 floats per chunk; scales: one per chunk.
// launch_chunk_quant_fp8 for an activation whose rows' max |x| are known
hipError_t launch_chunk_quant_rows_fp8(const void* x, long rows, int K, int rows_per_chunk, const float* row_amax,
                                       float* scales, uint8_t* codes, hipStream_t s);
hipError_t launch_chunk_quant_fp8(const void* x, long rows, int K, int rows_per_chunk, float* partial,
                                  float* scales, uint8_t* codes, hipStream_t s);

// ------------------------------------------------------------------ attention
// Encoder self-attention over the packed QKV [B*T, 3*H*64] -> out [B*T, H*64].
hipError_t launch_attn_encoder(ActType t, const void* qkv, int B, int T, int H, void* out, hipStream_t s);
// Decode causal self-attention over e4m3 codes [B][H][cap][64]; n_keys[b] = lengths[b] + add.
// rows_per_b (R): query row m reads cache batch row m / R and attends over
// n = lengths[m / R] + len_add + m % R keys (B = query rows)
// fmt: code format of k_codes / v_codes (FP8_E4M3 for the KV cache; either
// format for fp8 cross-attention K/V). order (R = 1 only; NULL: row order):
// B (row, length) pairs, longest first, as launch_embed writes them; the
// workgroups then take the rows in that order with the lengths given there.
hipError_t launch_attn_decode_self(ActType t, const void* q, long q_stride, const uint8_t* k_codes,
                                   const uint8_t* v_codes, const float* scales, const int32_t* lengths,
                                   int len_add, int B, int H, int cap, void* out, hipStream_t s, int rows_per_b = 1,
                                   int fmt = 0, const int2* order = nullptr);
// Decode cross-attention over head-major K/V [B / R][H][T][64] (query row m
// reads K/V batch row m / R, R = rows_per_b); one pass per (row, head).
hipError_t launch_attn_decode_cross(ActType t, const void* q, const void* k, const void* v, int B, int H, int T,
                                    void* out, hipStream_t s, int rows_per_b = 1);

// ------------------------------------------------------------------ log-mel
size_t logmel_ws(int B, int n_mels);
// row_stride / total: chunk b starts at audio + b * row_stride, total samples
// from audio[0] (row_stride <= 0: separate clips of n_samples each)
hipError_t launch_logmel(const float* audio, int B, int n_samples, int n_mels, float* mel_out, void* ws,
                         hipStream_t s, long row_stride = 0, long total = 0);

// ------------------------------------------------------------------ misc
hipError_t launch_mel_to_conv_input(ActType t, const float* mel, int B, int n_mels, int n_frames, void* x0,
                                    hipStream_t s);
hipError_t launch_zero_rows(ActType t, void* base, long row_elems, long rows_per_batch, int B, int row_a,
                            int row_b, hipStream_t s);
hipError_t launch_convert(ActType t, const float* src, void* dst, size_t n, hipStream_t s);
hipError_t launch_pack_conv(ActType t, const float* w, int c_out, int c_in, int k, void* dst, hipStream_t s);
hipError_t launch_sinusoids(float* pe, int T, int C, hipStream_t s);
hipError_t launch_fill_f32(float* dst, float v, size_t n, hipStream_t s);
hipError_t launch_copy_f32(const float* src, float* dst, size_t n, hipStream_t s);
hipError_t launch_embed(ActType t, const void* tok_emb, const void* pos_emb, const int32_t* tokens,
                        const int32_t* lengths, int B, int d, int n_vocab, int n_ctx, int cap, float* x,
                        int32_t* dev_error, hipStream_t s, int32_t* zero = nullptr, int n_zero = 0,
                        int x_tiled = 0, int rows_per_b = 1, int2* order = nullptr);  // x_tiled: x in the 16-row tiles of dec_x_index;
                        // rows_per_b (R): B rows, row m is token m of batch row m / R at lengths[m / R] + m % R;
                        // order (R = 1 only; NULL: off): [B] (row, lengths[row]) ranked longest first, ties by row
hipError_t launch_argmax_part(const int2* part, int B, int NB, int32_t* argmax, int32_t* lengths, hipStream_t s,
                              int len_inc = 1);
hipError_t launch_argmax(const float* logits, int B, int V, int32_t* argmax, int32_t* lengths, hipStream_t s,
                         int len_inc = 1);
// fp32 rows [M, d] (row-major) to the 16-row tiles of dec_x_index (to_tiles
// != 0), or back; d % 32 == 0
hipError_t launch_x_tiles(const float* src, float* dst, int M, int d, int to_tiles, hipStream_t s);
// x_dst row b = x_src row b * R + R - 1 (both in the 16-row tiles of dec_x_index)
hipError_t launch_gather_last_rows(const float* x_src, float* x_dst, int B, int R, int d, hipStream_t s);

// measured ceilings (peak.hip)
hipError_t launch_peak_mfma(int n_wg, int iters, float* out, hipStream_t s);
hipError_t launch_peak_read(const void* buf, size_t bytes, int n_wg, float* out, hipStream_t s);
double peak_mfma_flop(int n_wg, int iters);

}  // namespace wh
