// C-ABI host layer: argument validation, packed-weight and workspace layout,
// and the launch sequences of log-mel, encoder, cross K/V and decoder step.
// All checks run before the first launch; nothing throws across the ABI.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "internal.hpp"
#include "whisper_mi355x.h"

static_assert((int)WHISPER_FP8_E4M3 == (int)wh::FP8_E4M3 && (int)WHISPER_FP8_E5M2 == (int)wh::FP8_E5M2,
              "public fp8 format values must match the kernels' template values");

using namespace wh;

namespace {

thread_local std::string g_err;

whisper_status fail(whisper_status st, const std::string& msg) {
  g_err = msg;
  return st;
}

#define WH_TRY(expr)                                                                                \
  do {                                                                                              \
    hipError_t e_ = (expr);                                                                         \
    if (e_ != hipSuccess) return fail(WHISPER_ERR_HIP, std::string(#expr) + ": " + hipGetErrorString(e_)); \
  } while (0)

#define WH_CHECK(st)                   \
  do {                                 \
    whisper_status s_ = (st);          \
    if (s_ != WHISPER_OK) return s_;   \
  } while (0)

size_t al256(size_t x) { return (x + 255) & ~size_t(255); }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
ActType act_of(whisper_dtype t) { return t == WHISPER_BF16 ? ACT_BF16 : ACT_F32; }
size_t esz(whisper_dtype t) { return t == WHISPER_BF16 ? 2 : 4; }
hipStream_t S(void* s) { return (hipStream_t)s; }

constexpr int N_FRAMES = 3000;  // STFT frames per 30 s chunk; the conv stem halves them

whisper_status check_dims(const whisper_dims* d) {
  if (!d) return fail(WHISPER_ERR_INVALID_ARG, "dims is NULL");
  if (d->act != WHISPER_F32 && d->act != WHISPER_BF16) return fail(WHISPER_ERR_DTYPE, "dims->act must be F32 or BF16");
  if (d->head_dim != 64) return fail(WHISPER_ERR_SHAPE, "head_dim must be 64");
  if (d->n_heads <= 0 || d->n_heads * 64 != d->d_model) return fail(WHISPER_ERR_SHAPE, "n_heads * 64 must equal d_model");
  if (d->d_model > 2048) return fail(WHISPER_ERR_SHAPE, "d_model must be <= 2048");
  if (d->d_ffn <= 0 || d->d_ffn % 128) return fail(WHISPER_ERR_SHAPE, "d_ffn must be a positive multiple of 128");
  if (d->n_enc_layers < 0 || d->n_dec_layers < 0) return fail(WHISPER_ERR_SHAPE, "layer counts must be >= 0");
  if (d->n_audio_ctx <= 0 || d->n_audio_ctx * 2 != N_FRAMES) return fail(WHISPER_ERR_SHAPE, "n_audio_ctx must be 1500");
  if (d->n_mels <= 0 || d->n_mels > 512) return fail(WHISPER_ERR_SHAPE, "n_mels must be in 1..512");
  if (d->act == WHISPER_BF16 && (3 * d->n_mels) % 64) return fail(WHISPER_ERR_SHAPE, "bf16 needs 3*n_mels % 64 == 0");
  if (d->n_dec_layers > 0 && (d->n_vocab <= 0 || d->n_text_ctx <= 0)) return fail(WHISPER_ERR_SHAPE, "decoder needs n_vocab, n_text_ctx > 0");
  return WHISPER_OK;
}

// ------------------------------------------------------------------ packed layout
struct EncL { size_t ln1g, ln1b, wqkv, bqkv, wo, bo, ln2g, ln2b, w1, b1, w2, b2; };
// In bf16 mode the LayerNorm-consumer weights of the decoder (wqkv, wqc, w1
// and the vocabulary projection lmw) are stored gamma-folded, their biases
// beta-folded, with the row sums c1* beside them (see decode_gemm.hip), and
// all decoder GEMM weights (those and wo, woc, w2) are in the MFMA fragment
// order of decode_gemm.hip rather than row-major.
// bf16 mode also keeps, per layer, the cross-attention key weight transposed
// per head (wkt, [H][d][64]) and the value weight in fragment order (wvf), for
// the cross-attention over the encoder output (cross_enc.hip).
struct DecL {
  size_t ln1g, ln1b, wqkv, bqkv, wo, bo, ln2g, ln2b, wqc, bqc, woc, boc, ln3g, ln3b, w1, b1, w2, b2;
  size_t c1qkv = 0, c1qc = 0, c1w1 = 0, wkt = 0, wvf = 0;
};
struct Packed {
  size_t conv1w = 0, conv1b = 0, conv2w = 0, conv2b = 0, pe = 0, lnpg = 0, lnpb = 0;
  std::vector<EncL> enc;
  size_t tok = 0, pos = 0, ckvw = 0, ckvb = 0, lnfg = 0, lnfb = 0, lmw = 0, lmc1 = 0, lmb2 = 0;
  std::vector<DecL> dec;
  size_t total = 0;
};

Packed layout(const whisper_dims* d) {
  Packed P;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = al256(off + bytes); return o; };
  const size_t e = esz(d->act), D = d->d_model, F = d->d_ffn, f4 = 4;
  if (d->n_enc_layers > 0) {
    P.conv1w = take(D * 3 * d->n_mels * e); P.conv1b = take(D * f4);
    P.conv2w = take(D * 3 * D * e); P.conv2b = take(D * f4);
    P.pe = take((size_t)d->n_audio_ctx * D * f4);
    for (int l = 0; l < d->n_enc_layers; ++l) {
      EncL L;
      L.ln1g = take(D * f4); L.ln1b = take(D * f4);
      L.wqkv = take(3 * D * D * e); L.bqkv = take(3 * D * f4);
      L.wo = take(D * D * e); L.bo = take(D * f4);
      L.ln2g = take(D * f4); L.ln2b = take(D * f4);
      L.w1 = take(F * D * e); L.b1 = take(F * f4);
      L.w2 = take(D * F * e); L.b2 = take(D * f4);
      P.enc.push_back(L);
    }
    P.lnpg = take(D * f4); P.lnpb = take(D * f4);
  }
  if (d->n_dec_layers > 0) {
    P.tok = take((size_t)d->n_vocab * D * e);
    P.pos = take((size_t)d->n_text_ctx * D * e);
    for (int l = 0; l < d->n_dec_layers; ++l) {
      DecL L;
      L.ln1g = take(D * f4); L.ln1b = take(D * f4);
      L.wqkv = take(3 * D * D * e); L.bqkv = take(3 * D * f4);
      L.wo = take(D * D * e); L.bo = take(D * f4);
      L.ln2g = take(D * f4); L.ln2b = take(D * f4);
      L.wqc = take(D * D * e); L.bqc = take(D * f4);
      L.woc = take(D * D * e); L.boc = take(D * f4);
      L.ln3g = take(D * f4); L.ln3b = take(D * f4);
      L.w1 = take(F * D * e); L.b1 = take(F * f4);
      L.w2 = take(D * F * e); L.b2 = take(D * f4);
      if (d->act == WHISPER_BF16) {
        L.c1qkv = take(3 * D * f4); L.c1qc = take(D * f4); L.c1w1 = take(F * f4);
        L.wkt = take(D * D * e); L.wvf = take(D * D * e);
      }
      P.dec.push_back(L);
    }
    P.ckvw = take((size_t)d->n_dec_layers * 2 * D * D * e);
    P.ckvb = take((size_t)d->n_dec_layers * 2 * D * f4);
    P.lnfg = take(D * f4); P.lnfb = take(D * f4);
    if (d->act == WHISPER_BF16) {
      P.lmw = take((size_t)((d->n_vocab + 15) & ~15) * D * e);  // rows padded to the 16-row fragment
      P.lmc1 = take((size_t)d->n_vocab * f4);
      P.lmb2 = take((size_t)d->n_vocab * f4);
    }
  }
  P.total = off;
  return P;
}

int weight_count(const whisper_dims* d) {
  return (d->n_enc_layers > 0 ? 4 + 15 * d->n_enc_layers + 2 : 0) + (d->n_dec_layers > 0 ? 2 + 24 * d->n_dec_layers + 2 : 0);
}

// ------------------------------------------------------------------ workspace layout
struct EncWS { size_t x0, g1, x, a, dlt, qkv, att, hf, codes, part, ascale, rowmax, total; };
EncWS enc_ws(const whisper_dims* d, int B, bool fp8 = false) {
  EncWS W{};
  const size_t e = esz(d->act), D = d->d_model, T = d->n_audio_ctx, rows = (size_t)B * T;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = al256(off + bytes); return o; };
  W.x = take(rows * D * 4);  // fp32 residual stream
  W.a = take(rows * D * e);
  W.dlt = take(rows * D * e);
  W.att = take(rows * D * e);
  const size_t qkv_b = std::max(rows * 3 * D * e, (size_t)B * (N_FRAMES + 2) * d->n_mels * e);
  W.qkv = take(qkv_b);
  W.x0 = W.qkv;  // conv1 input lives in the QKV buffer before the first block
  const size_t hf_b = std::max(rows * d->d_ffn * e, (size_t)B * (N_FRAMES + 2) * D * e);
  W.hf = take(hf_b);
  W.g1 = W.hf;   // conv1 output lives in the MLP buffer before the first block
  if (fp8) {     // E4M3 codes of the activation entering an fp8 site, per-chunk amax partials and scales,
                 // and the LayerNorm outputs' row maxima
    W.codes = take(rows * std::max((size_t)d->d_ffn, D));
    W.part = take((size_t)B * 64 * 4);
    W.ascale = take((size_t)B * 4);
    W.rowmax = take(rows * 4);
  }
  W.total = off;
  return W;
}

// E4M3 weights of the mixed_fp8 sites. Encoder, per layer: query, key, value
// codes [3d, d] (one block, as the fused QKV), fc1 [f, d], fc2 [d, f]; then
// per layer 8 fp32 scales (query, key, value, fc1, fc2, 3 unused). Decoder
// MLP, per layer: fc1 codes [f, d] and fc2 codes [d, f] in the decode GEMM's
// fragment order, fc1's bias [f] fp32 (unfolded: the fp8 site takes LN(x)
// explicitly); then per layer 2 fp32 scales (fc1, fc2).
struct Packed8 {
  std::vector<size_t> qkv, w1, w2, dw1, dw2, db1;
  size_t scales = 0, dscales = 0, total = 0;
};
Packed8 layout8(const whisper_dims* d) {
  Packed8 P;
  const size_t D = d->d_model, F = d->d_ffn;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = al256(off + bytes); return o; };
  for (int l = 0; l < d->n_enc_layers; ++l) {
    P.qkv.push_back(take(3 * D * D));
    P.w1.push_back(take(F * D));
    P.w2.push_back(take(D * F));
  }
  P.scales = take((size_t)std::max(d->n_enc_layers, 1) * 8 * 4);
  const size_t F16 = (F + 15) & ~(size_t)15, D16 = (D + 15) & ~(size_t)15;  // whole 16-row fragments
  for (int l = 0; l < d->n_dec_layers; ++l) {
    P.dw1.push_back(take(F16 * D));
    P.dw2.push_back(take(D16 * F));
    P.db1.push_back(take(F * 4));
  }
  P.dscales = take((size_t)std::max(d->n_dec_layers, 1) * 2 * 4);
  P.total = off;
  return P;
}

// The MLP down-projection (K = d_ffn) runs split-K over DEC_KSPLIT workgroups
// per 16 x 80 output tile; its partials and tile counters live here.
constexpr int DEC_KSPLIT = 4, DEC_SPLIT_COLS = 80;
struct DecWS { size_t x, a, dlt, q, att, qc, hf, logits, part, cnt, n_cnt, xg, amx, order, total; };
DecWS dec_ws(const whisper_dims* d, int B, bool with_logits = true) {
  DecWS W;
  const size_t e = esz(d->act), D = d->d_model;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = al256(off + bytes); return o; };
  W.x = take((size_t)((B + 15) & ~15) * D * 4);  // bf16 path: 16-row tiles (dec_x_index)
  W.a = take(B * D * e); W.dlt = take(B * D * e); W.q = take(B * D * e);
  W.att = take(B * D * e); W.qc = take(B * D * e);
  W.hf = take((size_t)B * d->d_ffn * e);
  W.logits = with_logits ? take((size_t)B * d->n_vocab * 4) : 0;
  const size_t tiles = (size_t)((D + DEC_SPLIT_COLS - 1) / DEC_SPLIT_COLS) * ((B + 15) / 16);
  W.part = take(tiles * DEC_KSPLIT * (DEC_SPLIT_COLS / 16) * 64 * 16);
  W.n_cnt = tiles;
  W.cnt = take(tiles * 4);
  W.xg = take((size_t)((B + 15) & ~15) * D * 4);  // prefill: the last position of each batch row, 16-row tiles
  W.amx = take((size_t)B * ((d->n_vocab + 15) / 16) * 8);  // argmax: per-row maxima of 16-column blocks
  W.order = take((size_t)B * 8);  // rows by cache length, longest first (row, length)
  W.total = off;
  return W;
}

// Cross-attention over the encoder output (decode_step_enc): q' [M][H][d],
// the row-segment partials U [n_wg * kmax][H][d] bf16 and (max, sum)
// [n_wg * kmax][H][2] fp32, and the combined u [M][H][d], after the step's own
// workspace.
constexpr int XE_CU = 256;  // compute units the frame sequence is shared over
// With the decoder MLP as mixed_fp8 sites (fp8): the quantised LN(x) rows
// [M][d] bf16, their scales [M], and the hidden rows' 16-column block maxima
// [M][f / 16] (rewritten by each layer's up-projection).
struct DecEncWS { DecWS base; size_t qp, upart, ml, u, aq = 0, srow = 0, amx8 = 0, total; XePlan plan; };
DecEncWS dec_ws_enc(const whisper_dims* d, int M, bool fp8 = false) {
  DecEncWS W;
  W.base = dec_ws(d, M);
  size_t off = W.base.total;
  auto take = [&](size_t bytes) { size_t o = off; off = al256(off + bytes); return o; };
  cross_enc_plan(M, d->n_audio_ctx, XE_CU, W.plan);
  const size_t rows = (size_t)M * d->n_heads * d->d_model;
  const size_t slots = (size_t)W.plan.n_wg * W.plan.kmax;
  W.qp = take(rows * 2);
  W.upart = take(slots * d->n_heads * d->d_model * 2);
  W.ml = take(slots * d->n_heads * 2 * 4);
  W.u = take(rows * 2);
  if (fp8) {
    W.aq = take((size_t)M * d->d_model * 2);
    W.srow = take((size_t)M * 4);
    W.amx8 = take((size_t)M * (d->d_ffn / 16) * 4);
  }
  W.total = off;
  return W;
}

template <typename T> T* at(const void* base, size_t off) { return (T*)((char*)base + off); }

// ------------------------------------------------------------------ measurement hook
// Process-wide and not thread-safe by design: a measurement harness arms it,
// runs its timed region, and disarms it.
struct Profile {
  int kind = 0;
  hipEvent_t* start = nullptr;
  hipEvent_t* stop = nullptr;
  int cap = 0, n = 0;
};
Profile g_prof;

struct ProfScope {
  bool on;
  hipStream_t s;
  int i;
  ProfScope(int kind, hipStream_t s_) : on(g_prof.kind == kind && g_prof.n < g_prof.cap), s(s_), i(g_prof.n) {
    if (on) hipEventRecord(g_prof.start[i], s);
  }
  ~ProfScope() {
    if (on) { hipEventRecord(g_prof.stop[i], s); g_prof.n = i + 1; }
  }
};

// ------------------------------------------------------------------ KV-append debug hook
// While armed, the QKV epilogue of every decode call also stores the fp32 K / V
// values its fp8 codec is applied to (parity tests check the codec bit for bit
// on them). Process-wide and not thread-safe, like the measurement hook.
struct KvTrace {
  float* buf = nullptr;          // fp32 values the codec is applied to
  const int16_t* force = nullptr;  // codes written instead of the kernel's own (>= 0)
  size_t cap = 0;                // elements of each buffer
};
KvTrace g_kvtrace;

// The hook's buffers must hold [n_layers][2][rows][d_model] elements; checked
// before the first launch of a call.
whisper_status kvtrace_check(int n_layers, long rows, int d_model, const char* who) {
  if (!g_kvtrace.buf && !g_kvtrace.force) return WHISPER_OK;
  const size_t need = (size_t)n_layers * 2 * rows * d_model;
  if (need > g_kvtrace.cap)
    return fail(WHISPER_ERR_WORKSPACE, std::string(who) + ": the armed K/V debug buffers hold " +
                                           std::to_string(g_kvtrace.cap) + " elements, need " + std::to_string(need));
  return WHISPER_OK;
}

// ------------------------------------------------------------------ GEMM helpers
GemmParams gp(const void* A, long lda, const void* B, long ldb, int M, int N, int K, const float* bias, void* C,
              long ldc) {
  GemmParams p{};
  p.A = A; p.lda = lda; p.B = B; p.ldb = ldb; p.M = M; p.N = N; p.K = K; p.batch = 1;
  p.bias = bias; p.C = C; p.ldc = ldc;
  return p;
}

// ------------------------------------------------------------------ encoder blocks
// The residual stream X is fp32 in the workspace. `h_in` is either that
// buffer already holding the stem output (in_is_x) or caller hidden states in
// the activation type, which the first LayerNorm copies into X.
// packed8 non-NULL: the mixed_fp8 sites (query, key, value, fc1, fc2) run as
// E4M3 GEMMs on the per-chunk quantised activation (W from enc_ws(d, B, true)).
whisper_status run_enc_layers(const whisper_dims* d, const void* packed, const Packed& P, const EncWS& W,
                              const void* h_in, bool in_is_x, int B, int l0, int l1, bool ln_post, void* out,
                              void* ws, hipStream_t s, const void* packed8 = nullptr) {
  const ActType t = act_of(d->act);
  const int D = d->d_model, T = d->n_audio_ctx, M = B * T, F = d->d_ffn;
  float* X = at<float>(ws, W.x);
  void* A = at<void>(ws, W.a);
  void* Dl = at<void>(ws, W.dlt);
  void* QKV = at<void>(ws, W.qkv);
  void* ATT = at<void>(ws, W.att);
  void* HF = at<void>(ws, W.hf);
  const Packed8 P8 = packed8 ? layout8(d) : Packed8{};
  bool x_ready = in_is_x;  // X holds the residual stream
  bool have_delta = false; // Dl holds a block output not yet added to X
  for (int l = l0; l < l1; ++l) {
    const EncL& L = P.enc[l];
    const float* g1 = at<float>(packed, L.ln1g);
    const float* b1 = at<float>(packed, L.ln1b);
    // fp8 sites: the LayerNorm also leaves each row's max |output|, from which
    // the quantiser takes the chunk's scale without a pass of its own
    float* ROWMAX = packed8 ? at<float>(ws, W.rowmax) : nullptr;
    if (have_delta)
      WH_TRY(launch_layernorm(t, false, Dl, X, g1, b1, 1e-5f, M, D, A, X, s, ROWMAX));
    else if (x_ready)
      WH_TRY(launch_layernorm(t, true, X, nullptr, g1, b1, 1e-5f, M, D, A, nullptr, s, ROWMAX));
    else
      WH_TRY(launch_layernorm(t, false, h_in, nullptr, g1, b1, 1e-5f, M, D, A, X, s, ROWMAX));
    x_ready = true;
    const float* sc8 = packed8 ? at<float>(packed8, P8.scales) + 8 * l : nullptr;
    uint8_t* CODES = packed8 ? at<uint8_t>(ws, W.codes) : nullptr;
    float* PART = packed8 ? at<float>(ws, W.part) : nullptr;
    float* ASC = packed8 ? at<float>(ws, W.ascale) : nullptr;
    // one fp8 site: C[:, col0:col0+N] = epi(e4m3(A) . W8^T * sa * sw + bias)
    auto fp8_site = [&](Epi epi, const uint8_t* w8, const float* sw, int N, int K, const float* bias, void* C,
                        long ldc) -> hipError_t {
      GemmParams g = gp(CODES, K, w8, K, M, N, K, bias, C, ldc);
      g.a_scale = ASC; g.a_rows_per_scale = T; g.b_scale = sw;
      return launch_gemm_fp8(epi, g, s);
    };
    if (packed8) {
      const uint8_t* q8 = at<uint8_t>(packed8, P8.qkv[l]);
      const float* bq = at<float>(packed, L.bqkv);
      WH_TRY(launch_chunk_quant_rows_fp8(A, M, D, T, ROWMAX, ASC, CODES, s));
      for (int r = 0; r < 3; ++r)  // query, key, value: one weight scale each
        WH_TRY(fp8_site(EPI_STORE, q8 + (size_t)r * D * D, sc8 + r, D, D, bq + r * D, (u16_t*)QKV + r * D, 3 * D));
    } else {
      WH_TRY(launch_gemm(t, EPI_STORE, gp(A, D, at<void>(packed, L.wqkv), D, M, 3 * D, D, at<float>(packed, L.bqkv), QKV, 3 * D), s));
    }
    {
      ProfScope ps(WHISPER_PROF_ENCODER_ATTENTION, s);
      WH_TRY(launch_attn_encoder(t, QKV, B, T, d->n_heads, ATT, s));
    }
    WH_TRY(launch_gemm(t, EPI_STORE, gp(ATT, D, at<void>(packed, L.wo), D, M, D, D, at<float>(packed, L.bo), Dl, D), s));
    {
      ProfScope ps(WHISPER_PROF_ENCODER_LAYERNORM, s);
      WH_TRY(launch_layernorm(t, false, Dl, X, at<float>(packed, L.ln2g), at<float>(packed, L.ln2b), 1e-5f, M, D, A, X, s,
                              ROWMAX));
    }
    if (packed8) {
      WH_TRY(launch_chunk_quant_rows_fp8(A, M, D, T, ROWMAX, ASC, CODES, s));
      {
        ProfScope ps(WHISPER_PROF_ENCODER_FFN1, s);
        WH_TRY(fp8_site(EPI_GELU, at<uint8_t>(packed8, P8.w1[l]), sc8 + 3, F, D, at<float>(packed, L.b1), HF, F));
      }
      WH_TRY(launch_chunk_quant_fp8(HF, M, F, T, PART, ASC, CODES, s));
      WH_TRY(fp8_site(EPI_STORE, at<uint8_t>(packed8, P8.w2[l]), sc8 + 4, D, F, at<float>(packed, L.b2), Dl, D));
    } else {
      {
        ProfScope ps(WHISPER_PROF_ENCODER_FFN1, s);
        WH_TRY(launch_gemm(t, EPI_GELU, gp(A, D, at<void>(packed, L.w1), D, M, F, D, at<float>(packed, L.b1), HF, F), s));
      }
      WH_TRY(launch_gemm(t, EPI_STORE, gp(HF, F, at<void>(packed, L.w2), F, M, D, F, at<float>(packed, L.b2), Dl, D), s));
    }
    have_delta = true;
  }
  const float* gp_ = at<float>(packed, P.lnpg);
  const float* bp_ = at<float>(packed, P.lnpb);
  if (ln_post) {
    if (have_delta) WH_TRY(launch_layernorm(t, false, Dl, X, gp_, bp_, 1e-5f, M, D, out, nullptr, s));
    else if (x_ready) WH_TRY(launch_layernorm(t, true, X, nullptr, gp_, bp_, 1e-5f, M, D, out, nullptr, s));
    else WH_TRY(launch_layernorm(t, false, h_in, nullptr, gp_, bp_, 1e-5f, M, D, out, nullptr, s));
  } else {
    if (have_delta) WH_TRY(launch_layernorm(t, false, Dl, X, gp_, bp_, 1e-5f, M, D, nullptr, X, s));
    else if (!x_ready) WH_TRY(launch_layernorm(t, false, h_in, nullptr, gp_, bp_, 1e-5f, M, D, nullptr, X, s));
    WH_TRY(launch_convert(t, X, out, (size_t)M * D, s));
  }
  return WHISPER_OK;
}

whisper_status check_ptrs(std::initializer_list<const void*> ps, const char* what) {
  for (const void* p : ps) {
    if (!p) return fail(WHISPER_ERR_INVALID_ARG, std::string(what) + ": NULL pointer");
    if (!aligned16(p)) return fail(WHISPER_ERR_ALIGN, std::string(what) + ": pointer not 16-byte aligned");
  }
  return WHISPER_OK;
}

// Small index / scale arrays only need their element alignment.
whisper_status check_ptrs4(std::initializer_list<const void*> ps, const char* what) {
  for (const void* p : ps) {
    if (!p) return fail(WHISPER_ERR_INVALID_ARG, std::string(what) + ": NULL pointer");
    if ((uintptr_t)p & 3u) return fail(WHISPER_ERR_ALIGN, std::string(what) + ": pointer not 4-byte aligned");
  }
  return WHISPER_OK;
}

whisper_status check_ws(void* ws, size_t have, size_t need, const char* what) {
  if (need > have) return fail(WHISPER_ERR_WORKSPACE, std::string(what) + ": workspace of " + std::to_string(have) +
                                                          " bytes, need " + std::to_string(need));
  if (need && !ws) return fail(WHISPER_ERR_INVALID_ARG, std::string(what) + ": workspace is NULL");
  if (ws && !aligned16(ws)) return fail(WHISPER_ERR_ALIGN, std::string(what) + ": workspace not 16-byte aligned");
  return WHISPER_OK;
}

// Decoder step in bf16 with the residual + LayerNorm folded into the GEMMs:
// per layer QKV + cache append, self-attention, out-proj + residual,
// cross-query, cross-attention (over cross K/V: one launch; over the encoder
// output: query absorption, attention, combine, value projection), cross-out
// + residual, MLP up, MLP down + residual; then the vocabulary projection,
// whose epilogue also takes per-block row maxima, and the argmax over those.
// The residual stream stays fp32.
whisper_status decode_step_fused(const whisper_dims* d, const void* packed, const Packed& P, const DecWS& W, int B,
                                 int cap, const int32_t* tokens, int32_t* lengths, uint8_t* kv_cache,
                                 const float* kv_scales, const void* cross_kv, float* LG, int32_t* argmax,
                                 int32_t* dev_error, void* ws, hipStream_t s, const uint8_t* xcodes = nullptr,
                                 const float* xscales = nullptr, int R = 1, int xfmt = FP8_E4M3,
                                 const void* enc = nullptr, const DecEncWS* XW = nullptr,
                                 const void* packed8 = nullptr) {
  // B batch rows of the cache; R tokens per row (a prefill when R > 1): the
  // activations have B * R rows, row m being token m % R of batch row m / R
  const int Bc = B;
  B = Bc * R;
  const int D = d->d_model, H = d->n_heads, T = d->n_audio_ctx, F = d->d_ffn, L = d->n_dec_layers;
  float* X = at<float>(ws, W.x);
  u16_t* Q = at<u16_t>(ws, W.q);
  u16_t* ATT = at<u16_t>(ws, W.att);
  u16_t* QC = at<u16_t>(ws, W.qc);
  u16_t* HF = at<u16_t>(ws, W.hf);
  int32_t* CNT = at<int32_t>(ws, W.cnt);
  WH_CHECK(kvtrace_check(L, B, D, "decode"));
  int2* ORD = R == 1 ? at<int2>(ws, W.order) : nullptr;
  WH_TRY(launch_embed(ACT_BF16, at<void>(packed, P.tok), at<void>(packed, P.pos), tokens, lengths, B, D, d->n_vocab,
                      d->n_text_ctx, cap, X, dev_error, s, CNT, (int)W.n_cnt, 1, R, ORD));
  const Packed8 P8 = packed8 ? layout8(d) : Packed8{};
  auto gemm = [&](DecPro pro, DecEpi epi, size_t w_off, size_t b_off, size_t c1_off, int N, int K, const u16_t* A,
                  u16_t* out, float* out_f32, int layer, bool split = false, int a_group = 0) {
    DecGemmParams g{};
    g.M = B; g.N = N; g.K = K;
    g.W = at<u16_t>(packed, w_off);
    g.bias = b_off ? at<float>(packed, b_off) : nullptr;
    g.c1 = c1_off ? at<float>(packed, c1_off) : nullptr;
    g.A = A; g.lda = K; g.X = X; g.out = out; g.out_f32 = out_f32;
    if (a_group) {  // A is u [M][H][d]: output column n reads head n / a_group's row
      g.a_group = a_group; g.a_group_stride = K; g.lda = (long)H * K;
    }
    g.kv_cache = kv_cache; g.kv_scales = kv_scales; g.lengths = lengths; g.dev_error = dev_error;
    g.kv_cap = cap; g.kv_B = Bc; g.kv_H = H; g.kv_layer = layer; g.d_model = D; g.rows_per_b = R;
    g.kv_pre = epi == DEPI_QKV ? g_kvtrace.buf : nullptr;
    g.kv_force = epi == DEPI_QKV ? g_kvtrace.force : nullptr;
    g.amax_part = epi == DEPI_F32 ? at<int2>(ws, W.amx) : nullptr;  // the vocabulary projection
    int mb, cb;
    dec_gemm_tiles(B, N, mb, cb);
    // split-K where the long K would otherwise leave a third of the CUs idle
    // with 490 KB per busy one (the MLP down-projection)
    if (split && pro == PRO_A && N % DEC_SPLIT_COLS == 0 && (K / 32) % (DEC_KSPLIT * 8) == 0) {
      g.ks = DEC_KSPLIT; g.part = at<float>(ws, W.part); g.cnt = CNT;
      mb = 1; cb = DEC_SPLIT_COLS / 16;
    }
    return launch_gemm_dec(pro, epi, g, mb, cb, s);
  };
  const size_t kv_layer = (size_t)2 * Bc * H * cap * 64;
  const size_t ckv_layer = (size_t)2 * Bc * H * T * 64 * 2;
  for (int l = 0; l < L; ++l) {
    const DecL& Lw = P.dec[l];
    WH_TRY(gemm(PRO_X, DEPI_QKV, Lw.wqkv, Lw.bqkv, Lw.c1qkv, 3 * D, D, nullptr, Q, nullptr, l));
    const uint8_t* kc = kv_cache + l * kv_layer;
    {
      ProfScope ps(WHISPER_PROF_DECODE_SELF_ATTENTION, s);
      WH_TRY(launch_attn_decode_self(ACT_BF16, Q, D, kc, kc + kv_layer / 2, kv_scales + 2 * l, lengths, 1, B, H, cap,
                                     ATT, s, R, FP8_E4M3, ORD));
    }
    WH_TRY(gemm(PRO_A, DEPI_RESID, Lw.wo, Lw.bo, 0, D, D, ATT, nullptr, nullptr, l));
    WH_TRY(gemm(PRO_X, DEPI_STORE, Lw.wqc, Lw.bqc, Lw.c1qc, D, D, nullptr, QC, nullptr, l));
    if (enc) {  // cross-attention over the encoder output: q' = W_k^T q per head, attention over E, W_v u + b_v
      WH_TRY(launch_absorb_q(QC, at<void>(packed, Lw.wkt), B, H, D, at<void>(ws, XW->qp), s));
      {
        ProfScope ps(WHISPER_PROF_DECODE_CROSS_ATTENTION, s);
        // odd layers walk the frames backwards: a layer first re-reads the part of E
        // the previous layer read last
        WH_TRY(launch_attn_cross_enc(at<void>(ws, XW->qp), enc, B, H, T, D, R, XW->plan, l & 1,
                                     at<void>(ws, XW->upart), at<float>(ws, XW->ml), s));
      }
      WH_TRY(launch_absorb_combine(at<void>(ws, XW->upart), at<float>(ws, XW->ml), B, H, D, XW->plan,
                                   at<void>(ws, XW->u), s));
      WH_TRY(gemm(PRO_A, DEPI_STORE, Lw.wvf, P.ckvb + ((size_t)l * 2 + 1) * D * 4, 0, D, D, at<u16_t>(ws, XW->u),
                  ATT, nullptr, l, false, 64));
    } else {
      ProfScope ps(WHISPER_PROF_DECODE_CROSS_ATTENTION, s);
      if (xcodes) {  // fp8 cross K/V: the fp8 attention kernel over all T keys of each row
        const uint8_t* xc = xcodes + l * (ckv_layer / 2);
        WH_TRY(launch_attn_decode_self(ACT_BF16, QC, D, xc, xc + ckv_layer / 4, xscales + 2 * l, nullptr, 0, B, H, T,
                                       ATT, s, R, xfmt));
      } else {
        const char* ck = (const char*)cross_kv + l * ckv_layer;
        WH_TRY(launch_attn_decode_cross(ACT_BF16, QC, ck, ck + ckv_layer / 2, B, H, T, ATT, s, R));
      }
    }
    WH_TRY(gemm(PRO_A, DEPI_RESID, Lw.woc, Lw.boc, 0, D, D, ATT, nullptr, nullptr, l));
    if (packed8) {
      // the MLP as mixed_fp8 sites: LN(x) quantised per row, fc1 with E4M3
      // weights + GELU (recording each hidden row's amax), fc2 quantising its
      // input rows in registers, split-K + residual
      u16_t* AQ = at<u16_t>(ws, XW->aq);
      float* SROW = at<float>(ws, XW->srow);
      float* AMX = at<float>(ws, XW->amx8);
      const float* dsc = at<float>(packed8, P8.dscales) + 2 * l;
      WH_TRY(launch_ln_quant_rows(X, at<float>(packed, Lw.ln3g), at<float>(packed, Lw.ln3b), B, D, AQ, SROW, s));
      DecGemmParams g1{};
      g1.M = B; g1.N = F; g1.K = D; g1.A = AQ; g1.lda = D; g1.X = X; g1.out = HF;
      g1.W8 = at<uint8_t>(packed8, P8.dw1[l]); g1.w_scale8 = dsc; g1.row_scale = SROW; g1.amax_out = AMX;
      g1.amax_nblk = F / 16;
      g1.bias = at<float>(packed8, P8.db1[l]);
      WH_TRY(launch_gemm_dec_fp8(DEPI_GELU, g1, s));
      DecGemmParams g2{};
      g2.M = B; g2.N = D; g2.K = F; g2.A = HF; g2.lda = F; g2.X = X;
      g2.W8 = at<uint8_t>(packed8, P8.dw2[l]); g2.w_scale8 = dsc + 1; g2.aq_part = AMX; g2.amax_nblk = F / 16;
      g2.bias = at<float>(packed, Lw.b2);
      g2.ks = DEC_KSPLIT; g2.part = at<float>(ws, W.part); g2.cnt = CNT;
      WH_TRY(launch_gemm_dec_fp8(DEPI_RESID, g2, s));
    } else {
      WH_TRY(gemm(PRO_X, DEPI_GELU, Lw.w1, Lw.b1, Lw.c1w1, F, D, nullptr, HF, nullptr, l));
      WH_TRY(gemm(PRO_A, DEPI_RESID, Lw.w2, Lw.b2, 0, D, F, HF, nullptr, nullptr, l, true));
    }
  }
  if (R > 1) {  // vocabulary projection and argmax of each batch row's last position only
    float* XG = at<float>(ws, W.xg);
    WH_TRY(launch_gather_last_rows(X, XG, Bc, R, D, s));
    X = XG;
    B = Bc;
  }
  WH_TRY(gemm(PRO_X, DEPI_F32, P.lmw, P.lmb2, P.lmc1, d->n_vocab, D, nullptr, nullptr, LG, 0));
  WH_TRY(launch_argmax_part(at<int2>(ws, W.amx), B, (d->n_vocab + 15) / 16, argmax, lengths, s, R));
  return WHISPER_OK;
}

}  // namespace

extern "C" {

const char* whisper_status_string(whisper_status st) {
  switch (st) {
    case WHISPER_OK: return "ok";
    case WHISPER_ERR_INVALID_ARG: return "invalid argument";
    case WHISPER_ERR_SHAPE: return "unsupported or inconsistent shape";
    case WHISPER_ERR_DTYPE: return "unsupported dtype";
    case WHISPER_ERR_ALIGN: return "pointer not 16-byte aligned";
    case WHISPER_ERR_WORKSPACE: return "workspace too small";
    case WHISPER_ERR_CAPACITY: return "KV cache capacity exceeded";
    case WHISPER_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

const char* whisper_last_error(void) { return g_err.c_str(); }

whisper_status whisper_profile_arm(int kind, void* const* start_events, void* const* stop_events, int capacity) {
  if (kind < WHISPER_PROF_DECODE_CROSS_ATTENTION || kind > WHISPER_PROF_ENCODER_LAYERNORM)
    return fail(WHISPER_ERR_INVALID_ARG, "profile_arm: unknown kernel kind");
  if (!start_events || !stop_events || capacity <= 0) return fail(WHISPER_ERR_INVALID_ARG, "profile_arm: no events");
  g_prof.kind = kind;
  g_prof.start = (hipEvent_t*)start_events;
  g_prof.stop = (hipEvent_t*)stop_events;
  g_prof.cap = capacity;
  g_prof.n = 0;
  return WHISPER_OK;
}

int whisper_profile_disarm(void) {
  const int n = g_prof.n;
  g_prof = Profile();
  return n;
}

whisper_status whisper_debug_kv_arm(float* kv_pre, const int16_t* kv_force, size_t n_elems) {
  if ((!kv_pre && !kv_force) || n_elems == 0)
    return fail(WHISPER_ERR_INVALID_ARG, "debug_kv_arm: no buffer or zero size");
  if (((uintptr_t)kv_pre & 3u) || ((uintptr_t)kv_force & 1u))
    return fail(WHISPER_ERR_ALIGN, "debug_kv_arm: buffer not aligned to its element");
  g_kvtrace.buf = kv_pre;
  g_kvtrace.force = kv_force;
  g_kvtrace.cap = n_elems;
  return WHISPER_OK;
}

void whisper_debug_kv_disarm(void) { g_kvtrace = KvTrace(); }

int whisper_weight_count(const whisper_dims* d) {
  if (check_dims(d) != WHISPER_OK) return 0;
  return weight_count(d);
}

size_t whisper_packed_weights_size(const whisper_dims* d) {
  if (check_dims(d) != WHISPER_OK) return 0;
  return layout(d).total;
}

whisper_status whisper_pack_weights(const whisper_dims* d, const float* const* w, void* packed, void* stream) {
  WH_CHECK(check_dims(d));
  if (!w) return fail(WHISPER_ERR_INVALID_ARG, "pack: weight table is NULL");
  WH_CHECK(check_ptrs({packed}, "pack"));
  const int n = weight_count(d);
  for (int i = 0; i < n; ++i) {
    if (!w[i]) return fail(WHISPER_ERR_INVALID_ARG, "pack: weight " + std::to_string(i) + " is NULL");
    if (((uintptr_t)w[i] & 3u) != 0) return fail(WHISPER_ERR_ALIGN, "pack: weight " + std::to_string(i) + " not 4-byte aligned");
  }
  (void)hipGetLastError();
  const Packed P = layout(d);
  const ActType t = act_of(d->act);
  const hipStream_t s = S(stream);
  const size_t D = d->d_model, F = d->d_ffn, e = esz(d->act);
  int i = 0;
  auto cvt = [&](const float* src, size_t off, size_t cnt) { return launch_convert(t, src, at<void>(packed, off), cnt, s); };
  auto cpy = [&](const float* src, size_t off, size_t cnt) { return launch_copy_f32(src, at<float>(packed, off), cnt, s); };
  // decoder GEMM weights: in bf16 mode the fused decode step reads them in
  // fragment order (decode_gemm.hip); the other dtypes keep them row-major
  auto dw = [&](const float* src, size_t off, size_t n_rows, size_t k) {
    return t == ACT_BF16 ? launch_pack_dec_weight(src, (int)n_rows, (int)k, at<void>(packed, off), s)
                         : cvt(src, off, n_rows * k);
  };
  if (d->n_enc_layers > 0) {
    WH_TRY(launch_pack_conv(t, w[i++], D, d->n_mels, 3, at<void>(packed, P.conv1w), s));
    WH_TRY(cpy(w[i++], P.conv1b, D));
    WH_TRY(launch_pack_conv(t, w[i++], D, D, 3, at<void>(packed, P.conv2w), s));
    WH_TRY(cpy(w[i++], P.conv2b, D));
    WH_TRY(launch_sinusoids(at<float>(packed, P.pe), d->n_audio_ctx, D, s));
    for (int l = 0; l < d->n_enc_layers; ++l) {
      const EncL& L = P.enc[l];
      WH_TRY(cpy(w[i + 0], L.ln1g, D)); WH_TRY(cpy(w[i + 1], L.ln1b, D));
      WH_TRY(cvt(w[i + 2], L.wqkv, D * D)); WH_TRY(cpy(w[i + 3], L.bqkv, D));
      WH_TRY(cvt(w[i + 4], L.wqkv + D * D * e, D * D));
      WH_TRY(launch_fill_f32(at<float>(packed, L.bqkv + D * 4), 0.f, D, s));
      WH_TRY(cvt(w[i + 5], L.wqkv + 2 * D * D * e, D * D)); WH_TRY(cpy(w[i + 6], L.bqkv + 2 * D * 4, D));
      WH_TRY(cvt(w[i + 7], L.wo, D * D)); WH_TRY(cpy(w[i + 8], L.bo, D));
      WH_TRY(cpy(w[i + 9], L.ln2g, D)); WH_TRY(cpy(w[i + 10], L.ln2b, D));
      WH_TRY(cvt(w[i + 11], L.w1, F * D)); WH_TRY(cpy(w[i + 12], L.b1, F));
      WH_TRY(cvt(w[i + 13], L.w2, D * F)); WH_TRY(cpy(w[i + 14], L.b2, D));
      i += 15;
    }
    WH_TRY(cpy(w[i++], P.lnpg, D));
    WH_TRY(cpy(w[i++], P.lnpb, D));
  }
  if (d->n_dec_layers > 0) {
    const float* tok_logical = w[i];
    WH_TRY(cvt(w[i++], P.tok, (size_t)d->n_vocab * D));
    WH_TRY(cvt(w[i++], P.pos, (size_t)d->n_text_ctx * D));
    for (int l = 0; l < d->n_dec_layers; ++l) {
      const DecL& L = P.dec[l];
      const size_t ck = P.ckvw + (size_t)l * 2 * D * D * e, cb = P.ckvb + (size_t)l * 2 * D * 4;
      WH_TRY(cpy(w[i + 0], L.ln1g, D)); WH_TRY(cpy(w[i + 1], L.ln1b, D));
      WH_TRY(cvt(w[i + 2], L.wqkv, D * D)); WH_TRY(cpy(w[i + 3], L.bqkv, D));
      WH_TRY(cvt(w[i + 4], L.wqkv + D * D * e, D * D));
      WH_TRY(launch_fill_f32(at<float>(packed, L.bqkv + D * 4), 0.f, D, s));
      WH_TRY(cvt(w[i + 5], L.wqkv + 2 * D * D * e, D * D)); WH_TRY(cpy(w[i + 6], L.bqkv + 2 * D * 4, D));
      WH_TRY(dw(w[i + 7], L.wo, D, D)); WH_TRY(cpy(w[i + 8], L.bo, D));
      WH_TRY(cpy(w[i + 9], L.ln2g, D)); WH_TRY(cpy(w[i + 10], L.ln2b, D));
      WH_TRY(cvt(w[i + 11], L.wqc, D * D)); WH_TRY(cpy(w[i + 12], L.bqc, D));
      WH_TRY(cvt(w[i + 13], ck, D * D));
      WH_TRY(launch_fill_f32(at<float>(packed, cb), 0.f, D, s));
      WH_TRY(cvt(w[i + 14], ck + D * D * e, D * D)); WH_TRY(cpy(w[i + 15], cb + D * 4, D));
      WH_TRY(dw(w[i + 16], L.woc, D, D)); WH_TRY(cpy(w[i + 17], L.boc, D));
      WH_TRY(cpy(w[i + 18], L.ln3g, D)); WH_TRY(cpy(w[i + 19], L.ln3b, D));
      WH_TRY(cvt(w[i + 20], L.w1, F * D)); WH_TRY(cpy(w[i + 21], L.b1, F));
      WH_TRY(dw(w[i + 22], L.w2, D, F)); WH_TRY(cpy(w[i + 23], L.b2, D));
      if (t == ACT_BF16) {  // fold ln1 into q/k/v, ln2 into the cross query, ln3 into the MLP up-projection
        const size_t DD = D * D * e;
        float* c1 = at<float>(packed, L.c1qkv);
        float* bq = at<float>(packed, L.bqkv);
        WH_TRY(launch_fold_ln(w[i + 2], w[i + 0], w[i + 1], w[i + 3], D, D, at<void>(packed, L.wqkv), c1, bq, s));
        WH_TRY(launch_fold_ln(w[i + 4], w[i + 0], w[i + 1], nullptr, D, D, at<void>(packed, L.wqkv + DD), c1 + D,
                              bq + D, s));
        WH_TRY(launch_fold_ln(w[i + 5], w[i + 0], w[i + 1], w[i + 6], D, D, at<void>(packed, L.wqkv + 2 * DD),
                              c1 + 2 * D, bq + 2 * D, s));
        WH_TRY(launch_fold_ln(w[i + 11], w[i + 9], w[i + 10], w[i + 12], D, D, at<void>(packed, L.wqc),
                              at<float>(packed, L.c1qc), at<float>(packed, L.bqc), s));
        WH_TRY(launch_fold_ln(w[i + 20], w[i + 18], w[i + 19], w[i + 21], F, D, at<void>(packed, L.w1),
                              at<float>(packed, L.c1w1), at<float>(packed, L.b1), s));
        WH_TRY(launch_pack_kt(w[i + 13], D, at<void>(packed, L.wkt), s));
        WH_TRY(launch_pack_dec_weight(w[i + 14], D, D, at<void>(packed, L.wvf), s));
      }
      i += 24;
    }
    if (t == ACT_BF16)  // final LayerNorm folded into a copy of the (tied) token embedding
      WH_TRY(launch_fold_ln(tok_logical, w[i], w[i + 1], nullptr, d->n_vocab, D, at<void>(packed, P.lmw),
                            at<float>(packed, P.lmc1), at<float>(packed, P.lmb2), s));
    WH_TRY(cpy(w[i++], P.lnfg, D));
    WH_TRY(cpy(w[i++], P.lnfb, D));
  }
  return WHISPER_OK;
}

size_t whisper_workspace_size(const whisper_dims* d, int batch, int which) {
  if (check_dims(d) != WHISPER_OK || batch <= 0) return 0;
  switch (which) {
    case WHISPER_WS_LOGMEL: return al256(logmel_ws(batch, d->n_mels));
    case WHISPER_WS_ENCODE: return enc_ws(d, batch).total;
    case WHISPER_WS_CROSS_KV: return 0;
    case WHISPER_WS_DECODE: return dec_ws(d, batch).total;
    case WHISPER_WS_ENCODE_FP8: return enc_ws(d, batch, true).total;
    case WHISPER_WS_DECODE_ENC: return dec_ws_enc(d, batch).total;
    case WHISPER_WS_DECODE_ENC_FP8: return dec_ws_enc(d, batch, true).total;
  }
  return 0;
}

// Peak device footprint of one pass of B chunks under the stage schedule the
// header documents.
static void batch_footprint(const whisper_dims* d, int B, int cap, int P, bool fp8, bool logits,
                            whisper_batch_plan* p) {
  const size_t e = esz(d->act), b = (size_t)B, L = d->n_dec_layers, H = d->n_heads, T = d->n_audio_ctx;
  const size_t D = d->d_model;
  *p = whisper_batch_plan{};
  p->weights = al256(whisper_packed_weights_size(d));
  p->workspace = std::max({al256(logmel_ws(B, d->n_mels)), enc_ws(d, B).total, dec_ws(d, B).total,
                           dec_ws(d, B * std::max(P, 1)).total, fp8 ? al256(whisper_fp8_workspace_size()) : 0});
  p->audio = al256(b * 480000 * 4);
  p->mel = al256(b * d->n_mels * N_FRAMES * 4);
  p->encoder_out = al256(b * T * D * e);
  p->cross_kv = al256(L * 2 * b * H * T * 64 * e);
  p->cross_codes = fp8 ? al256(L * 2 * b * H * T * 64) + al256(L * 2 * 4) : 0;
  p->kv_cache = al256(L * 2 * b * H * (size_t)cap * 64);
  p->decode_state = al256(L * 2 * 4) + 3 * al256(b * 4) + al256(b * std::max(P, 1) * 4) + al256(16);
  p->logits = logits ? al256(b * d->n_vocab * 4) : 0;
  p->stage[0] = p->audio + p->mel;
  p->stage[1] = p->mel + p->encoder_out;
  p->stage[2] = p->encoder_out + p->cross_kv;
  p->stage[3] = fp8 ? p->cross_kv + p->cross_codes : 0;
  p->stage[4] = (fp8 ? p->cross_codes : p->cross_kv) + p->kv_cache + p->decode_state + p->logits;
  for (int i = 0; i < 5; ++i)
    if (p->stage[i] > p->stage[p->peak_stage]) p->peak_stage = i;
  p->total = p->weights + p->workspace + p->stage[p->peak_stage];
}

whisper_status whisper_plan_batch(const whisper_dims* d, size_t budget, int cap, int P, int cross_fp8,
                                  int want_logits, int max_batch, whisper_batch_plan* plan) {
  WH_CHECK(check_dims(d));
  if (!plan) return fail(WHISPER_ERR_INVALID_ARG, "plan_batch: plan is NULL");
  if (max_batch < 1) return fail(WHISPER_ERR_INVALID_ARG, "plan_batch: max_batch must be >= 1");
  if (d->n_enc_layers <= 0 || d->n_dec_layers <= 0)
    return fail(WHISPER_ERR_SHAPE, "plan_batch: needs both encoder and decoder layers");
  if (cap <= 0 || cap > 4096) return fail(WHISPER_ERR_SHAPE, "plan_batch: kv_cap must be in 1..4096");
  if (P < 0 || P > cap) return fail(WHISPER_ERR_SHAPE, "plan_batch: prompt_tokens must be in 0..kv_cap");
  const bool fp8 = cross_fp8 != 0, lg = want_logits != 0;
  int hi = std::min(max_batch, 4096 / std::max(P, 1));
  batch_footprint(d, 1, cap, P, fp8, lg, plan);
  if (plan->total > budget) {
    plan->batch = 0;
    return fail(WHISPER_ERR_CAPACITY, "plan_batch: one chunk does not fit in the budget");
  }
  int lo = 1;  // footprint is non-decreasing in B: the largest fitting B by bisection
  while (lo < hi) {
    const int mid = lo + (hi - lo + 1) / 2;
    whisper_batch_plan t;
    batch_footprint(d, mid, cap, P, fp8, lg, &t);
    if (t.total <= budget) lo = mid;
    else hi = mid - 1;
  }
  batch_footprint(d, lo, cap, P, fp8, lg, plan);
  plan->batch = lo;
  return WHISPER_OK;
}

whisper_status whisper_logmel(const whisper_dims* d, const float* audio, int B, int n_samples, float* mel_out,
                              void* ws, size_t ws_bytes, void* stream) {
  WH_CHECK(check_dims(d));
  if (B <= 0) return fail(WHISPER_ERR_INVALID_ARG, "logmel: batch must be > 0");
  if (n_samples <= 0 || n_samples > 480000) return fail(WHISPER_ERR_SHAPE, "logmel: n_samples must be in 1..480000");
  WH_CHECK(check_ptrs({audio, mel_out}, "logmel"));
  WH_CHECK(check_ws(ws, ws_bytes, whisper_workspace_size(d, B, WHISPER_WS_LOGMEL), "logmel"));
  (void)hipGetLastError();
  WH_TRY(launch_logmel(audio, B, n_samples, d->n_mels, mel_out, ws, S(stream)));
  return WHISPER_OK;
}

int whisper_chunk_plan(int64_t n_samples, int stride, int32_t* plan, int max_chunks) {
  constexpr long W = 480000, HOP = 160, NFR = 3000;
  if (n_samples <= 0 || stride <= 0 || stride > W || stride % HOP) return 0;
  const long n = n_samples <= W ? 1 : 1 + (n_samples - W + stride - 1) / stride;
  // plan entries are int32: every chunk's first sample must fit
  if (n_samples > 0x7fffffffL || (n - 1) * (long)stride > 0x7fffffffL) return 0;
  if (!plan) return (int)n;
  if (max_chunks < n) return 0;
  const long sf = stride / HOP, of = NFR - sf;  // frames per stride, frames of overlap
  for (long i = 0; i < n; ++i) {
    const long start = i * stride, valid = std::min(W, n_samples - start);
    const long vf = std::min(NFR, (valid + HOP - 1) / HOP);  // frames centred on real audio
    plan[4 * i + 0] = (int32_t)start;
    plan[4 * i + 1] = (int32_t)valid;
    plan[4 * i + 2] = (int32_t)(i == 0 ? 0 : of / 2);
    plan[4 * i + 3] = (int32_t)(i == n - 1 ? vf : NFR - (of - of / 2));
  }
  return (int)n;
}

whisper_status whisper_logmel_chunked(const whisper_dims* d, const float* audio, int64_t n_samples, int stride,
                                      float* mel_out, void* ws, size_t ws_bytes, void* stream) {
  WH_CHECK(check_dims(d));
  const int n = whisper_chunk_plan(n_samples, stride, nullptr, 0);
  if (n <= 0) return fail(WHISPER_ERR_SHAPE, "logmel_chunked: need n_samples > 0 and stride in 160..480000, a multiple of 160");
  if (n_samples > (1L << 40)) return fail(WHISPER_ERR_SHAPE, "logmel_chunked: n_samples too large");
  WH_CHECK(check_ptrs({audio, mel_out}, "logmel_chunked"));
  WH_CHECK(check_ws(ws, ws_bytes, whisper_workspace_size(d, n, WHISPER_WS_LOGMEL), "logmel_chunked"));
  (void)hipGetLastError();
  WH_TRY(launch_logmel(audio, n, 480000, d->n_mels, mel_out, ws, S(stream), stride, n_samples));
  return WHISPER_OK;
}

whisper_status whisper_encode_layers(const whisper_dims* d, const void* packed, const void* h_in, int B, int l0,
                                     int l1, int apply_ln_post, void* h_out, void* ws, size_t ws_bytes,
                                     void* stream) {
  WH_CHECK(check_dims(d));
  if (B <= 0) return fail(WHISPER_ERR_INVALID_ARG, "encode_layers: batch must be > 0");
  if (d->n_enc_layers <= 0 || l0 < 0 || l1 < l0 || l1 > d->n_enc_layers)
    return fail(WHISPER_ERR_SHAPE, "encode_layers: layer range outside the encoder");
  WH_CHECK(check_ptrs({packed, h_in, h_out}, "encode_layers"));
  const EncWS W = enc_ws(d, B);
  WH_CHECK(check_ws(ws, ws_bytes, W.total, "encode_layers"));
  (void)hipGetLastError();
  return run_enc_layers(d, packed, layout(d), W, h_in, false, B, l0, l1, apply_ln_post != 0, h_out, ws, S(stream));
}

static whisper_status encode_impl(const whisper_dims* d, const void* packed, const void* packed8, const float* mel,
                                  int B, void* enc_out, void* ws, size_t ws_bytes, void* stream) {
  const char* who = packed8 ? "encode_fp8" : "encode";
  WH_CHECK(check_dims(d));
  if (B <= 0) return fail(WHISPER_ERR_INVALID_ARG, std::string(who) + ": batch must be > 0");
  if (d->n_enc_layers <= 0) return fail(WHISPER_ERR_SHAPE, std::string(who) + ": no encoder layers");
  WH_CHECK(check_ptrs({packed, mel, enc_out}, who));
  const EncWS W = enc_ws(d, B, packed8 != nullptr);
  WH_CHECK(check_ws(ws, ws_bytes, W.total, who));
  (void)hipGetLastError();
  const Packed P = layout(d);
  const ActType t = act_of(d->act);
  const hipStream_t s = S(stream);
  const int D = d->d_model, T = d->n_audio_ctx, nm = d->n_mels;
  const long R = N_FRAMES + 2;  // padded time rows of the conv inputs
  void* X0 = at<void>(ws, W.x0);
  void* G1 = at<void>(ws, W.g1);
  float* X = at<float>(ws, W.x);
  WH_TRY(launch_mel_to_conv_input(t, mel, B, nm, N_FRAMES, X0, s));
  WH_TRY(launch_zero_rows(t, G1, D, R, B, 0, (int)R - 1, s));
  const size_t e = esz(d->act);
  // conv1 (k3, s1, p1): output row t reads padded input rows t..t+2 = one contiguous 3*n_mels slice
  GemmParams c1 = gp(X0, nm, at<void>(packed, P.conv1w), 3 * nm, N_FRAMES, D, 3 * nm, at<float>(packed, P.conv1b),
                     (char*)G1 + D * e, D);
  c1.batch = B; c1.strideA = R * nm; c1.strideC = R * D;
  WH_TRY(launch_gemm(t, EPI_GELU, c1, s));
  // conv2 (k3, s2, p1): output row t reads padded rows 2t..2t+2, so the row stride is 2*d
  GemmParams c2 = gp(G1, 2 * D, at<void>(packed, P.conv2w), 3 * D, T, D, 3 * D, at<float>(packed, P.conv2b), X, D);
  c2.batch = B; c2.strideA = R * D; c2.strideC = (long)T * D; c2.pe = at<float>(packed, P.pe);
  WH_TRY(launch_gemm(t, EPI_GELU_PE, c2, s));
  return run_enc_layers(d, packed, P, W, X, true, B, 0, d->n_enc_layers, true, enc_out, ws, s, packed8);
}

whisper_status whisper_encode(const whisper_dims* d, const void* packed, const float* mel, int B, void* enc_out,
                              void* ws, size_t ws_bytes, void* stream) {
  return encode_impl(d, packed, nullptr, mel, B, enc_out, ws, ws_bytes, stream);
}

static whisper_status check_fp8_model(const whisper_dims* d, const void* packed8, const char* who) {
  if (d->act != WHISPER_BF16) return fail(WHISPER_ERR_DTYPE, std::string(who) + ": bf16 models only");
  if (d->d_model % 256 || d->d_ffn % 256 || d->d_model < 512)
    return fail(WHISPER_ERR_SHAPE, std::string(who) + ": d_model and d_ffn must be multiples of 256, d_model >= 512");
  return check_ptrs({packed8}, who);
}

whisper_status whisper_encode_fp8(const whisper_dims* d, const void* packed, const void* packed8, const float* mel,
                                  int B, void* enc_out, void* ws, size_t ws_bytes, void* stream) {
  WH_CHECK(check_dims(d));
  WH_CHECK(check_fp8_model(d, packed8, "encode_fp8"));
  return encode_impl(d, packed, packed8, mel, B, enc_out, ws, ws_bytes, stream);
}

whisper_status whisper_encode_layers_fp8(const whisper_dims* d, const void* packed, const void* packed8,
                                         const void* h_in, int B, int l0, int l1, int apply_ln_post, void* h_out,
                                         void* ws, size_t ws_bytes, void* stream) {
  WH_CHECK(check_dims(d));
  WH_CHECK(check_fp8_model(d, packed8, "encode_layers_fp8"));
  if (B <= 0) return fail(WHISPER_ERR_INVALID_ARG, "encode_layers_fp8: batch must be > 0");
  if (d->n_enc_layers <= 0 || l0 < 0 || l1 < l0 || l1 > d->n_enc_layers)
    return fail(WHISPER_ERR_SHAPE, "encode_layers_fp8: layer range outside the encoder");
  WH_CHECK(check_ptrs({packed, h_in, h_out}, "encode_layers_fp8"));
  const EncWS W = enc_ws(d, B, true);
  WH_CHECK(check_ws(ws, ws_bytes, W.total, "encode_layers_fp8"));
  (void)hipGetLastError();
  return run_enc_layers(d, packed, layout(d), W, h_in, false, B, l0, l1, apply_ln_post != 0, h_out, ws, S(stream),
                        packed8);
}

size_t whisper_packed_weights_fp8_size(const whisper_dims* d) {
  if (check_dims(d) != WHISPER_OK || (d->n_enc_layers <= 0 && d->n_dec_layers <= 0)) return 0;
  return layout8(d).total;
}

whisper_status whisper_pack_weights_fp8(const whisper_dims* d, const float* const* w, void* packed8, void* ws,
                                        size_t ws_bytes, void* stream) {
  WH_CHECK(check_dims(d));
  WH_CHECK(check_fp8_model(d, packed8, "pack_fp8"));
  if (d->n_enc_layers <= 0 && d->n_dec_layers <= 0) return fail(WHISPER_ERR_SHAPE, "pack_fp8: no layers");
  if (!w) return fail(WHISPER_ERR_INVALID_ARG, "pack_fp8: weight table is NULL");
  WH_CHECK(check_ws(ws, ws_bytes, whisper_fp8_workspace_size(), "pack_fp8"));
  const int n = weight_count(d);
  for (int i = 0; i < n; ++i)
    if (!w[i] || ((uintptr_t)w[i] & 15u)) return fail(WHISPER_ERR_ALIGN, "pack_fp8: weight " + std::to_string(i) + " NULL or not 16-byte aligned");
  (void)hipGetLastError();
  const Packed8 P8 = layout8(d);
  const hipStream_t s = S(stream);
  const size_t D = d->d_model, F = d->d_ffn;
  float* sc = at<float>(packed8, P8.scales);
  // per weight tensor: amax scale (fl32(amax) / 448), then E4M3 codes
  auto q = [&](const float* src, size_t n_el, uint8_t* dst, float* scale) -> hipError_t {
    const size_t blocks = (n_el + 255) / 256;
    hipError_t e = launch_amax(ACT_F32, FP8_E4M3, src, n_el, (float*)ws, (int)std::min<size_t>(blocks, 1024), scale, s);
    if (e != hipSuccess) return e;
    return launch_fp8_quantize(ACT_F32, FP8_E4M3, src, n_el, scale, dst, s);
  };
  for (int l = 0; l < d->n_enc_layers; ++l) {
    const int i = 4 + 15 * l;  // logical order: conv1.{w,b}, conv2.{w,b}, then 15 tensors per layer
    uint8_t* qkv = at<uint8_t>(packed8, P8.qkv[l]);
    WH_TRY(q(w[i + 2], D * D, qkv, sc + 8 * l + 0));          // attn.query.weight
    WH_TRY(q(w[i + 4], D * D, qkv + D * D, sc + 8 * l + 1));  // attn.key.weight
    WH_TRY(q(w[i + 5], D * D, qkv + 2 * D * D, sc + 8 * l + 2));  // attn.value.weight
    WH_TRY(q(w[i + 11], F * D, at<uint8_t>(packed8, P8.w1[l]), sc + 8 * l + 3));  // mlp.0.weight
    WH_TRY(q(w[i + 13], D * F, at<uint8_t>(packed8, P8.w2[l]), sc + 8 * l + 4));  // mlp.2.weight
  }
  // decoder MLP: per tensor amax scale, then codes in the decode GEMM's fragment order
  const int dec0 = (d->n_enc_layers > 0 ? 4 + 15 * d->n_enc_layers + 2 : 0) + 2;  // after the token and position tables
  float* dsc = at<float>(packed8, P8.dscales);
  for (int l = 0; l < d->n_dec_layers; ++l) {
    const int i = dec0 + 24 * l;
    const size_t blocks1 = (F * D + 255) / 256;
    WH_TRY(launch_amax(ACT_F32, FP8_E4M3, w[i + 20], F * D, (float*)ws, (int)std::min<size_t>(blocks1, 1024),
                       dsc + 2 * l, s));  // mlp.0.weight
    WH_TRY(launch_pack_dec_weight_fp8(w[i + 20], (int)F, (int)D, dsc + 2 * l, at<void>(packed8, P8.dw1[l]), s));
    WH_TRY(launch_amax(ACT_F32, FP8_E4M3, w[i + 22], D * F, (float*)ws, (int)std::min<size_t>(blocks1, 1024),
                       dsc + 2 * l + 1, s));  // mlp.2.weight
    WH_TRY(launch_pack_dec_weight_fp8(w[i + 22], (int)D, (int)F, dsc + 2 * l + 1, at<void>(packed8, P8.dw2[l]), s));
    WH_TRY(launch_copy_f32(w[i + 21], at<float>(packed8, P8.db1[l]), F, s));  // mlp.0.bias, unfolded
  }
  return WHISPER_OK;
}

whisper_status whisper_gemm_fp8(const uint8_t* a, int M, int K, const float* a_scales, int rows_per_scale,
                                const uint8_t* w, int N, const float* w_scale, const float* bias, int gelu, void* c,
                                long ldc, void* stream) {
  if (M <= 0 || N <= 0 || K <= 0) return fail(WHISPER_ERR_INVALID_ARG, "gemm_fp8: sizes must be > 0");
  if (K % 256 || K < 512 || N % 256 || ldc < N || ldc % 8 || rows_per_scale < 256)
    return fail(WHISPER_ERR_SHAPE, "gemm_fp8: K % 256 == 0, K >= 512, N % 256 == 0, ldc >= N and % 8 == 0, rows_per_scale >= 256");
  if ((long)M * K > (1L << 31) || (long)N * K > (1L << 31) || (long)M * ldc * 2 > (1L << 31))
    return fail(WHISPER_ERR_SHAPE, "gemm_fp8: operands and output must be under 2 GB");
  WH_CHECK(check_ptrs({a, w, c}, "gemm_fp8"));
  WH_CHECK(check_ptrs4({a_scales, w_scale}, "gemm_fp8"));
  if (bias && !aligned16(bias)) return fail(WHISPER_ERR_ALIGN, "gemm_fp8: bias not 16-byte aligned");
  (void)hipGetLastError();
  GemmParams g = gp(a, K, w, K, M, N, K, bias, c, ldc);
  g.a_scale = a_scales; g.a_rows_per_scale = rows_per_scale; g.b_scale = w_scale;
  WH_TRY(launch_gemm_fp8(gelu ? EPI_GELU : EPI_STORE, g, S(stream)));
  return WHISPER_OK;
}

whisper_status whisper_cross_kv(const whisper_dims* d, const void* packed, const void* enc_out, int B, void* cross_kv,
                                void* ws, size_t ws_bytes, void* stream) {
  (void)ws; (void)ws_bytes;
  WH_CHECK(check_dims(d));
  if (B <= 0) return fail(WHISPER_ERR_INVALID_ARG, "cross_kv: batch must be > 0");
  if (d->n_dec_layers <= 0) return fail(WHISPER_ERR_SHAPE, "cross_kv: no decoder layers");
  WH_CHECK(check_ptrs({packed, enc_out, cross_kv}, "cross_kv"));
  (void)hipGetLastError();
  const Packed P = layout(d);
  const int D = d->d_model, T = d->n_audio_ctx;
  GemmParams p = gp(enc_out, D, at<void>(packed, P.ckvw), D, B * T, d->n_dec_layers * 2 * D, D,
                    at<float>(packed, P.ckvb), cross_kv, 0);
  p.ckv_T = T; p.ckv_B = B; p.ckv_H = d->n_heads; p.ckv_d = D;
  WH_TRY(launch_gemm(act_of(d->act), EPI_CROSSKV, p, S(stream)));
  return WHISPER_OK;
}

}  // extern "C"

// Allocation-free decoder step: its workspace (activations, split-K partials
// and tile counters) lives in this file-scope device array, one copy per GPU,
// held until the process ends. Host code uses the per-device address from
// hipGetSymbolAddress, never the array's name.
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)8 << 20;
static_assert(NOALLOC_SCRATCH_BYTES == (size_t)WHISPER_NOALLOC_SCRATCH_BYTES, "header and library limits agree");
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

namespace {

whisper_status decode_step_checks(const whisper_dims* d, const void* packed, int B, int cap, const int32_t* tokens,
                                  int32_t* lengths, uint8_t* kv_cache, const float* kv_scales, const void* cross_kv,
                                  const float* logits, int32_t* argmax, int32_t* dev_error, const char* who) {
  WH_CHECK(check_dims(d));
  if (B <= 0) return fail(WHISPER_ERR_INVALID_ARG, std::string(who) + ": batch must be > 0");
  if (d->n_dec_layers <= 0) return fail(WHISPER_ERR_SHAPE, std::string(who) + ": no decoder layers");
  if (cap <= 0 || cap > 4096) return fail(WHISPER_ERR_SHAPE, std::string(who) + ": kv_cap must be in 1..4096");
  WH_CHECK(check_ptrs({packed, kv_cache, cross_kv}, who));
  WH_CHECK(check_ptrs4({tokens, lengths, kv_scales, argmax}, who));
  if (logits && !aligned16(logits)) return fail(WHISPER_ERR_ALIGN, std::string(who) + ": logits not 16-byte aligned");
  if (dev_error && ((uintptr_t)dev_error & 3u)) return fail(WHISPER_ERR_ALIGN, std::string(who) + ": dev_error not 4-byte aligned");
  return WHISPER_OK;
}

// The decoder step over workspace `ws` laid out as W (arguments checked).
whisper_status decode_step_run(const whisper_dims* d, const void* packed, const DecWS& W, int B, int cap,
                               const int32_t* tokens, int32_t* lengths, uint8_t* kv_cache, const float* kv_scales,
                               const void* cross_kv, float* logits, int32_t* argmax, int32_t* dev_error, void* ws,
                               hipStream_t s) {
  (void)hipGetLastError();
  const Packed P = layout(d);
  const ActType t = act_of(d->act);
  const int D = d->d_model, H = d->n_heads, T = d->n_audio_ctx, F = d->d_ffn, L = d->n_dec_layers;
  const size_t e = esz(d->act);
  float* X = at<float>(ws, W.x);
  void* A = at<void>(ws, W.a);
  void* Dl = at<void>(ws, W.dlt);
  void* Q = at<void>(ws, W.q);
  void* ATT = at<void>(ws, W.att);
  void* QC = at<void>(ws, W.qc);
  void* HF = at<void>(ws, W.hf);
  float* LG = logits ? logits : at<float>(ws, W.logits);
  if (t == ACT_BF16) return decode_step_fused(d, packed, P, W, B, cap, tokens, lengths, kv_cache, kv_scales, cross_kv,
                                              LG, argmax, dev_error, ws, s);
  WH_CHECK(kvtrace_check(L, B, D, "decode_step"));
  WH_TRY(launch_embed(t, at<void>(packed, P.tok), at<void>(packed, P.pos), tokens, lengths, B, D, d->n_vocab,
                      d->n_text_ctx, cap, X, dev_error, s));
  const size_t kv_layer = (size_t)2 * B * H * cap * 64;
  const size_t ckv_layer = (size_t)2 * B * H * T * 64 * e;
  for (int l = 0; l < L; ++l) {
    const DecL& Lw = P.dec[l];
    if (l == 0)
      WH_TRY(launch_layernorm(t, true, X, nullptr, at<float>(packed, Lw.ln1g), at<float>(packed, Lw.ln1b), 1e-5f, B, D, A, nullptr, s));
    else
      WH_TRY(launch_layernorm(t, false, Dl, X, at<float>(packed, Lw.ln1g), at<float>(packed, Lw.ln1b), 1e-5f, B, D, A, X, s));
    GemmParams pq = gp(A, D, at<void>(packed, Lw.wqkv), D, B, 3 * D, D, at<float>(packed, Lw.bqkv), Q, D);
    pq.kv_cache = kv_cache; pq.kv_scales = kv_scales; pq.lengths = lengths; pq.dev_error = dev_error;
    pq.kv_cap = cap; pq.kv_B = B; pq.kv_H = H; pq.kv_layer = l; pq.d_model = D; pq.kv_pre = g_kvtrace.buf;
    pq.kv_force = g_kvtrace.force;
    WH_TRY(launch_gemm_skinny(t, EPI_DEC_QKV, pq, s));
    const uint8_t* kc = kv_cache + l * kv_layer;
    {
      ProfScope ps(WHISPER_PROF_DECODE_SELF_ATTENTION, s);
      WH_TRY(launch_attn_decode_self(t, Q, D, kc, kc + kv_layer / 2, kv_scales + 2 * l, lengths, 1, B, H, cap, ATT, s));
    }
    WH_TRY(launch_gemm_skinny(t, EPI_STORE, gp(ATT, D, at<void>(packed, Lw.wo), D, B, D, D, at<float>(packed, Lw.bo), Dl, D), s));
    WH_TRY(launch_layernorm(t, false, Dl, X, at<float>(packed, Lw.ln2g), at<float>(packed, Lw.ln2b), 1e-5f, B, D, A, X, s));
    WH_TRY(launch_gemm_skinny(t, EPI_STORE, gp(A, D, at<void>(packed, Lw.wqc), D, B, D, D, at<float>(packed, Lw.bqc), QC, D), s));
    const char* ck = (const char*)cross_kv + l * ckv_layer;
    {
      ProfScope ps(WHISPER_PROF_DECODE_CROSS_ATTENTION, s);
      WH_TRY(launch_attn_decode_cross(t, QC, ck, ck + ckv_layer / 2, B, H, T, ATT, s));
    }
    WH_TRY(launch_gemm_skinny(t, EPI_STORE, gp(ATT, D, at<void>(packed, Lw.woc), D, B, D, D, at<float>(packed, Lw.boc), Dl, D), s));
    WH_TRY(launch_layernorm(t, false, Dl, X, at<float>(packed, Lw.ln3g), at<float>(packed, Lw.ln3b), 1e-5f, B, D, A, X, s));
    WH_TRY(launch_gemm_skinny(t, EPI_GELU, gp(A, D, at<void>(packed, Lw.w1), D, B, F, D, at<float>(packed, Lw.b1), HF, F), s));
    WH_TRY(launch_gemm_skinny(t, EPI_STORE, gp(HF, F, at<void>(packed, Lw.w2), F, B, D, F, at<float>(packed, Lw.b2), Dl, D), s));
  }
  WH_TRY(launch_layernorm(t, false, Dl, X, at<float>(packed, P.lnfg), at<float>(packed, P.lnfb), 1e-5f, B, D, A, nullptr, s));
  WH_TRY(launch_gemm_skinny(t, EPI_F32, gp(A, D, at<void>(packed, P.tok), D, B, d->n_vocab, D, nullptr, LG, d->n_vocab), s));
  WH_TRY(launch_argmax(LG, B, d->n_vocab, argmax, lengths, s));
  return WHISPER_OK;
}


constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {nullptr};

// The current device's copy of `scratch`, looked up once per device with that
// device current.
whisper_status scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(WHISPER_ERR_HIP, std::string("decode_step_noalloc: hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= MAX_DEVICES) return fail(WHISPER_ERR_HIP, "decode_step_noalloc: device index out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(WHISPER_ERR_HIP, std::string("decode_step_noalloc: hipGetSymbolAddress: ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return WHISPER_OK;
}

}  // namespace

extern "C" {

whisper_status whisper_decode_step(const whisper_dims* d, const void* packed, int B, int cap, const int32_t* tokens,
                                   int32_t* lengths, uint8_t* kv_cache, const float* kv_scales, const void* cross_kv,
                                   float* logits, int32_t* argmax, int32_t* dev_error, void* ws, size_t ws_bytes,
                                   void* stream) {
  WH_CHECK(decode_step_checks(d, packed, B, cap, tokens, lengths, kv_cache, kv_scales, cross_kv, logits, argmax,
                              dev_error, "decode_step"));
  const DecWS W = dec_ws(d, B);
  WH_CHECK(check_ws(ws, ws_bytes, W.total, "decode_step"));
  return decode_step_run(d, packed, W, B, cap, tokens, lengths, kv_cache, kv_scales, cross_kv, logits, argmax,
                         dev_error, ws, S(stream));
}

whisper_status whisper_decode_step_noalloc(const whisper_dims* d, const void* packed, int B, int cap,
                                           const int32_t* tokens, int32_t* lengths, uint8_t* kv_cache,
                                           const float* kv_scales, const void* cross_kv, float* logits,
                                           int32_t* argmax, int32_t* dev_error, void* stream) {
  WH_CHECK(decode_step_checks(d, packed, B, cap, tokens, lengths, kv_cache, kv_scales, cross_kv, logits, argmax,
                              dev_error, "decode_step_noalloc"));
  if (!logits) return fail(WHISPER_ERR_INVALID_ARG, "decode_step_noalloc: logits must be given (no workspace holds them)");
  const DecWS W = dec_ws(d, B, false);
  if (W.total > NOALLOC_SCRATCH_BYTES)
    return fail(WHISPER_ERR_WORKSPACE, "decode_step_noalloc: batch " + std::to_string(B) + " needs " +
                                           std::to_string(W.total) + " bytes of scratch, the library holds " +
                                           std::to_string(NOALLOC_SCRATCH_BYTES));
  void* ws = nullptr;
  WH_CHECK(scratch_for_current_device(&ws));
  return decode_step_run(d, packed, W, B, cap, tokens, lengths, kv_cache, kv_scales, cross_kv, logits, argmax,
                         dev_error, ws, S(stream));
}

}  // extern "C"

// Prefill of n_tokens per row (n_tokens = 1: one decode step) through the
// fused bf16 step, with the cross-attention over precomputed K/V (cross_kv)
// or over the encoder output (enc).
static whisper_status prefill_impl(const char* who, const whisper_dims* d, const void* packed, int B, int n_tokens,
                                   int cap, const int32_t* tokens, int32_t* lengths, uint8_t* kv_cache,
                                   const float* kv_scales, const void* cross_kv, const void* enc, float* logits,
                                   int32_t* argmax, int32_t* dev_error, void* ws, size_t ws_bytes, void* stream,
                                   const void* packed8 = nullptr) {
  const std::string w(who);
  WH_CHECK(check_dims(d));
  if (d->act != WHISPER_BF16) return fail(WHISPER_ERR_DTYPE, w + ": bf16 models only");
  if (B <= 0 || n_tokens <= 0) return fail(WHISPER_ERR_INVALID_ARG, w + ": batch and n_tokens must be > 0");
  if ((long)B * n_tokens > 4096) return fail(WHISPER_ERR_SHAPE, w + ": batch * n_tokens must be <= 4096");
  if (d->n_dec_layers <= 0) return fail(WHISPER_ERR_SHAPE, w + ": no decoder layers");
  if (cap <= 0 || cap > 4096) return fail(WHISPER_ERR_SHAPE, w + ": kv_cap must be in 1..4096");
  if (enc && d->d_model != 512 && d->d_model != 768 && d->d_model != 1024 && d->d_model != 1280)
    return fail(WHISPER_ERR_SHAPE, w + ": d_model must be 512, 768, 1024 or 1280");
  WH_CHECK(check_ptrs({packed, kv_cache, enc ? enc : cross_kv}, who));
  WH_CHECK(check_ptrs4({tokens, lengths, kv_scales, argmax}, who));
  if (logits && !aligned16(logits)) return fail(WHISPER_ERR_ALIGN, w + ": logits not 16-byte aligned");
  if (dev_error && ((uintptr_t)dev_error & 3u)) return fail(WHISPER_ERR_ALIGN, w + ": dev_error not 4-byte aligned");
  if (packed8) {
    WH_CHECK(check_fp8_model(d, packed8, who));
    if (!enc) return fail(WHISPER_ERR_INVALID_ARG, w + ": the fp8 MLP sites run with the encoder output");
    if (d->d_ffn % 80 || d->d_ffn % (32 * 8 * DEC_KSPLIT) || d->d_model % 80)
      return fail(WHISPER_ERR_SHAPE, w + ": d_model and d_ffn must be multiples of 80, d_ffn of 1024");
  }
  const int M = B * n_tokens;
  const DecEncWS XW = enc ? dec_ws_enc(d, M, packed8 != nullptr) : DecEncWS{dec_ws(d, M)};
  WH_CHECK(check_ws(ws, ws_bytes, enc ? XW.total : XW.base.total, who));
  (void)hipGetLastError();
  const Packed P = layout(d);
  float* LG = logits ? logits : at<float>(ws, XW.base.logits);
  return decode_step_fused(d, packed, P, XW.base, B, cap, tokens, lengths, kv_cache, kv_scales, cross_kv, LG, argmax,
                           dev_error, ws, S(stream), nullptr, nullptr, n_tokens, FP8_E4M3, enc, enc ? &XW : nullptr,
                           packed8);
}

extern "C" {

whisper_status whisper_decode_prefill(const whisper_dims* d, const void* packed, int B, int n_tokens, int cap,
                                      const int32_t* tokens, int32_t* lengths, uint8_t* kv_cache,
                                      const float* kv_scales, const void* cross_kv, float* logits, int32_t* argmax,
                                      int32_t* dev_error, void* ws, size_t ws_bytes, void* stream) {
  return prefill_impl("decode_prefill", d, packed, B, n_tokens, cap, tokens, lengths, kv_cache, kv_scales, cross_kv,
                      nullptr, logits, argmax, dev_error, ws, ws_bytes, stream);
}

whisper_status whisper_decode_step_enc(const whisper_dims* d, const void* packed, int B, int cap,
                                       const int32_t* tokens, int32_t* lengths, uint8_t* kv_cache,
                                       const float* kv_scales, const void* enc_out, float* logits, int32_t* argmax,
                                       int32_t* dev_error, void* ws, size_t ws_bytes, void* stream) {
  return prefill_impl("decode_step_enc", d, packed, B, 1, cap, tokens, lengths, kv_cache, kv_scales, nullptr, enc_out,
                      logits, argmax, dev_error, ws, ws_bytes, stream);
}

whisper_status whisper_decode_step_enc_fp8(const whisper_dims* d, const void* packed, const void* packed8, int B,
                                           int cap, const int32_t* tokens, int32_t* lengths, uint8_t* kv_cache,
                                           const float* kv_scales, const void* enc_out, float* logits,
                                           int32_t* argmax, int32_t* dev_error, void* ws, size_t ws_bytes,
                                           void* stream) {
  return prefill_impl("decode_step_enc_fp8", d, packed, B, 1, cap, tokens, lengths, kv_cache, kv_scales, nullptr,
                      enc_out, logits, argmax, dev_error, ws, ws_bytes, stream, packed8);
}

whisper_status whisper_decode_prefill_enc(const whisper_dims* d, const void* packed, int B, int n_tokens, int cap,
                                          const int32_t* tokens, int32_t* lengths, uint8_t* kv_cache,
                                          const float* kv_scales, const void* enc_out, float* logits, int32_t* argmax,
                                          int32_t* dev_error, void* ws, size_t ws_bytes, void* stream) {
  return prefill_impl("decode_prefill_enc", d, packed, B, n_tokens, cap, tokens, lengths, kv_cache, kv_scales,
                      nullptr, enc_out, logits, argmax, dev_error, ws, ws_bytes, stream);
}

whisper_status whisper_decode_prefill_enc_fp8(const whisper_dims* d, const void* packed, const void* packed8, int B,
                                              int n_tokens, int cap, const int32_t* tokens, int32_t* lengths,
                                              uint8_t* kv_cache, const float* kv_scales, const void* enc_out,
                                              float* logits, int32_t* argmax, int32_t* dev_error, void* ws,
                                              size_t ws_bytes, void* stream) {
  return prefill_impl("decode_prefill_enc_fp8", d, packed, B, n_tokens, cap, tokens, lengths, kv_cache, kv_scales,
                      nullptr, enc_out, logits, argmax, dev_error, ws, ws_bytes, stream, packed8);
}

whisper_status whisper_decode_step_xq(const whisper_dims* d, const void* packed, int B, int cap,
                                      const int32_t* tokens, int32_t* lengths, uint8_t* kv_cache,
                                      const float* kv_scales, const uint8_t* cross_codes, const float* cross_scales,
                                      whisper_fp8_format cross_format, float* logits, int32_t* argmax,
                                      int32_t* dev_error, void* ws, size_t ws_bytes, void* stream) {
  WH_CHECK(check_dims(d));
  if (cross_format != WHISPER_FP8_E4M3 && cross_format != WHISPER_FP8_E5M2)
    return fail(WHISPER_ERR_INVALID_ARG, "decode_step_xq: cross_format must be WHISPER_FP8_E4M3 or WHISPER_FP8_E5M2");
  if (d->act != WHISPER_BF16) return fail(WHISPER_ERR_DTYPE, "decode_step_xq: bf16 models only");
  if (B <= 0) return fail(WHISPER_ERR_INVALID_ARG, "decode_step_xq: batch must be > 0");
  if (d->n_dec_layers <= 0) return fail(WHISPER_ERR_SHAPE, "decode_step_xq: no decoder layers");
  if (cap <= 0 || cap > 4096) return fail(WHISPER_ERR_SHAPE, "decode_step_xq: kv_cap must be in 1..4096");
  if (d->n_audio_ctx > 4096) return fail(WHISPER_ERR_SHAPE, "decode_step_xq: n_audio_ctx must be <= 4096");
  WH_CHECK(check_ptrs({packed, kv_cache, cross_codes}, "decode_step_xq"));
  WH_CHECK(check_ptrs4({tokens, lengths, kv_scales, cross_scales, argmax}, "decode_step_xq"));
  if (logits && !aligned16(logits)) return fail(WHISPER_ERR_ALIGN, "decode_step_xq: logits not 16-byte aligned");
  if (dev_error && ((uintptr_t)dev_error & 3u)) return fail(WHISPER_ERR_ALIGN, "decode_step_xq: dev_error not 4-byte aligned");
  const DecWS W = dec_ws(d, B);
  WH_CHECK(check_ws(ws, ws_bytes, W.total, "decode_step_xq"));
  (void)hipGetLastError();
  const Packed P = layout(d);
  float* LG = logits ? logits : at<float>(ws, W.logits);
  return decode_step_fused(d, packed, P, W, B, cap, tokens, lengths, kv_cache, kv_scales, nullptr, LG, argmax,
                           dev_error, ws, S(stream), cross_codes, cross_scales, 1, (int)cross_format);
}

// ------------------------------------------------------------------ one decoder projection
namespace {
struct DecLinWS { size_t wf, c1, b2, xt, part, cnt, n_cnt, total; };
bool declin_ln(int mode) { return mode <= WHISPER_DEC_LN_QKV; }
bool declin_split(int mode) { return mode == WHISPER_DEC_RESID_SPLITK; }
DecLinWS declin_ws(int mode, int M, int N, int K) {
  DecLinWS W{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = al256(off + bytes); return o; };
  const size_t Mp = (size_t)((M + 15) & ~15), Np = (size_t)((N + 15) & ~15);
  W.wf = take(Np * K * 2);
  W.c1 = take((size_t)N * 4);
  W.b2 = take((size_t)N * 4);
  W.xt = take(Mp * (declin_ln(mode) ? K : N) * 4);
  if (declin_split(mode)) {
    const size_t tiles = (size_t)((N + DEC_SPLIT_COLS - 1) / DEC_SPLIT_COLS) * ((M + 15) / 16);
    W.part = take(tiles * DEC_KSPLIT * (DEC_SPLIT_COLS / 16) * 64 * 16);
    W.cnt = take(tiles * 4);
    W.n_cnt = tiles;
  }
  W.total = off;
  return W;
}
}  // namespace

size_t whisper_decode_linear_workspace_size(int mode, int M, int N, int K) {
  if (mode < WHISPER_DEC_LN_STORE || mode > WHISPER_DEC_RESID_SPLITK || M <= 0 || M > 4096 || N <= 0 || K <= 0 ||
      K % 32)
    return 0;
  return declin_ws(mode, M, N, K).total;
}

whisper_status whisper_decode_linear(int mode, int M, int N, int K, float* x, const void* a, const float* w,
                                     const float* bias, const float* gamma, const float* beta, void* y,
                                     uint8_t* kv_cache, const float* kv_scales, const int32_t* lengths, int kv_cap,
                                     int32_t* dev_error, void* ws, size_t ws_bytes, void* stream) {
  if (mode < WHISPER_DEC_LN_STORE || mode > WHISPER_DEC_RESID_SPLITK)
    return fail(WHISPER_ERR_INVALID_ARG, "decode_linear: unknown mode");
  if (M <= 0 || M > 4096 || N <= 0 || K <= 0) return fail(WHISPER_ERR_INVALID_ARG, "decode_linear: need 1 <= M <= 4096, N, K > 0");
  if (K % 32) return fail(WHISPER_ERR_SHAPE, "decode_linear: K must be a multiple of 32");
  const bool ln = declin_ln(mode), split = declin_split(mode);
  if (!ln && N % 32) return fail(WHISPER_ERR_SHAPE, "decode_linear: residual modes need N % 32 == 0");
  if (split && (N % DEC_SPLIT_COLS || K % (DEC_KSPLIT * 8 * 32)))
    return fail(WHISPER_ERR_SHAPE, "decode_linear: split-K needs N % 80 == 0 and K % 1024 == 0");
  if (mode == WHISPER_DEC_LN_QKV && (N != 3 * K || K % 64))
    return fail(WHISPER_ERR_SHAPE, "decode_linear: QKV needs N == 3 K and K % 64 == 0");
  WH_CHECK(check_ptrs({x, w}, "decode_linear"));
  if (ln) {
    WH_CHECK(check_ptrs({gamma, beta, y}, "decode_linear"));
  } else {
    WH_CHECK(check_ptrs({a}, "decode_linear"));
  }
  if (bias && !aligned16(bias)) return fail(WHISPER_ERR_ALIGN, "decode_linear: bias not 16-byte aligned");
  if (mode == WHISPER_DEC_LN_QKV) {
    if (kv_cap <= 0 || kv_cap > 4096) return fail(WHISPER_ERR_SHAPE, "decode_linear: kv_cap must be in 1..4096");
    WH_CHECK(check_ptrs({kv_cache}, "decode_linear"));
    WH_CHECK(check_ptrs4({kv_scales, lengths}, "decode_linear"));
    if (dev_error && ((uintptr_t)dev_error & 3u)) return fail(WHISPER_ERR_ALIGN, "decode_linear: dev_error not 4-byte aligned");
    WH_CHECK(kvtrace_check(1, M, K, "decode_linear"));
  }
  const DecLinWS W = declin_ws(mode, M, N, K);
  WH_CHECK(check_ws(ws, ws_bytes, W.total, "decode_linear"));
  (void)hipGetLastError();
  const hipStream_t s = S(stream);
  u16_t* Wf = at<u16_t>(ws, W.wf);
  float* C1 = at<float>(ws, W.c1);
  float* B2 = at<float>(ws, W.b2);
  float* XT = at<float>(ws, W.xt);
  if (ln) WH_TRY(launch_fold_ln(w, gamma, beta, bias, N, K, Wf, C1, B2, s));
  else WH_TRY(launch_pack_dec_weight(w, N, K, Wf, s));
  WH_TRY(launch_x_tiles(x, XT, M, ln ? K : N, 1, s));
  DecGemmParams g{};
  g.M = M; g.N = N; g.K = K; g.W = Wf;
  g.bias = ln ? B2 : bias;
  g.c1 = ln ? C1 : nullptr;
  g.A = (const u16_t*)a; g.lda = K; g.X = XT;
  g.out = (u16_t*)y; g.out_f32 = (float*)y;
  if (mode == WHISPER_DEC_LN_QKV) {
    g.kv_cache = kv_cache; g.kv_scales = kv_scales; g.lengths = lengths; g.dev_error = dev_error;
    g.kv_cap = kv_cap; g.kv_B = M; g.kv_H = K / 64; g.kv_layer = 0; g.d_model = K; g.kv_pre = g_kvtrace.buf;
    g.kv_force = g_kvtrace.force;
  }
  int mb, cb;
  dec_gemm_tiles(M, N, mb, cb);
  if (split) {
    g.ks = DEC_KSPLIT; g.part = at<float>(ws, W.part); g.cnt = at<int32_t>(ws, W.cnt);
    mb = 1; cb = DEC_SPLIT_COLS / 16;
    WH_TRY(launch_fill_f32((float*)g.cnt, 0.f, W.n_cnt, s));  // the tile counters start at zero
  }
  static const DecEpi epis[] = {DEPI_STORE, DEPI_GELU, DEPI_F32, DEPI_QKV, DEPI_RESID, DEPI_RESID};
  WH_TRY(launch_gemm_dec(ln ? PRO_X : PRO_A, epis[mode], g, mb, cb, s));
  if (!ln) WH_TRY(launch_x_tiles(XT, x, M, N, 0, s));
  return WHISPER_OK;
}

// Workspace of whisper_decode_mlp_fp8: the two weights' codes in fragment
// order and their scales, amax partials, x in 16-row tiles, the quantised
// LN(x) rows and their scales, the hidden rows (when the caller takes none),
// the hidden rows' 16-column block maxima, split-K partials and tile
// counters.
struct DecMlp8WS { size_t w1, w2, sc, part_amax, xt, aq, srow, hf, amx, part, cnt, n_cnt, total; };
DecMlp8WS decmlp8_ws(int M, int D, int F) {
  DecMlp8WS W{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = al256(off + bytes); return o; };
  const size_t Mp = (size_t)((M + 15) & ~15), F16 = (size_t)((F + 15) & ~15), D16 = (size_t)((D + 15) & ~15);
  W.w1 = take(F16 * D);
  W.w2 = take(D16 * F);
  W.sc = take(2 * 4);
  W.part_amax = take(1024 * 4);
  W.xt = take(Mp * D * 4);
  W.aq = take((size_t)M * D * 2);
  W.srow = take((size_t)M * 4);
  W.hf = take((size_t)M * F * 2);
  W.amx = take((size_t)M * (F / 16) * 4);
  const size_t tiles = (size_t)((D + DEC_SPLIT_COLS - 1) / DEC_SPLIT_COLS) * ((M + 15) / 16);
  W.part = take(tiles * DEC_KSPLIT * (DEC_SPLIT_COLS / 16) * 64 * 16);
  W.cnt = take(tiles * 4);
  W.n_cnt = tiles;
  W.total = off;
  return W;
}
bool decmlp8_shape_ok(int M, int D, int F) {
  return M > 0 && M <= 4096 && D > 0 && F > 0 && D % DEC_SPLIT_COLS == 0 && D <= 2048 && F % DEC_SPLIT_COLS == 0 &&
         F % (DEC_KSPLIT * 8 * 32) == 0;
}

whisper_status whisper_e4m3_round_host(const float* x, float* y, size_t n) {
  if (n && (!x || !y)) return fail(WHISPER_ERR_INVALID_ARG, "e4m3_round_host: NULL buffer");
  e4m3_round_host(x, y, n);
  return WHISPER_OK;
}

size_t whisper_decode_mlp_fp8_workspace_size(int M, int d, int f) {
  return decmlp8_shape_ok(M, d, f) ? decmlp8_ws(M, d, f).total : 0;
}

whisper_status whisper_decode_mlp_fp8(int M, int d, int f, float* x, const float* gamma, const float* beta,
                                      const float* w1, const float* b1, const float* w2, const float* b2,
                                      void* hidden, float* hidden_amax, void* ws, size_t ws_bytes, void* stream) {
  if (!decmlp8_shape_ok(M, d, f))
    return fail(WHISPER_ERR_SHAPE, "decode_mlp_fp8: need 1 <= M <= 4096, d % 80 == 0, d <= 2048, f % 80 == 0, "
                                   "f % 1024 == 0");
  WH_CHECK(check_ptrs({x, w1, w2}, "decode_mlp_fp8"));
  WH_CHECK(check_ptrs4({gamma, beta, b1, b2}, "decode_mlp_fp8"));
  if (hidden && !aligned16(hidden)) return fail(WHISPER_ERR_ALIGN, "decode_mlp_fp8: hidden not 16-byte aligned");
  if (hidden_amax && ((uintptr_t)hidden_amax & 3u))
    return fail(WHISPER_ERR_ALIGN, "decode_mlp_fp8: hidden_amax not 4-byte aligned");
  const DecMlp8WS W = decmlp8_ws(M, d, f);
  WH_CHECK(check_ws(ws, ws_bytes, W.total, "decode_mlp_fp8"));
  (void)hipGetLastError();
  const hipStream_t s = S(stream);
  const size_t D = d, F = f;
  float* sc = at<float>(ws, W.sc);
  float* pa = at<float>(ws, W.part_amax);
  const size_t blocks = (F * D + 255) / 256;
  const int np = (int)std::min<size_t>(blocks, 1024);
  WH_TRY(launch_amax(ACT_F32, FP8_E4M3, w1, F * D, pa, np, sc, s));
  WH_TRY(launch_pack_dec_weight_fp8(w1, f, d, sc, at<void>(ws, W.w1), s));
  WH_TRY(launch_amax(ACT_F32, FP8_E4M3, w2, D * F, pa, np, sc + 1, s));
  WH_TRY(launch_pack_dec_weight_fp8(w2, d, f, sc + 1, at<void>(ws, W.w2), s));
  float* XT = at<float>(ws, W.xt);
  WH_TRY(launch_x_tiles(x, XT, M, d, 1, s));
  float* AMX = at<float>(ws, W.amx);
  WH_TRY(launch_fill_f32(at<float>(ws, W.cnt), 0.f, W.n_cnt, s));  // the tile counters start at 0
  u16_t* AQ = at<u16_t>(ws, W.aq);
  float* SROW = at<float>(ws, W.srow);
  u16_t* HF = hidden ? (u16_t*)hidden : at<u16_t>(ws, W.hf);
  WH_TRY(launch_ln_quant_rows(XT, gamma, beta, M, d, AQ, SROW, s));
  DecGemmParams g1{};
  g1.M = M; g1.N = f; g1.K = d; g1.A = AQ; g1.lda = d; g1.X = XT; g1.out = HF;
  g1.W8 = at<uint8_t>(ws, W.w1); g1.w_scale8 = sc; g1.row_scale = SROW; g1.amax_out = AMX; g1.amax_nblk = f / 16;
  g1.bias = b1;
  WH_TRY(launch_gemm_dec_fp8(DEPI_GELU, g1, s));
  DecGemmParams g2{};
  g2.M = M; g2.N = d; g2.K = f; g2.A = HF; g2.lda = f; g2.X = XT;
  g2.W8 = at<uint8_t>(ws, W.w2); g2.w_scale8 = sc + 1; g2.aq_part = AMX; g2.amax_nblk = f / 16; g2.bias = b2;
  g2.ks = DEC_KSPLIT; g2.part = at<float>(ws, W.part); g2.cnt = at<int32_t>(ws, W.cnt);
  WH_TRY(launch_gemm_dec_fp8(DEPI_RESID, g2, s));
  WH_TRY(launch_x_tiles(XT, x, M, d, 0, s));
  if (hidden_amax) WH_TRY(launch_rows_max(AMX, M, f / 16, hidden_amax, s));
  return WHISPER_OK;
}

whisper_status whisper_peak_mfma(int n_wg, int iters, float* out, void* stream) {
  if (n_wg <= 0 || iters <= 0) return fail(WHISPER_ERR_INVALID_ARG, "peak_mfma: n_wg and iters must be > 0");
  WH_CHECK(check_ptrs4({out}, "peak_mfma"));
  (void)hipGetLastError();
  WH_TRY(launch_peak_mfma(n_wg, iters, out, S(stream)));
  return WHISPER_OK;
}

double whisper_peak_mfma_flop(int n_wg, int iters) { return n_wg > 0 && iters > 0 ? peak_mfma_flop(n_wg, iters) : 0.0; }

whisper_status whisper_peak_read(const void* buf, size_t bytes, int n_wg, float* out, void* stream) {
  if (n_wg <= 0 || bytes < 16 || bytes % 16) return fail(WHISPER_ERR_INVALID_ARG, "peak_read: n_wg > 0, bytes a positive multiple of 16");
  WH_CHECK(check_ptrs({buf}, "peak_read"));
  WH_CHECK(check_ptrs4({out}, "peak_read"));
  (void)hipGetLastError();
  WH_TRY(launch_peak_read(buf, bytes, n_wg, out, S(stream)));
  return WHISPER_OK;
}

size_t whisper_fp8_workspace_size(void) { return 1024 * sizeof(float); }

whisper_status whisper_fp8_quantize(const void* x, whisper_dtype dt, whisper_fp8_format fmt, size_t n,
                                    const float* scale_in, uint8_t* codes, float* scale_out, void* ws,
                                    size_t ws_bytes, void* stream) {
  if (dt != WHISPER_F32 && dt != WHISPER_BF16) return fail(WHISPER_ERR_DTYPE, "fp8_quantize: dtype must be F32 or BF16");
  if (fmt != WHISPER_FP8_E4M3 && fmt != WHISPER_FP8_E5M2)
    return fail(WHISPER_ERR_INVALID_ARG, "fp8_quantize: fmt must be WHISPER_FP8_E4M3 or WHISPER_FP8_E5M2");
  if (n == 0) return fail(WHISPER_ERR_INVALID_ARG, "fp8_quantize: n must be > 0");
  WH_CHECK(check_ptrs({x, codes}, "fp8_quantize"));
  if (!scale_in && !scale_out) return fail(WHISPER_ERR_INVALID_ARG, "fp8_quantize: need scale_in or scale_out");
  if (scale_in && ((uintptr_t)scale_in & 3u)) return fail(WHISPER_ERR_ALIGN, "fp8_quantize: scale_in not 4-byte aligned");
  if (scale_out && ((uintptr_t)scale_out & 3u)) return fail(WHISPER_ERR_ALIGN, "fp8_quantize: scale_out not 4-byte aligned");
  if (!scale_in) WH_CHECK(check_ws(ws, ws_bytes, whisper_fp8_workspace_size(), "fp8_quantize"));
  (void)hipGetLastError();
  const hipStream_t s = S(stream);
  const float* sc = scale_in;
  if (!scale_in) {
    size_t blocks = (n + 255) / 256;
    const int np = (int)(blocks > 1024 ? 1024 : blocks);
    WH_TRY(launch_amax(act_of(dt), (int)fmt, x, n, (float*)ws, np, scale_out, s));
    sc = scale_out;
  } else if (scale_out) {
    WH_TRY(launch_copy_f32(scale_in, scale_out, 1, s));
  }
  WH_TRY(launch_fp8_quantize(act_of(dt), (int)fmt, x, n, sc, codes, s));
  return WHISPER_OK;
}

whisper_status whisper_fp8_dequantize(const uint8_t* codes, whisper_fp8_format fmt, size_t n, const float* scale,
                                      void* y, whisper_dtype dt, void* stream) {
  if (dt != WHISPER_F32 && dt != WHISPER_BF16) return fail(WHISPER_ERR_DTYPE, "fp8_dequantize: dtype must be F32 or BF16");
  if (fmt != WHISPER_FP8_E4M3 && fmt != WHISPER_FP8_E5M2)
    return fail(WHISPER_ERR_INVALID_ARG, "fp8_dequantize: fmt must be WHISPER_FP8_E4M3 or WHISPER_FP8_E5M2");
  if (n == 0) return fail(WHISPER_ERR_INVALID_ARG, "fp8_dequantize: n must be > 0");
  WH_CHECK(check_ptrs({codes, y}, "fp8_dequantize"));
  WH_CHECK(check_ptrs4({scale}, "fp8_dequantize"));
  (void)hipGetLastError();
  WH_TRY(launch_fp8_dequantize(act_of(dt), (int)fmt, codes, n, scale, y, S(stream)));
  return WHISPER_OK;
}

whisper_status whisper_layernorm_fused(const whisper_dims* d, const void* h, const float* res, const float* gamma,
                                       const float* beta, float eps, int M, void* normed, float* total, void* stream) {
  if (!d) return fail(WHISPER_ERR_INVALID_ARG, "layernorm: dims is NULL");
  if (d->act != WHISPER_F32 && d->act != WHISPER_BF16) return fail(WHISPER_ERR_DTYPE, "layernorm: bad dtype");
  if (d->d_model <= 0 || d->d_model % 4 || d->d_model > 2048) return fail(WHISPER_ERR_SHAPE, "layernorm: d_model must be a multiple of 4 in 4..2048");
  if (M <= 0) return fail(WHISPER_ERR_INVALID_ARG, "layernorm: M must be > 0");
  if (!(eps > 0.f)) return fail(WHISPER_ERR_INVALID_ARG, "layernorm: eps must be > 0");
  WH_CHECK(check_ptrs({h, gamma, beta}, "layernorm"));
  if (!normed && !total) return fail(WHISPER_ERR_INVALID_ARG, "layernorm: normed and total are both NULL");
  for (const void* p : {(const void*)res, (const void*)normed, (const void*)total})
    if (p && !aligned16(p)) return fail(WHISPER_ERR_ALIGN, "layernorm: pointer not 16-byte aligned");
  (void)hipGetLastError();
  WH_TRY(launch_layernorm(act_of(d->act), false, h, res, gamma, beta, eps, M, d->d_model, normed, total, S(stream)));
  return WHISPER_OK;
}

whisper_status whisper_linear(whisper_dtype dt, const void* x, int lda, const void* w, const float* bias, int M, int N,
                              int K, int act, void* y, int path, void* stream) {
  if (dt != WHISPER_F32 && dt != WHISPER_BF16) return fail(WHISPER_ERR_DTYPE, "linear: bad dtype");
  if (M <= 0 || N <= 0 || K <= 0 || lda <= 0) return fail(WHISPER_ERR_INVALID_ARG, "linear: sizes must be > 0");
  if (act != 0 && act != 1) return fail(WHISPER_ERR_INVALID_ARG, "linear: act must be 0 or 1");
  if (path < 0 || path > 9) return fail(WHISPER_ERR_INVALID_ARG, "linear: path must be in 0..9");
  WH_CHECK(check_ptrs({x, w, y}, "linear"));
  if (bias && !aligned16(bias)) return fail(WHISPER_ERR_ALIGN, "linear: bias not 16-byte aligned");
  if (dt == WHISPER_BF16 && (K % 64 || lda % 8)) return fail(WHISPER_ERR_SHAPE, "linear: bf16 needs K % 64 == 0 and lda % 8 == 0");
  if (path == 2 && (dt != WHISPER_BF16 || M > 128 || K % 128)) return fail(WHISPER_ERR_SHAPE, "linear: skinny path needs bf16, M <= 128, K % 128 == 0");
  (void)hipGetLastError();
  GemmParams p = gp(x, lda, w, K, M, N, K, bias, y, N);
  p.variant = path == 9 ? 9 : path >= 3 ? path - 2 : 0;
  const Epi epi = act ? EPI_GELU : EPI_STORE;
  const bool skinny = path == 2 || (path == 0 && dt == WHISPER_BF16 && M <= 128 && K % 128 == 0);
  WH_TRY(skinny ? launch_gemm_skinny(act_of(dt), epi, p, S(stream)) : launch_gemm(act_of(dt), epi, p, S(stream)));
  return WHISPER_OK;
}

whisper_status whisper_attention_encoder(whisper_dtype dt, const void* qkv, int B, int T, int H, void* out,
                                         void* stream) {
  if (dt != WHISPER_F32 && dt != WHISPER_BF16) return fail(WHISPER_ERR_DTYPE, "attention_encoder: bad dtype");
  if (B <= 0 || T <= 0 || H <= 0) return fail(WHISPER_ERR_INVALID_ARG, "attention_encoder: sizes must be > 0");
  WH_CHECK(check_ptrs({qkv, out}, "attention_encoder"));
  (void)hipGetLastError();
  WH_TRY(launch_attn_encoder(act_of(dt), qkv, B, T, H, out, S(stream)));
  return WHISPER_OK;
}

whisper_status whisper_attention_decode_self(whisper_dtype dt, const void* q, int B, int H, int cap,
                                             const uint8_t* k_codes, const uint8_t* v_codes, const float* scales,
                                             const int32_t* n_keys, void* out, void* stream) {
  if (dt != WHISPER_F32 && dt != WHISPER_BF16) return fail(WHISPER_ERR_DTYPE, "attention_decode_self: bad dtype");
  if (B <= 0 || H <= 0) return fail(WHISPER_ERR_INVALID_ARG, "attention_decode_self: sizes must be > 0");
  if (cap <= 0 || cap > 4096) return fail(WHISPER_ERR_SHAPE, "attention_decode_self: cap must be in 1..4096");
  WH_CHECK(check_ptrs({q, k_codes, v_codes, out}, "attention_decode_self"));
  WH_CHECK(check_ptrs4({scales, n_keys}, "attention_decode_self"));
  (void)hipGetLastError();
  WH_TRY(launch_attn_decode_self(act_of(dt), q, (long)H * 64, k_codes, v_codes, scales, n_keys, 0, B, H, cap, out,
                                 S(stream)));
  return WHISPER_OK;
}

size_t whisper_attention_decode_cross_workspace_size(int B, int H, int T) {
  (void)B; (void)H; (void)T;
  return 0;  // single pass, no partials
}

whisper_status whisper_attention_decode_cross(whisper_dtype dt, const void* q, const void* k, const void* v, int B,
                                              int H, int T, void* out, void* ws, size_t ws_bytes, void* stream) {
  if (dt != WHISPER_F32 && dt != WHISPER_BF16) return fail(WHISPER_ERR_DTYPE, "attention_decode_cross: bad dtype");
  if (B <= 0 || H <= 0 || T <= 0) return fail(WHISPER_ERR_INVALID_ARG, "attention_decode_cross: sizes must be > 0");
  if (T > 4096) return fail(WHISPER_ERR_SHAPE, "attention_decode_cross: T must be <= 4096");
  WH_CHECK(check_ptrs({q, k, v, out}, "attention_decode_cross"));
  (void)ws; (void)ws_bytes;
  (void)hipGetLastError();
  WH_TRY(launch_attn_decode_cross(act_of(dt), q, k, v, B, H, T, out, S(stream)));
  return WHISPER_OK;
}

}  // extern "C"
