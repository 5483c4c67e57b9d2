// GEMMs of the batched decoder step (M = batch rows, or batch rows x prompt
// tokens in a prefill; up to 4096), with the
// residual + LayerNorm of the whisper_blaze showcase page's layernorm_fused.cu
// card folded into them.
//
// At batch 64 each of these GEMMs streams a weight matrix once (3.3-13 MB)
// against a small activation block, so its time is set by how many dependent
// memory round trips a workgroup makes, not by bandwidth. The kernel is built
// to make one:
//  * a workgroup of 8 waves owns 16*CB output columns and 16*MB rows; the 8
//    waves split K among themselves, and every wave issues all of its weight
//    and activation loads (straight into MFMA operand registers) before its
//    first MFMA;
//  * the 8 partial tiles are summed through LDS in wave order (deterministic),
//    and one wave runs the epilogue. No global partials, counters or fences.
//
// LayerNorm folding. For y = LN(x) W^T + b with LN(x)_k = (x_k - mu) r g_k + be_k:
//    y_n = r * (sum_k x_k W'_nk - mu * c1_n) + b2_n,
//    W'_nk = bf16(g_k W_nk),  c1_n = sum_k W'_nk,  b2_n = b_n + sum_k be_k W_nk.
// W', c1 and b2 are made once when the weights are packed (fold_ln_kernel).
// The GEMM then reads the fp32 residual stream x directly, splits each value
// into bf16 hi + lo parts (two MFMAs, ~2^-17 relative error), and computes the
// row mean mu and r = 1/sqrt(var + eps) itself: the workgroup holds whole rows
// of x, so the statistics come from registers (per-lane sums shifted by the
// lane's first value, turned into a mean and a sum of squared deviations and
// merged across lanes and waves with the pairwise update of Chan, Golub and
// LeVeque). Since c1
// is summed from the rounded W', the fold cancels the mean exactly up to fp32
// accumulation error.
#include "common.hpp"
#include "internal.hpp"

namespace wh {

constexpr int DG_WAVES = 8;

// Fragment order of a decoder weight W [N, K] (K % 32 == 0, rows padded to a
// multiple of 16): block (n / 16, k / 32) is 512 contiguous elements, in which
// lane l = 16 * ((k % 32) / 8) + n % 16 holds its 8 consecutive k values: the
// B operand of one 16x16x32 MFMA, in lane order.
__host__ __device__ inline long dec_frag_index(long n, long k, long K) {
  return (((n >> 4) * (K >> 5) + (k >> 5)) * 64 + ((k & 31) >> 3) * 16 + (n & 15)) * 8 + (k & 7);
}
constexpr int DG_DEPTH = 1;         // k-steps of operand loads in flight per wave ahead of the MFMAs

// NS: k-steps per wave, fixed at compile time (K / 256 for K = 1280 or 5120),
// so the main loop is a straight-line software pipeline: the loads of step
// s + DG_DEPTH are issued before step s is computed, which keeps a bounded
// ~DG_DEPTH steps of operand bytes in flight per wave (streaming measured on
// MI355X: ~4-8 KB in flight per wave sustains ~12 TB/s from the caches, while
// issuing a wave's whole share at once congests and runs at about half that).
// NS = 0 is the generic path (any K % 32 == 0): one step at a time.
// One step of a (value, column) max across lanes: the partner lane's pair
// through the DPP control CTRL; larger value wins, the lower column on ties.
template <int CTRL>
__device__ __forceinline__ void amax_step(float& v, int& idx) {
  const float ov = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
  const int oi = __builtin_amdgcn_mov_dpp(idx, CTRL, 0xF, 0xF, true);
  if (ov > v || (ov == v && oi < idx)) {
    v = ov;
    idx = oi;
  }
}

// The value of the E4M3 code of y, e4m3_decode(e4m3_encode(y)), computed
// without forming the code, for finite y: normal magnitudes (>= 2^-6) keep 3
// mantissa bits (round to nearest even on the fp32 bits) and saturate at
// 448; smaller ones round to a multiple of 2^-9 (the subnormal step) by
// adding and removing 1.5 * 2^14, whose fp32 spacing is 2^-9; the sign is
// kept. Branch-free, so a wave whose lanes straddle the two ranges runs one
// path. Host and device evaluate it identically (plain fp32 adds).
__host__ __device__ __forceinline__ float e4m3_round(float y) {
  const uint32_t u = __builtin_bit_cast(uint32_t, y);
  const uint32_t sgn = u & 0x80000000u, a = u & 0x7fffffffu;
  const uint32_t rn = (a + 0x7ffffu + ((a >> 20) & 1u)) & 0xfff00000u;
  const float vn = fminf(__builtin_bit_cast(float, rn), 448.0f);
  const float vs = (__builtin_bit_cast(float, a) + 24576.0f) - 24576.0f;
  const float v = a < 0x3c800000u ? vs : vn;
  return __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, v) | sgn);
}

// Eight E4M3 codes -> eight bf16 (exact: every E4M3 value is a bf16 value).
__device__ __forceinline__ uint4 fp8x8_to_bf16x8(const uint2 w) {
  float a[4], b[4];
  e4m3x4_decode(w.x, a);
  e4m3x4_decode(w.y, b);
  auto pk = [](float lo, float hi) { return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u); };
  return make_uint4(pk(a[0], a[1]), pk(a[2], a[3]), pk(b[0], b[1]), pk(b[2], b[3]));
}
// The E4M3 scale of an amax: fl32(amax) / 448, 1 for 0.
__device__ __forceinline__ float e4m3_scale_of(float a) { return a > 0.f ? a / 448.0f : 1.0f; }

template <int PRO, int EPI, int MB, int CB, int NS, bool F8 = false>
__global__ __launch_bounds__(DG_WAVES * 64) void gemm_dec_kernel(DecGemmParams p) {
  constexpr int MR = MB * 16;
  constexpr bool XIN = PRO == PRO_X;
  __shared__ f32x4 red[DG_WAVES][MB * CB][64];
  __shared__ float2 s_st[XIN ? DG_WAVES : 1][MR];
  __shared__ float s_mu[MR], s_rs[MR];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // XCD-aware order: blocks are dispatched round-robin over the 8 XCDs
  // (block L on XCD L % 8), so the row tiles of one column tile are given
  // consecutive slots on one XCD and share its L2 copy of the weight slice.
  // split-K (PRO_A only): the KS_ workgroups of an output tile take
  // consecutive K slices and sit next to its row tiles in the order below
  const int KS_ = p.ks > 1 ? p.ks : 1;
  const int RT = (p.M + MR - 1) / MR, CT = (p.N + 16 * CB - 1) / (16 * CB), RTK = RT * KS_;
  const int L = blockIdx.x, xcd = L & 7, jj = L >> 3;
  const int ct = (jj / RTK) * 8 + xcd, rk = jj - (jj / RTK) * RTK;
  const int rt = rk / KS_, ksl = rk - (rk / KS_) * KS_;  // row tile, K slice
  if (ct >= CT) return;  // padding blocks (CT rounded up to a multiple of 8)
  const int n0 = ct * 16 * CB, m0 = rt * MR;
  const int M = p.M, N = p.N, K = p.K;
  const int S = K / 32;    // k-steps of a whole row (the LayerNorm statistics use these)
  const int SK = S / KS_;  // k-steps of this workgroup's slice
  const int s0 = ksl * SK + wave * SK / DG_WAVES, s1 = ksl * SK + (wave + 1) * SK / DG_WAVES;  // this wave's k-steps
  const int nsteps = s1 - s0;
  const int kq = (lane >> 4) * 8;

  // W is stored in fragment order (dec_frag_index): the 16 x 32 block of a
  // column group and k-step is 1 KB, lane-ordered, so each wave load is one
  // contiguous 1 KB read of whole cache lines
  const int NF = (N + 15) >> 4;
  const u16* wfr[CB];
  const uint8_t* wfr8[CB];  // F8: the same element offsets, one byte each
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const long fo = (long)min((n0 >> 4) + cb, NF - 1) * S * 512 + lane * 8;
    if constexpr (F8) wfr8[cb] = p.W8 + fo;
    else wfr[cb] = p.W + fo;
  }
  // F8 with aq_part: each A row's amax is the largest of its amax_nblk
  // partials (the 16-column block maxima the producing GEMM stored), reduced
  // once per workgroup into s_aq; then the reciprocal scale of this lane's A
  // row (in-register quantisation) and the epilogue's row scales. Run by
  // every wave once the first weight loads are in flight (it ends in a
  // barrier), so its loads overlap theirs.
  __shared__ float s_aq[MR];
  float aq_inv[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) aq_inv[mb] = 1.f;
  float e_rs[4] = {1.f, 1.f, 1.f, 1.f};  // F8: row scale x weight scale
  auto aq_reduce = [&]() {
    if constexpr (F8) {
      if (p.aq_part) {
        constexpr int TPR = DG_WAVES * 64 / MR;  // threads per row, a power of two <= 64
        static_assert(TPR * MR == DG_WAVES * 64 && TPR <= 64 && (TPR & (TPR - 1)) == 0, "row split");
        const int row = tid / TPR, j0 = tid - row * TPR;
        // float4 loads (amax_nblk % 4 == 0), four in flight per thread
        const float4* pr = (const float4*)(p.aq_part + (long)min(m0 + row, M - 1) * p.amax_nblk);
        const int n4 = p.amax_nblk >> 2;
        float a = 0.f;
        for (int base = 0; base < n4; base += 4 * TPR) {
          float4 v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int j = base + j0 + i * TPR;
            v[i] = j < n4 ? pr[j] : make_float4(0.f, 0.f, 0.f, 0.f);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) a = fmaxf(a, fmaxf(fmaxf(v[i].x, v[i].y), fmaxf(v[i].z, v[i].w)));
        }
        for (int o = TPR / 2; o > 0; o >>= 1) a = fmaxf(a, __shfl_xor(a, o, 64));
        if (j0 == 0) s_aq[row] = a;
        __syncthreads();
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) aq_inv[mb] = 1.0f / e4m3_scale_of(s_aq[mb * 16 + (lane & 15)]);
      }
      if (wave < MB * CB) {
        const int emb_ = wave / CB;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int ml = emb_ * 16 + (lane >> 4) * 4 + r;
          e_rs[r] = (p.aq_part ? e4m3_scale_of(s_aq[ml]) : p.row_scale[min(m0 + ml, M - 1)]) * p.w_scale8[0];
        }
      }
    }
  };
  long arow[MB];
  // grouped A: this column tile's rows of A start at its group's offset
  const long agoff = p.a_group > 0 ? (long)(n0 / p.a_group) * p.a_group_stride : 0;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) arow[mb] = (long)min(m0 + mb * 16 + (lane & 15), M - 1) * p.lda + agoff;
  // x tiles (dec_x_index): this lane's 4 + 4 values of k-step s sit at
  // xoff + 512 s and 256 floats further
  long xoff[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const long r = min(m0 + mb * 16 + (lane & 15), M - 1);
    xoff[mb] = (r >> 4) * S * 512 + ((lane >> 4) * 16 + (r & 15)) * 4;
  }

  // ---- epilogue: the MB * CB output blocks (16 rows x 16 columns) go to waves
  // 0 .. MB*CB-1, one each. A block's operands are fetched by its wave before
  // the main loads, so the epilogue makes no memory round trip of its own
  // (its stores may alias these addresses: loads left in the store loop would
  // serialise).
  constexpr bool RES = EPI == DEPI_RESID, QKV = EPI == DEPI_QKV;
  const int RPB = p.rows_per_b > 1 ? p.rows_per_b : 1;  // rows per batch row (prefill)
  static_assert(MB * CB <= DG_WAVES, "one output block per wave");
  const bool ewave = wave < MB * CB;
  const int emb = ewave ? wave / CB : 0, ecb = ewave ? wave - (wave / CB) * CB : 0;
  const int en = n0 + ecb * 16 + (lane & 15);  // this lane's output column
  float e_bias = 0.f, e_c1 = 0.f, e_x[4] = {0.f, 0.f, 0.f, 0.f}, e_inv[2] = {0.f, 0.f};
  int e_pos[4] = {0, 0, 0, 0};
  if (ewave) {
    const int n = min(en, N - 1);
    e_bias = p.bias ? p.bias[n] : 0.f;
    e_c1 = XIN ? p.c1[n] : 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = min(m0 + emb * 16 + (lane >> 4) * 4 + r, M - 1);
      if constexpr (RES) e_x[r] = p.X[dec_x_index(m, n, N)];
      if constexpr (QKV) e_pos[r] = p.lengths[m / RPB] + m % RPB;
    }
    if constexpr (QKV) {
      e_inv[0] = 1.0f / p.kv_scales[p.kv_layer * 2];
      e_inv[1] = 1.0f / p.kv_scales[p.kv_layer * 2 + 1];
    }
  }

  f32x4 acc[MB][CB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[mb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float st_c[MB], st_s1[MB], st_s2[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) st_c[mb] = st_s1[mb] = st_s2[mb] = 0.f;

  // operand slots: step j of this wave lives in slot j % NSLOT
  constexpr int NSLOT = NS > 0 ? DG_DEPTH + 1 : 1;
  uint4 wv[F8 ? 1 : NSLOT][CB];
  uint2 w8[F8 ? NSLOT : 1][CB];  // F8: eight codes per lane and fragment
  float4 xa[XIN ? NSLOT : 1][MB], xb[XIN ? NSLOT : 1][MB];
  uint4 av[XIN ? 1 : NSLOT][MB];
#define DG_ISSUE(J, SL)                                                                        \
  {                                                                                            \
    const int k_ = (s0 + (J)) * 32;                                                            \
    _Pragma("unroll") for (int cb = 0; cb < CB; ++cb) {                                        \
      if constexpr (F8) w8[F8 ? SL : 0][cb] = *(const uint2*)(wfr8[cb] + k_ * 16);              \
      else wv[F8 ? 0 : SL][cb] = *(const uint4*)(wfr[cb] + k_ * 16);                            \
    }                                                                                          \
    _Pragma("unroll") for (int mb = 0; mb < MB; ++mb) {                                        \
      if constexpr (XIN) {                                                                     \
        const float* x_ = p.X + xoff[mb] + k_ * 16;                                             \
        xa[XIN ? SL : 0][mb] = *(const float4*)x_;                                             \
        xb[XIN ? SL : 0][mb] = *(const float4*)(x_ + 256);                                     \
      } else {                                                                                 \
        av[XIN ? 0 : SL][mb] = *(const uint4*)(p.A + arow[mb] + k_ + kq);                      \
      }                                                                                        \
    }                                                                                          \
  }
#define DG_COMPUTE(J, SL)                                                                      \
  {                                                                                            \
    _Pragma("unroll") for (int mb = 0; mb < MB; ++mb) {                                        \
      if constexpr (XIN) {                                                                     \
        const float4 a_ = xa[XIN ? SL : 0][mb], e_ = xb[XIN ? SL : 0][mb];                     \
        const float v_[8] = {a_.x, a_.y, a_.z, a_.w, e_.x, e_.y, e_.z, e_.w};                  \
        uint32_t hi_[4], lo_[4];                                                               \
        _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                        \
          hi_[i] = f2bf2(v_[2 * i], v_[2 * i + 1]);                                            \
          lo_[i] = f2bf2(v_[2 * i] - __uint_as_float(hi_[i] << 16),                            \
                         v_[2 * i + 1] - __uint_as_float(hi_[i] & 0xffff0000u));               \
        }                                                                                      \
        const bf16x8 ah_ = bitcast<bf16x8>(make_uint4(hi_[0], hi_[1], hi_[2], hi_[3]));        \
        const bf16x8 al_ = bitcast<bf16x8>(make_uint4(lo_[0], lo_[1], lo_[2], lo_[3]));        \
        _Pragma("unroll") for (int cb = 0; cb < CB; ++cb) {                                    \
          acc[mb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah_, bitcast<bf16x8>(wv[F8 ? 0 : SL][cb]), acc[mb][cb], 0, 0, 0); \
          acc[mb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al_, bitcast<bf16x8>(wv[F8 ? 0 : SL][cb]), acc[mb][cb], 0, 0, 0); \
        }                                                                                      \
        /* shifted sums: S1 += x - c, S2 += (x - c)^2, c = this lane's first value of the row */ \
        if ((J) == 0) st_c[mb] = a_.x;                                                         \
        _Pragma("unroll") for (int i = 0; i < 8; ++i) {                                        \
          const float d_ = v_[i] - st_c[mb];                                                   \
          st_s1[mb] += d_;                                                                     \
          st_s2[mb] = fmaf(d_, d_, st_s2[mb]);                                                 \
        }                                                                                      \
      } else {                                                                                 \
        uint4 a8_ = av[XIN ? 0 : SL][mb];                                                       \
        if constexpr (F8) {                                                                    \
          if (p.aq_part) { /* quantise the bf16 row in registers: the code values, as bf16 */  \
            const uint32_t q_[4] = {a8_.x, a8_.y, a8_.z, a8_.w};                                \
            uint32_t o_[4];                                                                    \
            _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                    \
              const float lo_ = e4m3_round(__uint_as_float(q_[i] << 16) * aq_inv[mb]);          \
              const float hi_ = e4m3_round(__uint_as_float(q_[i] & 0xffff0000u) * aq_inv[mb]);  \
              o_[i] = (__float_as_uint(lo_) >> 16) | (__float_as_uint(hi_) & 0xffff0000u);     \
            }                                                                                  \
            a8_ = make_uint4(o_[0], o_[1], o_[2], o_[3]);                                      \
          }                                                                                    \
        }                                                                                      \
        _Pragma("unroll") for (int cb = 0; cb < CB; ++cb) {                                    \
          uint4 wb_;                                                                           \
          if constexpr (F8) wb_ = fp8x8_to_bf16x8(w8[F8 ? SL : 0][cb]);                         \
          else wb_ = wv[F8 ? 0 : SL][cb];                                                      \
          acc[mb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8>(a8_), bitcast<bf16x8>(wb_), \
                                                                acc[mb][cb], 0, 0, 0);         \
        }                                                                                      \
      }                                                                                        \
    }                                                                                          \
  }
  if constexpr (NS > 0) {
    // straight-line pipeline: issue step t, compute step t - DG_DEPTH
#pragma unroll
    for (int t = 0; t < NS + DG_DEPTH; ++t) {
      if (t < NS) DG_ISSUE(t, t % NSLOT)
      __builtin_amdgcn_sched_barrier(0);
      if (t == DG_DEPTH) aq_reduce();
      if (t >= DG_DEPTH) DG_COMPUTE(t - DG_DEPTH, (t - DG_DEPTH) % NSLOT)
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    aq_reduce();
    for (int j = 0; j < nsteps; ++j) {
      DG_ISSUE(j, 0)
      DG_COMPUTE(j, 0)
    }
  }
#undef DG_ISSUE
#undef DG_COMPUTE

  // ---- row moments: per lane (mean, M2) from the shifted sums, merged over the
  // 4 lanes holding a row (equal counts), published per wave
  if constexpr (XIN) {
    const float n = 8.f * nsteps, inv_n = nsteps ? 1.f / n : 0.f;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      float mu = st_c[mb] + st_s1[mb] * inv_n;
      float m2 = fmaxf(st_s2[mb] - st_s1[mb] * st_s1[mb] * inv_n, 0.f);
      float cnt = n;
#pragma unroll
      for (int o = 16; o <= 32; o <<= 1) {
        const float mu2 = __shfl_xor(mu, o, 64), m22 = __shfl_xor(m2, o, 64);
        const float d = mu - mu2;
        mu = 0.5f * (mu + mu2);
        m2 = (m2 + m22) + d * d * (0.5f * cnt);
        cnt *= 2.f;
      }
      if (lane < 16) s_st[wave][mb * 16 + lane] = make_float2(mu, m2);
    }
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) red[wave][mb * CB + cb][lane] = acc[mb][cb];
  __syncthreads();
  if constexpr (XIN) {
    if (tid < MR) {
      float mu = 0.f, m2 = 0.f;
#pragma unroll
      for (int w = 0; w < DG_WAVES; ++w) mu += (32.f * ((w + 1) * S / DG_WAVES - w * S / DG_WAVES)) * s_st[w][tid].x;
      mu *= 1.0f / (32.f * S);
#pragma unroll
      for (int w = 0; w < DG_WAVES; ++w) {
        const float2 sw = s_st[w][tid];
        const float d = sw.x - mu;
        m2 += sw.y + (32.f * ((w + 1) * S / DG_WAVES - w * S / DG_WAVES)) * d * d;
      }
      s_mu[tid] = mu;
      s_rs[tid] = 1.0f / sqrtf(m2 * (1.0f / (32.f * S)) + 1e-5f);
    }
    __syncthreads();
  }
  // this wave's block, summed over the 8 partial tiles in wave order
  f32x4 v4 = f32x4{0.f, 0.f, 0.f, 0.f};
  if (ewave) {
    v4 = red[0][wave][lane];
#pragma unroll
    for (int w = 1; w < DG_WAVES; ++w) v4 += red[w][wave][lane];
  }
  if (KS_ > 1) {
    // split-K: the blocks go out with device-scope stores (coherent across
    // XCDs without an L2 write-back); once every wave's stores are
    // acknowledged, a device-scope counter picks the tile's last workgroup,
    // which sums the KS_ partials in slice order (device-scope loads) and runs
    // the epilogue, then resets the counter
    __shared__ int s_last;
    const int tile = ct * RT + rt;
    const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(p.part, (short)0, 0x7fffffff, 0x00020000);
    if (ewave)
      __builtin_amdgcn_raw_buffer_store_b128(v4, rp, (uint32_t)((((tile * KS_ + ksl) * (MB * CB) + wave) * 64 + lane) * 16),
                                             0, 16);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) s_last = atomicAdd(p.cnt + tile, 1) == KS_ - 1;
    __syncthreads();
    if (!s_last) return;
    if (ewave) {
      v4 = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int q = 0; q < KS_; ++q)
        v4 += __builtin_amdgcn_raw_buffer_load_b128(rp, (uint32_t)((((tile * KS_ + q) * (MB * CB) + wave) * 64 + lane) * 16), 0, 16);
    }
    if (tid == 0) p.cnt[tile] = 0;
  }
  if (!ewave) return;

  // ---- epilogue: lane holds rows emb*16 + (lane>>4)*4 + r of column en
  float vr[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int ml = emb * 16 + (lane >> 4) * 4 + r;
    vr[r] = XIN ? s_rs[ml] * (v4[r] - s_mu[ml] * e_c1) + e_bias : (F8 ? v4[r] * e_rs[r] : v4[r]) + e_bias;
  }
  if constexpr (F8 && EPI == DEPI_GELU) {
    if (p.amax_out) {
      // the next site's scale: each row's max |stored bf16 value| over the
      // block's 16 columns (DPP permutes as in the argmax), stored as that
      // row's partial for this 16-column block
      const int blk = (n0 >> 4) + ecb;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float a = en < N ? fabsf(__uint_as_float((uint32_t)f2bf(gelu_erf(vr[r])) << 16)) : 0.f;
        a = fmaxf(a, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, a), 0xB1, 0xF, 0xF, true)));
        a = fmaxf(a, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, a), 0x4E, 0xF, 0xF, true)));
        a = fmaxf(a, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, a), 0x141, 0xF, 0xF, true)));
        a = fmaxf(a, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, a), 0x140, 0xF, 0xF, true)));
        const int m = m0 + emb * 16 + (lane >> 4) * 4 + r;
        if ((lane & 15) == 0 && m < M && blk < p.amax_nblk) p.amax_out[(long)m * p.amax_nblk + blk] = a;
      }
    }
  }
  if constexpr (EPI == DEPI_F32) {
    if (p.amax_part) {
      // greedy argmax, first stage: each row's largest value over this block's
      // 16 columns (the 16 lanes of a row group), lowest column on ties, NaN
      // and columns past N never chosen
      const int NB = (N + 15) >> 4;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = vr[r];
        int idx = en;
        if (en >= N || !(v == v)) {
          v = -INFINITY;
          idx = 0x7fffffff;
        }
        // across the 16 lanes of the row group with DPP lane permutes (no trip
        // through the LDS crossbar): quad_perm(1,0,3,2), quad_perm(2,3,0,1),
        // then row_half_mirror (lane i <-> 7 - i of each 8) and row_mirror
        // (lane i <-> 15 - i): after the four steps every lane holds the max
        amax_step<0xB1>(v, idx);
        amax_step<0x4E>(v, idx);
        amax_step<0x141>(v, idx);
        amax_step<0x140>(v, idx);
        // blocks wholly past N (the last column tile's tail) have no entry
        const int m = m0 + emb * 16 + (lane >> 4) * 4 + r, blk = (n0 >> 4) + ecb;
        if ((lane & 15) == 0 && m < M && blk < NB) p.amax_part[(long)m * NB + blk] = make_int2(__float_as_int(v), idx);
      }
    }
  }
  if (en >= N) return;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int ml = emb * 16 + (lane >> 4) * 4 + r, m = m0 + ml;
    if (m >= M) continue;
    const int n = en;
    const float v = vr[r];
    if constexpr (EPI == DEPI_RESID) {
      p.X[dec_x_index(m, n, N)] = e_x[r] + v;
    } else if constexpr (EPI == DEPI_F32) {
      p.out_f32[(long)m * N + n] = v;
    } else if constexpr (EPI == DEPI_STORE) {
      p.out[(long)m * N + n] = f2bf(v);
    } else if constexpr (EPI == DEPI_GELU) {
      p.out[(long)m * N + n] = f2bf(gelu_erf(v));
    } else if constexpr (EPI == DEPI_QKV) {
      // q -> bf16; k, v -> e4m3 codes at cache slot lengths[m]
      const int d = p.d_model;
      if (n < d) {
        p.out[(long)m * d + n] = f2bf(v);
      } else {
        const int kv = (n - d) / d, c = (n - d) - kv * d, pos = e_pos[r];
        const long dbg = ((long)(p.kv_layer * 2 + kv) * M + m) * d + c;
        if (p.kv_pre) p.kv_pre[dbg] = v;
        if (pos >= 0 && pos < p.kv_cap) {
          const long idx =
              ((((long)(p.kv_layer * 2 + kv) * p.kv_B + m / RPB) * p.kv_H + (c >> 6)) * p.kv_cap + pos) * 64 + (c & 63);
          uint32_t code = e4m3_encode(v * (kv ? e_inv[1] : e_inv[0]));
          if (p.kv_force && p.kv_force[dbg] >= 0) code = (uint32_t)p.kv_force[dbg];
          p.kv_cache[idx] = (uint8_t)code;
        } else if (p.dev_error) {
          *p.dev_error = 6;  // capacity exceeded: the write is skipped
        }
      }
    }
  }
}

template <int PRO, int EPI, int MB, int CB, int NS, bool F8 = false>
static hipError_t dec_launch_ns(const DecGemmParams& p, hipStream_t s) {
  const int CT = (p.N + 16 * CB - 1) / (16 * CB), RT = (p.M + 16 * MB - 1) / (16 * MB);
  const dim3 grid(((CT + 7) / 8) * 8 * RT * (p.ks > 1 ? p.ks : 1));
  hipLaunchKernelGGL((gemm_dec_kernel<PRO, EPI, MB, CB, NS, F8>), grid, dim3(DG_WAVES * 64), 0, s, p);
  return hipGetLastError();
}

// The pipelined kernel for the two K of the model (d = 1280 -> 5 steps per
// wave, 4d = 5120 -> 20), the generic one otherwise.
template <int PRO, int EPI, int MB, int CB, bool F8 = false>
static hipError_t dec_launch_t(const DecGemmParams& p, hipStream_t s) {
  const int S = p.K / 32 / (p.ks > 1 ? p.ks : 1);  // k-steps of one workgroup's slice
  if (S == DG_WAVES * 5) return dec_launch_ns<PRO, EPI, MB, CB, 5, F8>(p, s);
  if constexpr (!F8)  // (the fp8 kernel's 20-step form spills; the model's fp8 sites run 5 steps per wave)
    if (S == DG_WAVES * 20) return dec_launch_ns<PRO, EPI, MB, CB, 20, F8>(p, s);
  return dec_launch_ns<PRO, EPI, MB, CB, 0, F8>(p, s);
}

hipError_t launch_gemm_dec_fp8(DecEpi epi, const DecGemmParams& p, hipStream_t s) {
  if (p.M <= 0 || p.M > 4096 || p.N <= 0 || p.K <= 0 || p.K % 32 || !p.W8 || !p.w_scale8 || !p.A)
    return hipErrorInvalidValue;
  if (!p.row_scale == !p.aq_part) return hipErrorInvalidValue;  // exactly one source of the row scale
  if (p.aq_part && (p.amax_nblk <= 0 || p.amax_nblk % 4 || ((uintptr_t)p.aq_part & 15))) return hipErrorInvalidValue;
  if (p.amax_out && (epi != DEPI_GELU || p.amax_nblk != p.N / 16)) return hipErrorInvalidValue;
  if (p.N % 80) return hipErrorInvalidValue;                     // 16 x 80 tiles
  if (epi == DEPI_GELU && p.ks <= 1) return dec_launch_t<PRO_A, DEPI_GELU, 1, 5, true>(p, s);
  if (epi == DEPI_RESID && p.ks > 1 && p.part && p.cnt && p.ks <= 16 && (p.K / 32) % (p.ks * DG_WAVES) == 0)
    return dec_launch_t<PRO_A, DEPI_RESID, 1, 5, true>(p, s);
  return hipErrorInvalidValue;
}

// Tile shapes with MB * CB <= 4, and one 16-row block of 80 columns (larger
// ones run out of registers).
template <int PRO, int EPI>
static hipError_t dec_launch(const DecGemmParams& p, int mb, int cb, hipStream_t s) {
  if (cb == 1 && mb == 1) return dec_launch_t<PRO, EPI, 1, 1>(p, s);
  if (cb == 1 && mb == 2) return dec_launch_t<PRO, EPI, 2, 1>(p, s);
  if (cb == 1 && mb == 4) return dec_launch_t<PRO, EPI, 4, 1>(p, s);
  if (cb == 2 && mb == 1) return dec_launch_t<PRO, EPI, 1, 2>(p, s);
  if (cb == 2 && mb == 2) return dec_launch_t<PRO, EPI, 2, 2>(p, s);
  if (cb == 4 && mb == 1) return dec_launch_t<PRO, EPI, 1, 4>(p, s);
  if (cb == 5 && mb == 1) return dec_launch_t<PRO, EPI, 1, 5>(p, s);
  return hipErrorInvalidValue;
}

// Rows (16 * mb) and columns (16 * cb) per workgroup. One 16-row block per
// workgroup keeps the activation slice a workgroup streams small (it is
// re-read by every column tile); 64 columns for N of 2K-4K (about one
// workgroup per CU at batch 64), 80 for N = 4d and for the vocabulary (fewer
// column tiles re-reading the activation slice: 61.7 -> 60.3 us against 64
// columns), 32 otherwise. Chosen by measurement at batch 64: the time follows
// the bytes the busiest compute unit streams (about 40 GB/s per unit), so the
// tile count is matched to the 256 units.
void dec_gemm_tiles(int M, int N, int& mb, int& cb) {
  (void)M;
  mb = 1;
  cb = (N >= 2048 && N <= 4096) ? 4 : N > 16384 ? 5 : 2;
  // the MLP up-projection (N = 4d): 80-column tiles give one workgroup per
  // compute unit at batch <= 64 (5120 / 80 * 4 = 256) instead of 2.5, so no
  // unit streams three tiles while others stream two
  if (N % 80 == 0 && N > 4096 && N <= 8192) cb = 5;
}

hipError_t launch_gemm_dec(DecPro pro, DecEpi epi, const DecGemmParams& p, int mb, int cb, hipStream_t s) {
  if (p.M <= 0 || p.M > 4096 || p.N <= 0 || p.K <= 0 || p.K % 32) return hipErrorInvalidValue;
  if (p.ks > 1 && (pro != PRO_A || !p.part || !p.cnt || p.ks > 16 || (p.K / 32) % (p.ks * DG_WAVES)))
    return hipErrorInvalidValue;  // split-K: bf16 activations, whole k-steps per wave, workspace given
  if (p.a_group > 0 && (pro != PRO_A || p.a_group % (16 * cb))) return hipErrorInvalidValue;
  if (pro == PRO_X) {
    switch (epi) {
      case DEPI_QKV: return dec_launch<PRO_X, DEPI_QKV>(p, mb, cb, s);
      case DEPI_STORE: return dec_launch<PRO_X, DEPI_STORE>(p, mb, cb, s);
      case DEPI_GELU: return dec_launch<PRO_X, DEPI_GELU>(p, mb, cb, s);
      case DEPI_F32: return dec_launch<PRO_X, DEPI_F32>(p, mb, cb, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (epi) {
    case DEPI_RESID: return dec_launch<PRO_A, DEPI_RESID>(p, mb, cb, s);
    case DEPI_STORE: return dec_launch<PRO_A, DEPI_STORE>(p, mb, cb, s);
    default: return hipErrorInvalidValue;
  }
}

// Weight packing for a LayerNorm-consumer GEMM (one workgroup per output row
// n): W'[n,k] = bf16(gamma_k W[n,k]), c1[n] = sum_k W'[n,k],
// b2[n] = bias[n] + sum_k beta_k W[n,k]; sums in fp64. W' goes out in
// fragment order; rows N .. 16*ceil(N/16) - 1 are zero padding.
__global__ __launch_bounds__(256) void fold_ln_kernel(const float* W, const float* gamma, const float* beta,
                                                      const float* bias, int N, int K, u16* Wf, float* c1,
                                                      float* b2) {
  const int n = blockIdx.x, tid = threadIdx.x;
  if (n >= N) {
    for (int k = tid; k < K; k += 256) Wf[dec_frag_index(n, k, K)] = 0;
    return;
  }
  const float* w = W + (long)n * K;
  double s1 = 0.0, s2 = 0.0;
  for (int k = tid; k < K; k += 256) {
    const u16 f = f2bf(gamma[k] * w[k]);
    Wf[dec_frag_index(n, k, K)] = f;
    s1 += (double)bf2f(f);
    s2 += (double)beta[k] * (double)w[k];
  }
  __shared__ double r1[256], r2[256];
  r1[tid] = s1;
  r2[tid] = s2;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) {
      r1[tid] += r1[tid + o];
      r2[tid] += r2[tid + o];
    }
    __syncthreads();
  }
  if (tid == 0) {
    c1[n] = (float)r1[0];
    b2[n] = (float)((bias ? (double)bias[n] : 0.0) + r2[0]);
  }
}

hipError_t launch_fold_ln(const float* W, const float* gamma, const float* beta, const float* bias, int N, int K,
                          void* Wf, float* c1, float* b2, hipStream_t s) {
  if (N <= 0) return hipSuccess;
  if (K <= 0 || K % 32) return hipErrorInvalidValue;
  hipLaunchKernelGGL(fold_ln_kernel, dim3((N + 15) & ~15), dim3(256), 0, s, W, gamma, beta, bias, N, K, (u16*)Wf,
                     c1, b2);
  return hipGetLastError();
}

// fp32 row-major [N, K] -> bf16 in fragment order, rows padded to a multiple
// of 16 with zeros (weights read straight from the residual-free activations:
// attention outputs and the MLP hidden layer)
__global__ __launch_bounds__(256) void pack_frag_kernel(const float* W, int N, int K, u16* Wf) {
  const int n = blockIdx.x, tid = threadIdx.x;
  for (int k = tid; k < K; k += 256) Wf[dec_frag_index(n, k, K)] = n < N ? f2bf(W[(long)n * K + k]) : (u16)0;
}

hipError_t launch_pack_dec_weight(const float* W, int N, int K, void* Wf, hipStream_t s) {
  if (N <= 0) return hipSuccess;
  if (K <= 0 || K % 32) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pack_frag_kernel, dim3((N + 15) & ~15), dim3(256), 0, s, W, N, K, (u16*)Wf);
  return hipGetLastError();
}

// E4M3 codes of a decoder weight W [N, K] with the per-tensor scale
// scale[0] (code = e4m3(fl32(w * fl32(1 / s)))), in the fragment order of
// dec_frag_index, one byte per element; rows N .. 16*ceil(N/16) - 1 are zero.
__global__ __launch_bounds__(256) void pack_frag8_kernel(const float* W, int N, int K, const float* scale,
                                                         uint8_t* Wf) {
  const int n = blockIdx.x, tid = threadIdx.x;
  const float inv = 1.0f / scale[0];
  for (int k = tid; k < K; k += 256)
    Wf[dec_frag_index(n, k, K)] = n < N ? (uint8_t)e4m3_encode(W[(long)n * K + k] * inv) : (uint8_t)0;
}

hipError_t launch_pack_dec_weight_fp8(const float* W, int N, int K, const float* scale, void* Wf, hipStream_t s) {
  if (N <= 0) return hipSuccess;
  if (K <= 0 || K % 32) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pack_frag8_kernel, dim3((N + 15) & ~15), dim3(256), 0, s, W, N, K, scale, (uint8_t*)Wf);
  return hipGetLastError();
}

// The decoder MLP's fp8 input site: per row m of the fp32 residual stream X
// (16-row tiles, dec_x_index), a = bf16(LayerNorm(x)) (fp32 two-pass
// statistics, biased variance, eps 1e-5; rounded to bf16 as every activation
// of the step is, so the code decisions are taken on bf16 values), its scale
// s = fl32(amax |a|) / 448 (1 for an all-zero row), and the values of the
// codes e4m3(fl32(a * fl32(1 / s))), stored as bf16 (every E4M3 value is a
// bf16 value) in A [M, K]; s to srow[m]. One workgroup of 256 threads per
// row, K <= 2048.
__global__ __launch_bounds__(256) void ln_quant_rows_kernel(const float* __restrict__ X, const float* __restrict__ g,
                                                            const float* __restrict__ b, int K, u16* __restrict__ A,
                                                            float* __restrict__ srow) {
  constexpr int PER = 8;
  const int m = blockIdx.x, tid = threadIdx.x;
  __shared__ float red[8];
  float v[PER];
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int k = tid + i * 256;
    v[i] = k < K ? X[dec_x_index(m, k, K)] : 0.f;
    sum += v[i];
  }
  auto block_sum = [&](float x) {
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    __syncthreads();
    if ((tid & 63) == 0) red[tid >> 6] = x;
    __syncthreads();
    return (red[0] + red[1]) + (red[2] + red[3]);
  };
  const float mu = block_sum(sum) / (float)K;
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int k = tid + i * 256;
    const float dlt = k < K ? v[i] - mu : 0.f;
    sq = fmaf(dlt, dlt, sq);
  }
  const float r = 1.0f / sqrtf(block_sum(sq) / (float)K + 1e-5f);
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int k = tid + i * 256;
    v[i] = k < K ? bf2f(f2bf((v[i] - mu) * r * g[k] + b[k])) : 0.f;
    amax = fmaxf(amax, fabsf(v[i]));
  }
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  __syncthreads();
  if ((tid & 63) == 0) red[4 + (tid >> 6)] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[4], red[5]), fmaxf(red[6], red[7]));
  const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
  const float inv = 1.0f / sc;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int k = tid + i * 256;
    if (k < K) A[(long)m * K + k] = (u16)(__float_as_uint(e4m3_decode(e4m3_encode(v[i] * inv))) >> 16);
  }
  if (tid == 0) srow[m] = sc;
}

// The in-register rounding of the fp8 decode GEMM, evaluated on the host.
void e4m3_round_host(const float* x, float* y, size_t n) {
  for (size_t i = 0; i < n; ++i) y[i] = e4m3_round(x[i]);
}

// out[m] = max over j of part[m][j], j < nblk (one wave per row).
__global__ __launch_bounds__(64) void rows_max_kernel(const float* part, int nblk, float* out) {
  const int m = blockIdx.x, lane = threadIdx.x;
  float a = 0.f;
  for (int j = lane; j < nblk; j += 64) a = fmaxf(a, part[(long)m * nblk + j]);
  for (int o = 32; o > 0; o >>= 1) a = fmaxf(a, __shfl_xor(a, o, 64));
  if (lane == 0) out[m] = a;
}

hipError_t launch_rows_max(const float* part, int M, int nblk, float* out, hipStream_t s) {
  if (M <= 0 || nblk <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rows_max_kernel, dim3(M), dim3(64), 0, s, part, nblk, out);
  return hipGetLastError();
}

hipError_t launch_ln_quant_rows(const float* X, const float* g, const float* b, int M, int K, void* A, float* srow,
                                hipStream_t s) {
  if (M <= 0 || K <= 0 || K > 2048 || K % 32) return hipErrorInvalidValue;
  hipLaunchKernelGGL(ln_quant_rows_kernel, dim3(M), dim3(256), 0, s, X, g, b, K, (u16*)A, srow);
  return hipGetLastError();
}

}  // namespace wh
