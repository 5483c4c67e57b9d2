// Decoder cross-attention read straight from the encoder output.
//
// The cross-attention of the whisper_blaze showcase page's flash_attn_hopper.cu
// card attends over keys and values that are linear in the encoder output E:
// K = E W_k^T and V = E W_v^T + b_v. For one head h with query q_h,
//    score_t = q_h . (W_k,h E_t) / 8 = (W_k,h^T q_h) . E_t / 8 = q'_h . E_t / 8,
//    sum_t p_t V_t,h = W_v,h (sum_t p_t E_t) + b_v,h = W_v,h u_h + b_v,h,
// because the softmax weights p_t sum to one. Decoding at batch 64 is bound
// by HBM, and E (1500 x d per row) is half the bytes of K and V together, so
// each layer reads E once instead of K and V: the keys and values are never
// formed, and the once-per-batch projection of K and V disappears too.
//
// Per layer:
//   absorb_q_kernel       q'[m][h][:] = W_k,h^T q_h       (W_k packed per head, transposed)
//   attn_cross_enc_kernel  per workgroup, an even share of all rows' frames: scores
//                          S = E q'^T, online softmax per head, U = P^T E;
//                          unnormalised U and (max, sum) per head for each row
//                          segment of the share
//   absorb_combine_kernel u[m][h][:] = sum_c w_c U_c / sum_c w_c l_c
//   value projection      the decoder GEMM with one A row per head group
//                          (decode_gemm.hip), + b_v
#include "common.hpp"
#include "internal.hpp"

namespace wh {

// ------------------------------------------------------------------ packing
// W_kT[h][n][j] = bf16(W_k[h * 64 + j][n]): each head's 64 key rows, transposed,
// so the contraction index j of q' = W_k,h^T q_h is contiguous.
__global__ __launch_bounds__(256) void pack_kt_kernel(const float* __restrict__ wk, int d, u16* __restrict__ wkt) {
  const int h = blockIdx.y, n = blockIdx.x * 4 + (threadIdx.x >> 6), j = threadIdx.x & 63;
  if (n >= d) return;
  wkt[((long)h * d + n) * 64 + j] = f2bf(wk[(long)(h * 64 + j) * d + n]);
}

hipError_t launch_pack_kt(const float* wk, int d, void* wkt, hipStream_t s) {
  if (d <= 0 || d % 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pack_kt_kernel, dim3((d + 3) / 4, d / 64), dim3(256), 0, s, wk, d, (u16*)wkt);
  return hipGetLastError();
}

// ------------------------------------------------------------------ q' = W_k,h^T q_h
// q'^T[n][m] = sum_j W_kT[h][n][j] q[m][h*64 + j] with MFMA 16x16x32: A = W_kT
// rows (16 n x 32 j), B = q^T (32 j x 16 rows m); the result lane holds 4
// consecutive n of one row m (one 8-byte store). Workgroup: one wave, one
// head, 64 columns n, 64 rows m, so at batch 64 the 400 workgroups spread the
// 3.3 MB of W_k^T and of q' over every compute unit.
__global__ __launch_bounds__(64) void absorb_q_kernel(const u16* __restrict__ q, const u16* __restrict__ wkt,
                                                      int M, int H, int d, u16* __restrict__ qp) {
  const int h = blockIdx.x, lane = threadIdx.x & 63;
  const int n0 = blockIdx.y * 64, m0 = blockIdx.z * 64;
  if (n0 >= d) return;
  const int r16 = lane & 15, kq = (lane >> 4) * 8;
  uint4 a[4][2], bq[4][2];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      a[nb][ks] = *(const uint4*)(wkt + ((long)h * d + n0 + nb * 16 + r16) * 64 + ks * 32 + kq);
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const long mm = min(m0 + mb * 16 + r16, M - 1);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) bq[mb][ks] = *(const uint4*)(q + mm * H * 64 + h * 64 + ks * 32 + kq);
  }
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8>(a[nb][ks]), bitcast<bf16x8>(bq[mb][ks]), acc,
                                                      0, 0, 0);
      const int m = m0 + mb * 16 + r16;
      if (m < M) {
        uint2 o;
        o.x = f2bf2(acc[0], acc[1]);
        o.y = f2bf2(acc[2], acc[3]);
        *(uint2*)(qp + ((long)m * H + h) * d + n0 + nb * 16 + (lane >> 4) * 4) = o;
      }
    }
}

hipError_t launch_absorb_q(const void* q, const void* wkt, int M, int H, int d, void* qp, hipStream_t s) {
  if (M <= 0 || H <= 0 || d % 256 || H * 64 != d) return hipErrorInvalidValue;
  hipLaunchKernelGGL(absorb_q_kernel, dim3(H, d / 64, (M + 63) / 64), dim3(64), 0, s, (const u16*)q,
                     (const u16*)wkt, M, H, d, (u16*)qp);
  return hipGetLastError();
}

// ------------------------------------------------------------------ attention over E
// The frames of all query rows form one sequence of sub-tiles of 16 frames,
// G = M * nsub long (row-major: row m's sub-tiles are m * nsub .. m * nsub +
// nsub - 1). Workgroup w takes the contiguous share [w G / n_wg, (w + 1) G /
// n_wg), so every compute unit gets the same number of sub-tiles whatever
// the batch; a share may begin or end inside a row, and each row segment it
// covers leaves one partial (unnormalised U, running max, sum) in slot
// w * kmax + (row - first row of the share).
//
// In a workgroup, NW waves each own CB blocks of 32 columns of E (d = NW CB
// 32). Per sub-tile:
//  * S [16 frames x 32 heads] partial over the wave's columns with MFMA
//    16x16x32 (E and q' from registers; heads past H are zero rows of q'),
//    summed over the waves through LDS;
//  * online softmax per head (the U layout: lane l holds head l % 32 for 8 of
//    the frames, the other 8 in lane l ^ 32);
//  * U^T [32 columns x 32 heads] += E^T P^T with MFMA 32x32x16, the E^T
//    fragments read from LDS with the gfx950 transpose read.
// Software pipeline per row segment, one barrier per sub-tile. The global
// loads put E straight into the A operand of the score MFMAs (lane l: frame
// l % 16, eight columns), XR sub-tiles ahead. In step i a wave computes the
// partial scores of sub-tile i + 1 from those registers, stores the same
// registers into its LDS slice (two stages) for the transposed reads of U, and
// issues the loads of sub-tile i + 1 + XR into them; after the barrier it
// takes the summed scores of sub-tile i through softmax into U while a few
// threads sum the partials of sub-tile i + 1. A share that crosses a row
// boundary runs one pipeline per row (q' is loaded once per row segment).
constexpr int XE_F = 16;      // frames per sub-tile
constexpr int XE_MAXH = 20;   // heads (real ones are stored, padded ones are zero)
constexpr int XE_HS = 20;     // floats per head in a score tile (16 frames + 4 pad: conflict-free rows)
constexpr int XE_XR = 2;      // register stages of global loads in flight
constexpr int XE_MIN_PER_WG = 4;

__device__ __forceinline__ int xe_off(int kb, int f, int col) {  // u16 offset in a wave's slice of one stage
  return kb * (XE_F * 16) + ((f ^ (kb & 3)) << 4) + col;
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 xe_read_tr16(const u16* p) {
  return bitcast<uint2>(__builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p));
}

template <int NW, int CB>
__global__ __launch_bounds__(NW * 64) void attn_cross_enc_kernel(const u16* __restrict__ qp, const u16* __restrict__ E,
                                                                 int H, int T, int nsub, long G, int n_wg, int kmax,
                                                                 int rows_per_b, int reverse, u16* __restrict__ upart,
                                                                 float* __restrict__ ml) {
  constexpr int WC = CB * 32;         // columns per wave
  constexpr int d = NW * WC;
  constexpr int SLICE = 2 * CB * XE_F * 16;  // u16 per wave per stage
  constexpr int SN = XE_MAXH * XE_HS; // floats per score tile
  __shared__ __attribute__((aligned(16))) u16 sE[2][NW][SLICE];
  __shared__ __attribute__((aligned(16))) float sS[2][NW][SN];
  __shared__ __attribute__((aligned(16))) float sSum[2][SN];

  const int w = blockIdx.x;
  const long g0 = (long)w * G / n_wg, g1 = (long)(w + 1) * G / n_wg;
  const int n = (int)(g1 - g0);
  const int row0 = (int)(g0 / nsub);
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col0 = wave * WC;
  // sub-tile i of this share: global index, its row and first frame
  auto gidx = [&](int i) -> long { return reverse ? g1 - 1 - i : g0 + i; };
  auto row_of = [&](int i) -> int { return (int)(gidx(i) / nsub); };
  auto t0_of = [&](int i) -> int { return (int)(gidx(i) - (gidx(i) / nsub) * nsub) * XE_F; };

  // ---- E of one sub-tile in the score MFMAs' A layout: register ks of lane
  // l holds frame l % 16, columns 32 ks + 8 (l / 16) .. +7 of the wave's
  // columns; frames past T read frame T - 1 (their scores are masked)
  const int fl = lane & 15, kk = lane >> 4;
  uint4 rg[XE_XR][CB];
  auto gload = [&](int slot, int i) {
    const int r = row_of(i), fr = min(t0_of(i) + fl, T - 1);
    const u16* base = E + (long)(r / rows_per_b) * T * d;
    const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, 0x7fffffff, 0x00020000);
    const uint32_t off = (uint32_t)(fr * d + col0 + kk * 8) * 2;
#pragma unroll
    for (int ks = 0; ks < CB; ++ks)
      rg[slot][ks] = bitcast<uint4>(__builtin_amdgcn_raw_buffer_load_b128(rc, off + ks * 64, 0, 0));
  };
  // into the wave's LDS slice: k-block 2 ks + kk / 2, frame fl, column 8 (kk % 2)
  auto sstore = [&](int slot, int stage) {
    u16* sw = sE[stage][wave];
#pragma unroll
    for (int ks = 0; ks < CB; ++ks) *(uint4*)&sw[xe_off(2 * ks + (kk >> 1), fl, (kk & 1) * 8)] = rg[slot][ks];
  };

  // ---- q' of one row for this wave's columns: the B operand of the score
  // MFMAs, lane l holding head 16 hb + l % 16, columns 32 ks + 8 (l / 16) ..+7
  uint4 qreg[2][CB];
  auto qload = [&](int r) {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int h = hb * 16 + fl;
#pragma unroll
      for (int ks = 0; ks < CB; ++ks) {
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (h < H) v = *(const uint4*)(qp + ((long)r * H + h) * d + col0 + ks * 32 + kk * 8);
        qreg[hb][ks] = v;
      }
    }
  };

  // ---- partial scores of the sub-tile in register stage slot, into
  // sS[buf][wave]: element (frame f, head h) at h * XE_HS + f, real heads only
  auto scores = [&](int slot, int buf) {
    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < CB; ++ks)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
        acc[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8>(rg[slot][ks]), bitcast<bf16x8>(qreg[hb][ks]),
                                                          acc[hb], 0, 0, 0);
    // output lane l, element e: frame 4 (l / 16) + e, head 16 hb + l % 16
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int h = hb * 16 + fl;
      if (h < H) *(f32x4*)&sS[buf][wave][h * XE_HS + kk * 4] = acc[hb];
    }
  };
  // the waves' partials of a score tile summed in wave order (threads < 4 H)
  auto reduce = [&](int buf) {
    if (tid < H * 4) {
      const int e = (tid >> 2) * XE_HS + (tid & 3) * 4;
      f32x4 v = *(const f32x4*)&sS[buf][0][e];
#pragma unroll
      for (int w_ = 1; w_ < NW; ++w_) v += *(const f32x4*)&sS[buf][w_][e];
      *(f32x4*)&sSum[buf][e] = v;
    }
  };

  // ---- softmax state and U accumulators of the current row segment
  const int g = lane >> 5, l32 = lane & 31, jl = lane & 15;
  const bool hv = l32 < H;
  f32x16 o[CB];
  float m_run = -INFINITY, l_run = 0.f;  // running max in base-2 units (score * log2(e) / 8)
  auto reset = [&]() {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[cb][e] = 0.f;
    m_run = -INFINITY;
    l_run = 0.f;
  };
  reset();
  const float cs = 1.4426950408889634f * 0.125f;
  // softmax of sub-tile i's summed scores, then U += E^T P^T from LDS stage st.
  // This lane's frames (in the P fragment's order): 4 g .. 4 g + 3, 8 + 4 g .. 8 + 4 g + 3
  auto softmax_u = [&](int i, int st, int buf) {
    const int t0 = t0_of(i);
    float sc[8];
    if (hv) {
      const f32x4 a = *(const f32x4*)&sSum[buf][l32 * XE_HS + 4 * g];
      const f32x4 b = *(const f32x4*)&sSum[buf][l32 * XE_HS + 8 + 4 * g];
      sc[0] = a[0]; sc[1] = a[1]; sc[2] = a[2]; sc[3] = a[3];
      sc[4] = b[0]; sc[5] = b[1]; sc[6] = b[2]; sc[7] = b[3];
    }
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int fr = t0 + (e >> 2) * 8 + 4 * g + (e & 3);
      // a padded head (not stored) gets zero scores, so its lanes stay finite
      sc[e] = hv ? (fr < T ? sc[e] * cs : -INFINITY) : 0.f;
      mx = fmaxf(mx, sc[e]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    float psum = 0.f;
    uint32_t pk[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const float p0 = __builtin_amdgcn_exp2f(sc[e] - m_new), p1 = __builtin_amdgcn_exp2f(sc[e + 1] - m_new);
      psum += p0 + p1;
      pk[e >> 1] = f2bf2(p0, p1);
    }
    if (__any(m_new > m_run)) {  // exp2(0) = 1 for the lanes whose max did not move
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[cb][e] *= alpha;
    }
    l_run += psum;
    m_run = m_new;
    const bf16x8 pf = bitcast<bf16x8>(make_uint4(pk[0], pk[1], pk[2], pk[3]));
    const u16* sw = sE[st][wave];
    // transposed reads: the 16 lanes of group lane / 16 read a 4-frame x 16-column
    // block; lane jl gets column jl of it
    const int G4 = lane >> 4, fr = (G4 >> 1) * 4 + (jl >> 2);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int kb = cb * 2 + (G4 & 1);
      const uint2 lo = xe_read_tr16(&sw[xe_off(kb, fr, (jl & 3) * 4)]);
      const uint2 hi = xe_read_tr16(&sw[xe_off(kb, fr + 8, (jl & 3) * 4)]);
      o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bitcast<bf16x8>(make_uint4(lo.x, lo.y, hi.x, hi.y)), pf, o[cb], 0,
                                                      0, 0);
    }
  };
  // the segment of row r ends: its unnormalised U, max and sum to its slot
  auto flush = [&](int r) {
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    if (hv) {
      const long slot = ((long)w * kmax + (r - row0)) * H + l32;
      u16* up = upart + slot * d + col0;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          uint2 u;
          u.x = f2bf2(o[cb][e4 * 4 + 0], o[cb][e4 * 4 + 1]);
          u.y = f2bf2(o[cb][e4 * 4 + 2], o[cb][e4 * 4 + 3]);
          *(uint2*)(up + cb * 32 + e4 * 8 + g * 4) = u;
        }
      if (wave == 0 && g == 0) {
        ml[slot * 2 + 0] = m_run;
        ml[slot * 2 + 1] = l_tot;
      }
    }
  };

  // ---- pipeline over one row segment [i0, i1) of the share (q' loaded
  // once). Register stage of sub-tile i0 + j: j % XR; LDS stage and score
  // buffers: j % 2. Prologue: loads of the first XR sub-tiles issued, scores
  // of the first summed, its E in LDS, the next loads issued.
  static_assert(XE_XR == 2, "the prologue and the unrolled loop assume two register stages");
  auto segment = [&](const int i0, const int i1) {
    const int ns = i1 - i0;
    gload(0, i0);
    if (ns > 1) gload(1, i0 + 1);
    qload(row_of(i0));
    scores(0, 0);
    sstore(0, 0);
    if (XE_XR < ns) gload(0, i0 + XE_XR);
    __syncthreads();
    reduce(0);
    // step j with k = (j + 1) % XR, the register stage of sub-tile j + 1,
    // given as a constant (registers cannot be indexed at run time)
    auto step = [&](int j, const int k) __attribute__((always_inline)) {
      // (a) partial scores of sub-tile j + 1, its E into LDS, the loads of
      // sub-tile j + 1 + XR into the freed registers
      if (j + 1 < ns) {
        scores(k, (j + 1) & 1);
        sstore(k, (j + 1) & 1);
        if (j + 1 + XE_XR < ns) gload(k, i0 + j + 1 + XE_XR);
      }
      __syncthreads();
      // (b) softmax and U of sub-tile j; the partials of j + 1 summed
      softmax_u(i0 + j, j & 1, j & 1);
      if (j + 1 < ns) reduce((j + 1) & 1);
    };
    for (int j = 0; j < ns; j += 2) {
      step(j, 1);
      if (j + 1 < ns) step(j + 1, 0);
    }
    flush(row_of(i0));
    reset();
    __syncthreads();  // the next segment reuses the LDS stages and score buffers
  };
  if (n <= 0) return;
  for (int i0 = 0; i0 < n;) {
    const int r = row_of(i0);
    // the segment runs to the share's end or the row's end
    const long lim = reverse ? g1 - (long)r * nsub : (long)(r + 1) * nsub - g0;
    const int i1 = (int)(lim < n ? lim : n);
    segment(i0, i1);
    i0 = i1;
  }
}

// The workgroup count of the plan: one per compute unit, fewer when that
// would give a workgroup fewer than XE_MIN_PER_WG sub-tiles; kmax = the most
// rows one share touches.
void cross_enc_plan(int M, int T, int n_cu, XePlan& p) {
  p.nsub = (T + XE_F - 1) / XE_F;
  p.G = (long)M * p.nsub;
  const long want = (p.G + XE_MIN_PER_WG - 1) / XE_MIN_PER_WG;
  p.n_wg = (int)(want < n_cu ? (want > 1 ? want : 1) : n_cu);
  p.kmax = 1;
  for (int w = 0; w < p.n_wg; ++w) {
    const long a = (long)w * p.G / p.n_wg, b = (long)(w + 1) * p.G / p.n_wg;
    const int k = (int)((b - 1) / p.nsub - a / p.nsub + 1);
    if (k > p.kmax) p.kmax = k;
  }
}

hipError_t launch_attn_cross_enc(const void* qp, const void* E, int M, int H, int T, int d, int rows_per_b,
                                 const XePlan& pl, int reverse, void* upart, float* ml, hipStream_t s) {
  if (M <= 0 || T <= 0 || rows_per_b < 1 || M % rows_per_b || H * 64 != d || H > XE_MAXH) return hipErrorInvalidValue;
  if (pl.nsub != (T + XE_F - 1) / XE_F || pl.G != (long)M * pl.nsub || pl.n_wg <= 0 || pl.kmax <= 0)
    return hipErrorInvalidValue;
#define XE_LAUNCH(NWV, CBV)                                                                                       \
  hipLaunchKernelGGL((attn_cross_enc_kernel<NWV, CBV>), dim3(pl.n_wg), dim3(NWV * 64), 0, s, (const u16*)qp,       \
                     (const u16*)E, H, T, pl.nsub, pl.G, pl.n_wg, pl.kmax, rows_per_b, reverse, (u16*)upart, ml)
  switch (d) {
    case 1280: XE_LAUNCH(8, 5); break;
    case 1024: XE_LAUNCH(8, 4); break;
    case 768: XE_LAUNCH(6, 4); break;
    case 512: XE_LAUNCH(4, 4); break;
    default: return hipErrorInvalidValue;
  }
#undef XE_LAUNCH
  return hipGetLastError();
}

// ------------------------------------------------------------------ combine
// u[m][h][:] = sum_s w_s U_s[h][:] / sum_s w_s l_s over the segments s of row
// m (w_s = exp2(max_s - max)): the shares of workgroups w_first .. w_last,
// in the slot of row m within each share. One workgroup of 256 threads per
// (row, head): the first threads read the segments' slots, maxima and sums
// (at most 256 segments: one per workgroup of the attention) at once, then
// every thread combines 8 columns per pass, with the loads of up to
// XC_SEG segments issued before their sums (a row has 4-5 segments at batch
// 64), in segment order.
constexpr int XC_SEG = 8;
__global__ __launch_bounds__(256) void absorb_combine_kernel(const u16* __restrict__ upart,
                                                             const float* __restrict__ ml, int H, int d, int nsub,
                                                             long G, int n_wg, int kmax, u16* __restrict__ u) {
  __shared__ long s_slot[256];
  __shared__ float s_w[256], s_l[256];
  __shared__ float s_inv;
  const int mh = blockIdx.x, m = mh / H, h = mh - (mh / H) * H, tid = threadIdx.x;
  auto wg_of = [&](long g_) { return (int)(((g_ + 1) * n_wg - 1) / G); };
  const int wf = wg_of((long)m * nsub), ns = wg_of((long)(m + 1) * nsub - 1) - wf + 1;
  float mseg = -INFINITY, lseg = 0.f;
  if (tid < ns) {
    const int w_ = wf + tid;
    const int r0 = (int)(((long)w_ * G / n_wg) / nsub);
    const long slot = ((long)w_ * kmax + (m - r0)) * H + h;
    s_slot[tid] = slot;
    const float2 v = *(const float2*)(ml + slot * 2);
    mseg = v.x;
    lseg = v.y;
  }
  // the row's max over its segments, then each segment's weight
  float mx = mseg;
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  __shared__ float s_mx[4];
  if ((tid & 63) == 0) s_mx[tid >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(s_mx[0], s_mx[1]), fmaxf(s_mx[2], s_mx[3]));
  if (tid < ns) {
    s_w[tid] = __builtin_amdgcn_exp2f(mseg - mx);
    s_l[tid] = lseg;
  }
  __syncthreads();
  if (tid == 0) {
    float den = 0.f;
    for (int k = 0; k < ns; ++k) den += s_w[k] * s_l[k];
    s_inv = 1.0f / den;
  }
  __syncthreads();
  const float inv = s_inv;
  for (int ch = tid; ch < d / 8; ch += 256) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < ns; k0 += XC_SEG) {
      uint4 v[XC_SEG];
#pragma unroll
      for (int k = 0; k < XC_SEG; ++k)
        if (k0 + k < ns) v[k] = *(const uint4*)(upart + s_slot[k0 + k] * d + ch * 8);
#pragma unroll
      for (int k = 0; k < XC_SEG; ++k) {
        if (k0 + k >= ns) break;
        const float wt = s_w[k0 + k];
        const uint32_t a[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] = fmaf(wt, __uint_as_float(a[q] << 16), acc[2 * q]);
          acc[2 * q + 1] = fmaf(wt, __uint_as_float(a[q] & 0xffff0000u), acc[2 * q + 1]);
        }
      }
    }
    *(uint4*)(u + ((long)m * H + h) * d + ch * 8) =
        make_uint4(f2bf2(acc[0] * inv, acc[1] * inv), f2bf2(acc[2] * inv, acc[3] * inv),
                   f2bf2(acc[4] * inv, acc[5] * inv), f2bf2(acc[6] * inv, acc[7] * inv));
  }
}

hipError_t launch_absorb_combine(const void* upart, const float* ml, int M, int H, int d, const XePlan& pl, void* u,
                                 hipStream_t s) {
  if (M <= 0 || H <= 0 || d % 8 || pl.G != (long)M * pl.nsub || pl.n_wg <= 0 || pl.n_wg > 256)
    return hipErrorInvalidValue;  // a row has at most one segment per attention workgroup
  hipLaunchKernelGGL(absorb_combine_kernel, dim3(M * H), dim3(256), 0, s, (const u16*)upart, ml, H, d, pl.nsub, pl.G,
                     pl.n_wg, pl.kmax, (u16*)u);
  return hipGetLastError();
}

}  // namespace wh
