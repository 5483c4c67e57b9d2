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
//   attn_cross_enc_kernel  per (query row, frame chunk): scores S = E q'^T, online
//                          softmax per head, U = P^T E; unnormalised U and the
//                          chunk's (max, sum) per head
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
// consecutive n of one row m (one 8-byte store). Workgroup: one head, 256
// columns n, 64 rows m; wave w takes columns 64 w .. 64 w + 63.
__global__ __launch_bounds__(256) void absorb_q_kernel(const u16* __restrict__ q, const u16* __restrict__ wkt,
                                                       int M, int H, int d, u16* __restrict__ qp) {
  const int h = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = blockIdx.y * 256 + wave * 64, m0 = blockIdx.z * 64;
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
  hipLaunchKernelGGL(absorb_q_kernel, dim3(H, d / 256, (M + 63) / 64), dim3(256), 0, s, (const u16*)q,
                     (const u16*)wkt, M, H, d, (u16*)qp);
  return hipGetLastError();
}

// ------------------------------------------------------------------ attention over E
// One workgroup per (query row m, chunk c of the frames); NW waves, wave w
// owning CB blocks of 32 columns of E (d = NW * CB * 32). Frames go in
// sub-tiles of 32:
//  * S^T [32 frames x 32 heads] = E_sub q'^T with MFMA 32x32x16 (heads padded
//    to 32 with zero rows of q'); each wave contracts its own columns, and the
//    NW partial tiles are summed through LDS;
//  * online softmax per head: in the S^T layout lane l holds head l % 32 for 16
//    of the frames (the other 16 in lane l ^ 32), so its max, sum and rescale
//    factor are per lane;
//  * U^T [32 CB columns x 32 heads] += E_sub^T P^T, the E^T fragments read from
//    the wave's LDS slice with the gfx950 LDS transpose read.
// Streaming: E is read once and decode is bound by HBM, so each wave keeps two
// sub-tiles of loads in flight (two register stages, 2 x 10 KB per wave at
// d = 1280) while it computes on a third held in LDS.
// LDS slice of a wave: 2 CB k-blocks (16 columns each) of 32 frame rows x 32
// bytes; frame f of k-block kb sits at row f ^ (kb & 3), so the fragment reads
// stay conflict-free (a permutation within aligned groups of 4 rows). Each wave
// reads only its own slice.
constexpr int XE_SUB = 32;
// q' rows in LDS are padded by 16 bytes so the 20 rows a fragment read touches
// (one per head, same columns) spread over the banks; partial scores are kept
// for the real heads only: element (i, g, head) of a wave's 32x32 tile at
// i * 2 XE_MAXH + g XE_MAXH + head.
constexpr int XE_MAXH = 20;

__device__ __forceinline__ int xe_off(int kb, int f, int col) {  // u16 offset in a wave's slice
  return kb * 512 + ((f ^ (kb & 3)) << 4) + col;
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 xe_read_tr16(const u16* p) {
  return bitcast<uint2>(__builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p));
}

// NW waves x CB column blocks; QREG: q' held in registers for the whole chunk
// (else in LDS, re-read per sub-tile); STAGES: sub-tiles of loads in flight
// in registers (1 or 2). reverse != 0 walks the chunk's sub-tiles last to
// first (alternate layers reverse, so a layer first re-reads the part of E the
// previous layer read last, while it may still sit in the last-level cache).
template <int NW, int CB, bool QREG, int STAGES>
__global__ __launch_bounds__(NW * 64) void attn_cross_enc_kernel(const u16* __restrict__ qp, const u16* __restrict__ E,
                                                                 int H, int T, int NC, int SPC, int rows_per_b,
                                                                 int reverse, u16* __restrict__ upart,
                                                                 float* __restrict__ ml) {
  constexpr int WC = CB * 32;        // columns per wave
  constexpr int d = NW * WC;
  constexpr int NCH = WC / 8;        // 16-byte chunks per frame row of a wave's slice
  constexpr int QS = WC + 8;         // q' row stride in LDS (u16)
  constexpr int SN = 32 * XE_MAXH;   // stored score elements per wave tile
  constexpr int KS = 2 * CB;         // 16-column k-steps per wave
  __shared__ __attribute__((aligned(16))) u16 sE[NW][2 * CB * 512];
  __shared__ __attribute__((aligned(16))) u16 sQ[QREG ? 1 : NW][QREG ? 8 : XE_MAXH * QS];
  __shared__ __attribute__((aligned(16))) float sS[NW][SN];
  __shared__ __attribute__((aligned(16))) float sSum[SN];
  const int m = blockIdx.x / NC, c = blockIdx.x - (blockIdx.x / NC) * NC;
  // the wave index is uniform across the wave: keep it (and the slice base and
  // buffer resource derived from it) in scalar registers
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const int col0 = wave * WC;
  const bool hv = l32 < H;  // this lane's head is real (H <= XE_MAXH)
  const u16* Eb = E + (long)(m / rows_per_b) * T * d + col0;
  const int t_begin = c * SPC * XE_SUB, t_end = min(T, t_begin + SPC * XE_SUB);
  const int nsub = (t_end - t_begin + XE_SUB - 1) / XE_SUB;
  u16* sw = sE[wave];
  // lane-major score tiles: a real-head lane's 16 values (frames of its half g)
  // are 16 consecutive floats at (g * XE_MAXH + l32) * 16
  const int so = (g * XE_MAXH + l32) * 16;

  // q' of this row and this wave's columns (the B operand of the score MFMAs:
  // lane holds head l32, columns ks*16 + g*8 .. +7)
  bf16x8 qreg[QREG ? KS : 1];
  u16* sq = sQ[QREG ? 0 : wave];
  if constexpr (QREG) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (hv) v = *(const uint4*)(qp + ((long)m * H + l32) * d + col0 + ks * 16 + g * 8);
      qreg[ks] = bitcast<bf16x8>(v);
    }
  } else {
    for (int e = lane; e < H * NCH; e += 64) {
      const int h = e / NCH, k = e - (e / NCH) * NCH;
      *(uint4*)&sq[h * QS + k * 8] = *(const uint4*)(qp + ((long)m * H + h) * d + col0 + k * 8);
    }
  }

  // staging of a sub-tile (32 frames x WC columns): loads 0..7 of a lane take
  // frame 4 i + lane / 16, 16-byte chunk lane % 16 of the first 128 columns
  // (4 frames x 256 bytes per instruction); for CB = 5, loads 8, 9 take frame
  // lane / 4 + 16 j, chunk 16 + lane % 4 of the last 32 columns. Every LDS
  // store of a lane is its base plus a constant. Frames past T read frame
  // T - 1 (their scores are masked). Buffer loads take a 32-bit byte offset
  // from the wave's base.
  static_assert(CB == 4 || CB == 5, "128 or 160 columns per wave");
  constexpr int NLD = CB == 5 ? 10 : 8;
  const __amdgpu_buffer_rsrc_t erc = __builtin_amdgcn_make_buffer_rsrc((void*)Eb, (short)0, 0x7fffffff, 0x00020000);
  const int ka = lane & 15, fa = lane >> 4;       // pattern A
  const int kb4 = 16 + (lane & 3), fb = lane >> 2;  // pattern B (CB = 5)
  u16* const sta = &sw[xe_off(ka >> 1, fa, (ka & 1) * 8)];   // + 64 i
  u16* const stb = &sw[xe_off(kb4 >> 1, fb, (kb4 & 1) * 8)];  // + 256 j
  uint4 ra[NLD], rb[STAGES == 2 ? NLD : 1];
  auto tsub = [&](int s_) { return t_begin + (reverse ? nsub - 1 - s_ : s_) * XE_SUB; };
  auto gload = [&](uint4* rg, int t0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int fr = min(t0 + i * 4 + fa, T - 1);
      rg[i] = bitcast<uint4>(__builtin_amdgcn_raw_buffer_load_b128(erc, (uint32_t)(fr * d * 2 + ka * 16), 0, 0));
    }
    if constexpr (CB == 5) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int fr = min(t0 + j * 16 + fb, T - 1);
        rg[8 + j] = bitcast<uint4>(__builtin_amdgcn_raw_buffer_load_b128(erc, (uint32_t)(fr * d * 2 + kb4 * 16), 0, 0));
      }
    }
  };
  auto sstore = [&](const uint4* rg) {
#pragma unroll
    for (int i = 0; i < 8; ++i) *(uint4*)(sta + i * 64) = rg[i];
    if constexpr (CB == 5) {
#pragma unroll
      for (int j = 0; j < 2; ++j) *(uint4*)(stb + j * 256) = rg[8 + j];
    }
  };

  f32x16 o[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[cb][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;  // running max in base-2 units (score * log2(e) / 8), per head
  const float cs = 1.4426950408889634f * 0.125f;
  // E^T fragment addressing (see xe_read_tr16): group G = lane / 16 serves
  // k-block cb*2 + (G & 1) and frame quad G >> 1 of each 8 frames
  const int G = lane >> 4, jl = lane & 15;

  // one sub-tile held in LDS, starting at frame t0
  auto compute = [&](const int t0) {
    // ---- partial scores over this wave's columns
    f32x16 st;
#pragma unroll
    for (int i = 0; i < 16; ++i) st[i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 ef = bitcast<bf16x8>(*(const uint4*)&sw[xe_off(ks, l32, g * 8)]);
      bf16x8 qf;
      if constexpr (QREG) {
        qf = qreg[ks];
      } else {
        uint4 qv = make_uint4(0u, 0u, 0u, 0u);
        if (hv) qv = *(const uint4*)&sq[l32 * QS + ks * 16 + g * 8];
        qf = bitcast<bf16x8>(qv);
      }
      st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ef, qf, st, 0, 0, 0);
    }
    if (hv) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        *(f32x4*)&sS[wave][so + i4 * 4] = f32x4{st[i4 * 4], st[i4 * 4 + 1], st[i4 * 4 + 2], st[i4 * 4 + 3]};
    }
    __syncthreads();
    for (int e = tid * 4; e < SN; e += NW * 64 * 4) {
      f32x4 v = *(const f32x4*)&sS[0][e];
#pragma unroll
      for (int w = 1; w < NW; ++w) v += *(const f32x4*)&sS[w][e];
      *(f32x4*)&sSum[e] = v;
    }
    __syncthreads();
    // ---- online softmax of this lane's head over the sub-tile's frames
    float sc[16];
    if (hv) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x4 v = *(const f32x4*)&sSum[so + i4 * 4];
        sc[i4 * 4] = v[0]; sc[i4 * 4 + 1] = v[1]; sc[i4 * 4 + 2] = v[2]; sc[i4 * 4 + 3] = v[3];
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int fr = t0 + (i >> 2) * 8 + g * 4 + (i & 3);
      // a padded head (not stored) gets zero scores, so its lanes stay finite
      sc[i] = hv ? (fr < t_end ? sc[i] * cs : -INFINITY) : 0.f;
      mx = fmaxf(mx, sc[i]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    // probabilities, packed to bf16 at once: P^T fragment t holds sc[8 t .. 8 t + 7]
    float psum = 0.f;
    uint32_t pk[8];
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      const float p0 = __builtin_amdgcn_exp2f(sc[i] - m_new), p1 = __builtin_amdgcn_exp2f(sc[i + 1] - m_new);
      psum += p0 + p1;
      pk[i >> 1] = f2bf2(p0, p1);
    }
    if (__any(m_new > m_run)) {  // exp2(0) = 1 for the lanes whose max did not move
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[cb][i] *= alpha;
    }
    l_run += psum;
    m_run = m_new;
    // ---- U^T += E^T P^T over the two 16-frame k-blocks of the sub-tile
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const bf16x8 pf = bitcast<bf16x8>(make_uint4(pk[t * 4 + 0], pk[t * 4 + 1], pk[t * 4 + 2], pk[t * 4 + 3]));
      const int fr = t * 16 + (G >> 1) * 4 + (jl >> 2);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int kb = cb * 2 + (G & 1);
        const uint2 lo = xe_read_tr16(&sw[xe_off(kb, fr, (jl & 3) * 4)]);
        const uint2 hi = xe_read_tr16(&sw[xe_off(kb, fr + 8, (jl & 3) * 4)]);
        o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bitcast<bf16x8>(make_uint4(lo.x, lo.y, hi.x, hi.y)), pf, o[cb],
                                                        0, 0, 0);
      }
    }
  };

  // Pipeline: sub-tile s in LDS, the next STAGES in flight in registers. The
  // slice is private to the wave and its own reads of s have completed (their
  // values fed the MFMAs) before s + 1 is stored over it.
  gload(ra, tsub(0));
  sstore(ra);
  if (nsub > 1) gload(ra, tsub(1));
  if constexpr (STAGES == 2) {
    if (nsub > 2) gload(rb, tsub(2));
    for (int s = 0; s < nsub; s += 2) {
      compute(tsub(s));
      if (s + 1 >= nsub) break;
      sstore(ra);
      if (s + 3 < nsub) gload(ra, tsub(s + 3));
      compute(tsub(s + 1));
      if (s + 2 >= nsub) break;
      sstore(rb);
      if (s + 4 < nsub) gload(rb, tsub(s + 4));
    }
  } else {
    for (int s = 0; s < nsub; ++s) {
      compute(tsub(s));
      if (s + 1 < nsub) sstore(ra);
      if (s + 2 < nsub) gload(ra, tsub(s + 2));
    }
  }
  // ---- this chunk's unnormalised U, max and sum per head
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (hv) {
    const long row = ((long)m * NC + c) * H + l32;
    u16* up = upart + row * d + col0;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        uint2 u;
        u.x = f2bf2(o[cb][i4 * 4 + 0], o[cb][i4 * 4 + 1]);
        u.y = f2bf2(o[cb][i4 * 4 + 2], o[cb][i4 * 4 + 3]);
        *(uint2*)(up + cb * 32 + i4 * 8 + g * 4) = u;
      }
    if (wave == 0 && g == 0) {
      ml[row * 2 + 0] = m_run;
      ml[row * 2 + 1] = l_tot;
    }
  }
}

// Frame chunks per query row: the count that balances rounds of workgroups
// (one per compute unit) against sub-tiles per workgroup; no chunk is empty.
void cross_enc_chunks(int M, int T, int n_cu, int& NC, int& SPC) {
  const int nsub = (T + XE_SUB - 1) / XE_SUB;
  long best = -1;
  NC = 1;
  SPC = nsub;
  for (int nc = 1; nc <= nsub; ++nc) {
    const int spc = (nsub + nc - 1) / nc;
    const int nc_eff = (nsub + spc - 1) / spc;
    const long rounds = ((long)M * nc_eff + n_cu - 1) / n_cu;
    const long cost = rounds * spc;
    if (best < 0 || cost < best) {
      best = cost;
      NC = nc_eff;
      SPC = spc;
    }
  }
}

hipError_t launch_attn_cross_enc(const void* qp, const void* E, int M, int H, int T, int d, int rows_per_b, int NC,
                                 int SPC, int reverse, void* upart, float* ml, hipStream_t s) {
  if (M <= 0 || T <= 0 || NC <= 0 || SPC <= 0 || rows_per_b < 1 || M % rows_per_b || H * 64 != d || H > XE_MAXH)
    return hipErrorInvalidValue;
  if ((long)(NC - 1) * SPC * XE_SUB >= T) return hipErrorInvalidValue;  // an empty chunk
#define XE_LAUNCH(NWV, CBV, QR, ST)                                                                              \
  hipLaunchKernelGGL((attn_cross_enc_kernel<NWV, CBV, QR, ST>), dim3(M * NC), dim3(NWV * 64), 0, s, (const u16*)qp, \
                     (const u16*)E, H, T, NC, SPC, rows_per_b, reverse, (u16*)upart, ml)
  switch (d) {
    case 1280: XE_LAUNCH(8, 5, true, 1); break;
    case 1024: XE_LAUNCH(8, 4, true, 1); break;
    case 768: XE_LAUNCH(6, 4, true, 1); break;
    case 512: XE_LAUNCH(4, 4, true, 1); break;
    default: return hipErrorInvalidValue;
  }
#undef XE_LAUNCH
  return hipGetLastError();
}

// ------------------------------------------------------------------ combine
// u[m][h][:] = sum_c w_c U_c[m][h][:] / sum_c w_c l_c,  w_c = exp2(max_c - max).
// One workgroup of 256 threads per (row, head); 8 columns per thread and pass.
__global__ __launch_bounds__(256) void absorb_combine_kernel(const u16* __restrict__ upart,
                                                             const float* __restrict__ ml, int H, int d, int NC,
                                                             u16* __restrict__ u) {
  const int mh = blockIdx.x, m = mh / H, h = mh - (mh / H) * H;
  float mx = -INFINITY;
  for (int c = 0; c < NC; ++c) mx = fmaxf(mx, ml[(((long)m * NC + c) * H + h) * 2]);
  float den = 0.f;
  for (int c = 0; c < NC; ++c) {
    const long r = ((long)m * NC + c) * H + h;
    den += __builtin_amdgcn_exp2f(ml[r * 2] - mx) * ml[r * 2 + 1];
  }
  const float inv = 1.0f / den;
  for (int ch = threadIdx.x; ch < d / 8; ch += 256) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < NC; ++c) {
      const long r = ((long)m * NC + c) * H + h;
      const float w = __builtin_amdgcn_exp2f(ml[r * 2] - mx);
      const uint4 v = *(const uint4*)(upart + r * d + ch * 8);
      const uint32_t a[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        acc[2 * k] = fmaf(w, __uint_as_float(a[k] << 16), acc[2 * k]);
        acc[2 * k + 1] = fmaf(w, __uint_as_float(a[k] & 0xffff0000u), acc[2 * k + 1]);
      }
    }
    *(uint4*)(u + ((long)m * H + h) * d + ch * 8) =
        make_uint4(f2bf2(acc[0] * inv, acc[1] * inv), f2bf2(acc[2] * inv, acc[3] * inv),
                   f2bf2(acc[4] * inv, acc[5] * inv), f2bf2(acc[6] * inv, acc[7] * inv));
  }
}

hipError_t launch_absorb_combine(const void* upart, const float* ml, int M, int H, int d, int NC, void* u,
                                 hipStream_t s) {
  if (M <= 0 || H <= 0 || NC <= 0 || d % 8) return hipErrorInvalidValue;
  hipLaunchKernelGGL(absorb_combine_kernel, dim3(M * H), dim3(256), 0, s, (const u16*)upart, ml, H, d, NC, (u16*)u);
  return hipGetLastError();
}

}  // namespace wh
