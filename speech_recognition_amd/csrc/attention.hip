// Attention kernels of the hot path, after the whisper_blaze showcase page's
// flash_attn_hopper.cu card ("The Solution"): encoder self-attention, decoder
// causal self-attention and decoder cross-attention, each with an online or
// LDS-resident softmax so no score matrix ever reaches HBM. Scale 1/sqrt(64).
//
// Encoder (bf16): one workgroup per (chunk, head, 128 queries); each wave owns
// 32 queries. Scores are computed transposed, S^T = K Q^T, with MFMA 32x32x16
// so the C layout puts one query per lane column: that query's running max,
// sum and output rows all live in the same lane and the softmax needs a
// single cross-lane exchange (lane ^ 32). P^T then feeds O^T = V^T P^T
// directly from registers; V stays key-major in LDS (stored like K) and its
// transposed fragments come from LDS transpose reads.
//
// Decoder self-attention reads the caller's e4m3 KV cache and dequantises on
// read (the Inference Endpoints post, "Inference Stack": K/V stored as float8,
// compute in bfloat16). Decoder cross-attention streams head-major bf16 K/V
// in one pass per (row, head); its fp8 form (E4M3 or E5M2 codes with
// per-tensor scales, the showcase page's precision presets) runs through the
// fp8 decode kernel over all frames.
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace wh {

// ------------------------------------------------------------------ encoder, bf16 MFMA
__device__ __forceinline__ int k_swz(int row, int kc) { return row * 64 + ((kc ^ (row & 7)) << 3); }

// V^T fragment straight from the key-major V tile with the gfx950 LDS
// transpose read (ds_read_b64_tr_b16): in each group of 16 lanes, lane j
// names 4 consecutive 16-bit elements (8 bytes); the group's 16 x 4 elements,
// in lane order, form a sequence E of 64, and lane i receives E[i], E[16+i],
// E[32+i], E[48+i]. When lane j of the group points at key k0 + j/4, columns
// e0 + 4(j%4) .. +3, lane i receives keys k0 .. k0+3 of column e0 + i.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_read_tr16(const u16* p) {
  return bitcast<uint2>(__builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p));
}

// eight fp32 -> bf16 with the gfx950 converter (round to nearest even; the
// probabilities packed here are finite)
__device__ __forceinline__ bf16x8 pack_bf16x8(float a0, float a1, float a2, float a3, float a4, float a5, float a6,
                                              float a7) {
  return bitcast<bf16x8>(make_uint4(f2bf2(a0, a1), f2bf2(a2, a3), f2bf2(a4, a5), f2bf2(a6, a7)));
}

// 4 waves per SIMD (at most 128 registers): the softmax between the two MFMA
// groups of a tile is VALU work, and more resident waves keep the matrix
// cores busy across it (2 -> 4 waves per SIMD measured 1.49 -> 1.21 ms per
// layer at batch 64; the only spill is one pointer kept over the tile loop)
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 8))) void attn_encoder_bf16(const u16* __restrict__ qkv, int T, int H, int B,
                                                         u16* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) u16 sK[2][64 * 64];
  __shared__ __attribute__((aligned(16))) u16 sV[2][64 * 64];
  const int d = H * 64, ld = 3 * d;
  // XCD-aware order (block L runs on XCD L % 8): the query tiles of one
  // (chunk, head) get consecutive slots on one XCD, so its K/V are fetched
  // into that XCD's L2 once instead of once per query tile.
  const int QT = (T + 127) / 128;
  const int L = blockIdx.x, xcdi = L & 7, jj = L >> 3;
  const int bh = (jj / QT) * 8 + xcdi, qtile = jj - (jj / QT) * QT;
  if (bh >= B * H) return;  // padding blocks ((chunk, head) count rounded up to a multiple of 8)
  const int b = bh / H, h = bh - (bh / H) * H;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const u16* Qp = qkv + (long)b * T * ld + h * 64;
  const u16* Kp = Qp + d;
  const u16* Vp = Qp + 2 * d;
  const int q0 = qtile * 128 + wave * 32;
  const int qi = min(q0 + l32, T - 1);

  bf16x8 qf[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) qf[s] = bitcast<bf16x8>(*(const uint4*)(Qp + (long)qi * ld + s * 16 + g * 8));

  // tile loader: 64 keys x 64 dims of K and of V, 2 chunks of 16 B each per thread
  // thread stages chunk kc of keys row and row + 32 (8 dims = 16 bytes each)
  const int row = tid >> 3, kc = tid & 7;
  uint4 rk0, rk1, rv0, rv1;
  auto gload = [&](int kb) {
    const int k0 = min(kb * 64 + row, T - 1), k1 = min(kb * 64 + row + 32, T - 1);
    rk0 = *(const uint4*)(Kp + (long)k0 * ld + kc * 8);
    rk1 = *(const uint4*)(Kp + (long)k1 * ld + kc * 8);
    rv0 = *(const uint4*)(Vp + (long)k0 * ld + kc * 8);
    rv1 = *(const uint4*)(Vp + (long)k1 * ld + kc * 8);
  };
  auto sstore = [&](int buf) {
    *(uint4*)&sK[buf][k_swz(row, kc)] = rk0;
    *(uint4*)&sK[buf][k_swz(row + 32, kc)] = rk1;
    *(uint4*)&sV[buf][k_swz(row, kc)] = rv0;
    *(uint4*)&sV[buf][k_swz(row + 32, kc)] = rv1;
  };
  // this lane's part of the transpose reads: group G = lane / 16 serves columns
  // 16 (G & 1) .. +15 of a 32-column block and key quad G >> 1 of each 8 keys
  const int tr_key = ((lane >> 5) << 2) + ((lane & 15) >> 2);        // key offset within 8
  const int tr_col = (((lane >> 4) & 1) << 4) + ((lane & 3) << 2);   // column offset within 32
  auto v_addr = [&](int key, int col) { return key * 64 + ((((col >> 3) ^ (key & 7))) << 3) + (col & 7); };

  f32x16 o[2];
#pragma unroll
  for (int e = 0; e < 2; ++e)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[e][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float c = 1.4426950408889634f * 0.125f;  // log2(e) / sqrt(64)
  const int nkb = (T + 63) / 64;

  // One 64-key tile: S^T = K Q^T, online softmax (base-2 exponent with the
  // 1/sqrt(64) scale folded in), O^T += V^T P^T. Only the last tile can run
  // past T, so the key mask is compiled into that copy alone; the output rows
  // are rescaled only when some lane's running max moved.
  auto tile = [&](const int kb, const bool last) {
    const int cur = kb & 1;
    f32x16 st[2];
#pragma unroll
    for (int j2 = 0; j2 < 2; ++j2) {
#pragma unroll
      for (int i = 0; i < 16; ++i) st[j2][i] = 0.f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8 kf = bitcast<bf16x8>(*(const uint4*)&sK[cur][k_swz(j2 * 32 + l32, s * 2 + g)]);
        st[j2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], st[j2], 0, 0, 0);
      }
    }
    if (last) {
#pragma unroll
      for (int j2 = 0; j2 < 2; ++j2)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kb * 64 + j2 * 32 + (i >> 2) * 8 + g * 4 + (i & 3);
          if (key >= T) st[j2][i] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int j2 = 0; j2 < 2; ++j2)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, st[j2][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float mc = m_new * c;
    float psum = 0.f;
#pragma unroll
    for (int j2 = 0; j2 < 2; ++j2)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(st[j2][i], c, -mc));
        st[j2][i] = p;
        psum += p;
      }
    if (__any(m_new > m_run)) {  // wave-uniform: exp2(0) = 1 for the lanes whose max did not move
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);
      l_run *= alpha;
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[e][i] *= alpha;
    }
    l_run += psum;
    m_run = m_new;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int j2 = t >> 1, hs = (t & 1) * 8;
      const bf16x8 pf = pack_bf16x8(st[j2][hs + 0], st[j2][hs + 1], st[j2][hs + 2], st[j2][hs + 3],
                                    st[j2][hs + 4], st[j2][hs + 5], st[j2][hs + 6], st[j2][hs + 7]);
#pragma unroll
      for (int eb = 0; eb < 2; ++eb) {
        // V^T rows eb*32 + l32, keys t*16 + 4g + 0..3 and t*16 + 8 + 4g + 0..3 (the
        // key order of the P^T fragment)
        const uint2 lo = lds_read_tr16(&sV[cur][v_addr(t * 16 + tr_key, eb * 32 + tr_col)]);
        const uint2 hi = lds_read_tr16(&sV[cur][v_addr(t * 16 + 8 + tr_key, eb * 32 + tr_col)]);
        const uint4 vv = make_uint4(lo.x, lo.y, hi.x, hi.y);
        o[eb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bitcast<bf16x8>(vv), pf, o[eb], 0, 0, 0);
      }
    }
  };

  gload(0);
  sstore(0);
  __syncthreads();
  const bool ragged = nkb * 64 > T;
  const int nfull = ragged ? nkb - 1 : nkb;
  for (int kb = 0; kb < nfull; ++kb) {
    if (kb + 1 < nkb) gload(kb + 1);
    tile(kb, false);
    if (kb + 1 < nkb) sstore((kb & 1) ^ 1);
    __syncthreads();
  }
  if (ragged) tile(nkb - 1, true);
  const float l = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.0f / l;
  // the output row and column group from the lane id again (mbcnt needs no
  // input register), so nothing address-like stays live across the key loop
  const int lane_o = __lane_id(), go = lane_o >> 5;
  const int q = q0 + (lane_o & 31);
  if (q < T) {
    u16* op = out + (long)(b * T) * d + h * 64 + (uint32_t)(q * d);
#pragma unroll
    for (int eb = 0; eb < 2; ++eb)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        uint2 u;
        u.x = (uint32_t)f2bf(o[eb][i4 * 4 + 0] * inv) | ((uint32_t)f2bf(o[eb][i4 * 4 + 1] * inv) << 16);
        u.y = (uint32_t)f2bf(o[eb][i4 * 4 + 2] * inv) | ((uint32_t)f2bf(o[eb][i4 * 4 + 3] * inv) << 16);
        *(uint2*)(op + eb * 32 + i4 * 8 + go * 4) = u;
      }
  }
}

// ------------------------------------------------------------------ encoder, fp32 SIMT (tiny fp32 config)
// One thread per query; 64 keys at a time staged in LDS; online softmax.
__global__ __launch_bounds__(64) void attn_encoder_f32(const float* __restrict__ qkv, int T, int H,
                                                       float* __restrict__ out) {
  __shared__ float sK[64][65];
  __shared__ float sV[64][65];
  const int d = H * 64, ld = 3 * d;
  const int b = blockIdx.z, h = blockIdx.y, tid = threadIdx.x;
  const int q = blockIdx.x * 64 + tid;
  const float* base = qkv + (long)b * T * ld + h * 64;
  float qv[64], o[64];
  const int qc = min(q, T - 1);
#pragma unroll
  for (int e = 0; e < 64; ++e) { qv[e] = base[(long)qc * ld + e] * 0.125f; o[e] = 0.f; }
  float m = -INFINITY, l = 0.f;
  for (int k0 = 0; k0 < T; k0 += 64) {
    __syncthreads();
    for (int r = 0; r < 64; ++r) {
      const int key = min(k0 + r, T - 1);
      sK[r][tid] = base[(long)key * ld + d + tid];
      sV[r][tid] = base[(long)key * ld + 2 * d + tid];
    }
    __syncthreads();
    const int nk = min(64, T - k0);
    for (int r = 0; r < nk; ++r) {
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < 64; ++e) s = fmaf(qv[e], sK[r][e], s);
      const float mn = fmaxf(m, s);
      const float a = expf(m - mn), p = expf(s - mn);
      l = l * a + p;
#pragma unroll
      for (int e = 0; e < 64; ++e) o[e] = o[e] * a + p * sV[r][e];
      m = mn;
    }
  }
  if (q < T) {
    float* op = out + ((long)b * T + q) * d + h * 64;
#pragma unroll
    for (int e = 0; e < 64; ++e) op[e] = o[e] / l;
  }
}

hipError_t launch_attn_encoder(ActType t, const void* qkv, int B, int T, int H, void* out, hipStream_t s) {
  if (t == ACT_BF16)
    hipLaunchKernelGGL(attn_encoder_bf16, dim3((T + 127) / 128 * ((B * H + 7) / 8) * 8), dim3(256), 0, s,
                       (const u16*)qkv, T, H, B, (u16*)out);
  else
    hipLaunchKernelGGL(attn_encoder_f32, dim3((T + 63) / 64, H, B), dim3(64), 0, s, (const float*)qkv, T, H,
                       (float*)out);
  return hipGetLastError();
}

// ------------------------------------------------------------------ decoder attention over fp8 codes
// Keys 0..n-1 (n = lengths[b] + len_add, or all cap keys when lengths is
// NULL, as for the fp8 cross-attention K/V) are 64-byte code rows read as 4
// lanes x 16 codes, in E4M3 (the KV cache) or E5M2 (an option for the
// cross-attention K/V, for range), decoded by the gfx950 converters.
constexpr int DEC_MAX_CAP = 4096;

// Sums over 4 or 8 consecutive lanes with DPP lane permutes folded into the
// adds (no trip through the LDS crossbar as a generic shuffle takes):
// quad_perm(1,0,3,2) and (2,3,0,1) pair lanes within a quad, row_half_mirror
// (lane i <-> 7 - i of each 8) pairs the two quads of an 8-lane group.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float sum4_lanes(float d) {
  d += dpp_f<0xB1>(d);
  return d + dpp_f<0x4E>(d);
}
__device__ __forceinline__ float sum8_lanes(float d) {
  d = sum4_lanes(d);
  return d + dpp_f<0x141>(d);
}
constexpr float LOG2E = 1.4426950408889634f;

template <int FMT>
__device__ __forceinline__ float dot16_fp8(const uint4 c, const float* q) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float v[4];
    fp8x4_decode<FMT>(w[i], v);
#pragma unroll
    for (int k = 0; k < 4; ++k) acc = fmaf(q[4 * i + k], v[k], acc);
  }
  return acc;
}

// One workgroup per (row, head). Lane (part = tid & 3, kg = tid >> 2) owns 16
// of the 64 dims of keys kg, kg + 64, ...; per batch of SELF_KB keys it loads
// the K and V codes together (addresses clamped to the last valid key, so the
// batch is straight-line code and all its loads are in flight at once), keeps
// a private online softmax (running max, sum and 16 output dims), and the 256
// private states are merged once at the end: block max, rescale, sum over
// the 64 key groups (DPP within each 16-lane row, LDS across the 16 rows).
// q goes straight from global to registers. Given a row order (longest cache
// first), workgroup y takes row order[y]: the longest rows start in the first
// round of workgroups and the shortest fill the last one.
constexpr int SELF_KB = 8;

template <typename T, int FMT>
__global__ __launch_bounds__(256) void attn_decode_self_kernel(const T* __restrict__ q, long q_stride,
                                                               const uint8_t* __restrict__ kc,
                                                               const uint8_t* __restrict__ vc,
                                                               const float* __restrict__ scales,
                                                               const int32_t* __restrict__ lengths, int len_add, int H,
                                                               int cap, T* __restrict__ out, int rows_per_b,
                                                               const int2* __restrict__ order) {
  __shared__ __attribute__((aligned(16))) float red[16][64];
  __shared__ float rowmax[16], rsum[16];
  const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // with order (one query row per cache row): workgroups take rows longest
  // first, each row's length read with its index
  int b = blockIdx.y, len = 0;
  if (order) {
    const int2 o = order[blockIdx.y];
    b = o.x;
    len = o.y;
  } else if (lengths) {
    len = lengths[b / rows_per_b];
  }
  const int bc = b / rows_per_b;  // cache batch row of query row b
  const int n = (lengths || order) ? max(0, min(len + len_add + b % rows_per_b, cap)) : cap;
  const int part = tid & 3, kg = tid >> 2;
  float qreg[16];
  {
    const T* qp = q + (long)b * q_stride + h * 64 + part * 16;
#pragma unroll
    for (int i = 0; i < 16; ++i) qreg[i] = Act<T>::cvt(qp[i]);
  }
  const float sscale = scales[0] * (0.125f * LOG2E), sv = scales[1];  // scores in base-2 units
  const long head = ((long)bc * H + h) * cap * 64 + part * 16;
  const uint8_t* K = kc + head;
  const uint8_t* V = vc + head;
  float m = -INFINITY, l = 0.f, acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  for (int base = 0; base < n; base += 64 * SELF_KB) {
    uint4 ck[SELF_KB], cv[SELF_KB];
#pragma unroll
    for (int i = 0; i < SELF_KB; ++i) {
      const long j = min(base + kg + 64 * i, n - 1);
      ck[i] = *(const uint4*)(K + j * 64);
      cv[i] = *(const uint4*)(V + j * 64);
    }
    __builtin_amdgcn_sched_barrier(0);
    // key slot i of this wave covers keys base + 64 i + 16 wave .. + 15: a slot
    // wholly past n is skipped by the whole wave (its loads were clamped)
    float sj[SELF_KB];
    float bm = -INFINITY;
#pragma unroll
    for (int i = 0; i < SELF_KB; ++i) {
      sj[i] = -INFINITY;
      if (base + 64 * i + 16 * wave < n) {
        const float d = sum4_lanes(dot16_fp8<FMT>(ck[i], qreg));
        if (base + kg + 64 * i < n) sj[i] = d * sscale;
      }
      bm = fmaxf(bm, sj[i]);
    }
    const float mn = fmaxf(m, bm);
    const float alpha = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - mn);
    l *= alpha;
#pragma unroll
    for (int k = 0; k < 16; ++k) acc[k] *= alpha;
#pragma unroll
    for (int i = 0; i < SELF_KB; ++i) {
      if (!(base + 64 * i + 16 * wave < n)) continue;
      const float p = (sj[i] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sj[i] - mn);
      l += p;
      const uint32_t w[4] = {cv[i].x, cv[i].y, cv[i].z, cv[i].w};
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        float v[4];
        fp8x4_decode<FMT>(w[e4], v);
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[4 * e4 + k] = fmaf(p, v[k], acc[4 * e4 + k]);
      }
    }
    m = mn;
  }
  // merge the private states. A 16-lane row holds key groups 4 r .. 4 r + 3
  // of its wave, each in 4 parts: the row's max and the sums over its 4 key
  // groups of equal part (scaled to that max) come from DPP row rotations
  // (VALU, no LDS traffic); the 16 rows of the block then meet in LDS once:
  // each output dim rescales the rows' sums to the block max as it adds them.
  const int rrow = wave * 4 + (lane >> 4);  // this lane's row, 0..15
  float rm = m;
  rm = fmaxf(rm, dpp_f<0x128>(rm));  // row_ror:8
  rm = fmaxf(rm, dpp_f<0x124>(rm));  // row_ror:4
  rm = fmaxf(rm, dpp_f<0x122>(rm));  // row_ror:2
  rm = fmaxf(rm, dpp_f<0x121>(rm));  // row_ror:1
  const float f = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - rm);
  float ls = l * f;
  ls += dpp_f<0x128>(ls);
  ls += dpp_f<0x124>(ls);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float a = acc[i] * f;
    a += dpp_f<0x128>(a);
    a += dpp_f<0x124>(a);
    acc[i] = a;
  }
  if ((lane & 12) == 0) {  // lanes 0..3 of the row: its 4 parts
#pragma unroll
    for (int i = 0; i < 16; i += 4)
      *(float4*)&red[rrow][part * 16 + i] = make_float4(acc[i], acc[i + 1], acc[i + 2], acc[i + 3]);
    if (part == 0) {
      rsum[rrow] = ls;
      rowmax[rrow] = rm;
    }
  }
  __syncthreads();
  if (tid < 64) {
    float mx = rowmax[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, rowmax[r]);
    float sum = 0.f, sacc = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float w = rowmax[r] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(rowmax[r] - mx);
      sum = fmaf(rsum[r], w, sum);
      sacc = fmaf(red[r][tid], w, sacc);
    }
    const float v = (n > 0) ? sacc * sv / sum : 0.f;
    out[(long)b * H * 64 + h * 64 + tid] = Act<T>::st(v);
  }
}

template <int FMT>
static void decode_self_fmt(ActType t, const void* q, long q_stride, const uint8_t* k_codes, const uint8_t* v_codes,
                            const float* scales, const int32_t* lengths, int len_add, int B, int H, int cap,
                            void* out, hipStream_t s, int rows_per_b, const int2* order) {
  dim3 grid(H, B);
  if (t == ACT_BF16)
    hipLaunchKernelGGL((attn_decode_self_kernel<u16, FMT>), grid, dim3(256), 0, s, (const u16*)q, q_stride, k_codes,
                       v_codes, scales, lengths, len_add, H, cap, (u16*)out, rows_per_b, order);
  else
    hipLaunchKernelGGL((attn_decode_self_kernel<float, FMT>), grid, dim3(256), 0, s, (const float*)q, q_stride,
                       k_codes, v_codes, scales, lengths, len_add, H, cap, (float*)out, rows_per_b, order);
}

hipError_t launch_attn_decode_self(ActType t, const void* q, long q_stride, const uint8_t* k_codes,
                                   const uint8_t* v_codes, const float* scales, const int32_t* lengths, int len_add,
                                   int B, int H, int cap, void* out, hipStream_t s, int rows_per_b, int fmt,
                                   const int2* order) {
  if (cap > DEC_MAX_CAP || rows_per_b < 1 || B % rows_per_b || (order && rows_per_b != 1)) return hipErrorInvalidValue;
  if (fmt == FP8_E5M2)
    decode_self_fmt<FP8_E5M2>(t, q, q_stride, k_codes, v_codes, scales, lengths, len_add, B, H, cap, out, s,
                              rows_per_b, order);
  else
    decode_self_fmt<FP8_E4M3>(t, q, q_stride, k_codes, v_codes, scales, lengths, len_add, B, H, cap, out, s,
                              rows_per_b, order);
  return hipGetLastError();
}

// ------------------------------------------------------------------ decoder cross-attention
// One workgroup per (row, head) streams that head's whole K and V slabs
// (1500 x 64 each, head-major, so a wave's 16-byte loads cover 1 KB of
// consecutive key rows). Lane (part, kg) owns EPT of the 64 dims of keys
// kg, kg + KPP, ...; per batch of CROSS_NB passes it loads the K and V rows
// together (addresses clamped to the last frame, so the batch is
// straight-line code), keeps a private online softmax, and the private states
// are merged once at the end (DPP within each 16-lane row, LDS across the 16
// rows) and written as the final output: no partials, no combine pass.
constexpr int CROSS_NB = 8;

// 16 bytes of a K or V row as fp32 (no address-taken register arrays)
__device__ __forceinline__ void unpack16(const uint4 w, float o[8]) {
  const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = __uint_as_float(a[i] << 16);
    o[2 * i + 1] = __uint_as_float(a[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void unpack16(const float4 w, float o[4]) {
  o[0] = w.x; o[1] = w.y; o[2] = w.z; o[3] = w.w;
}

template <typename T>
__global__ __launch_bounds__(256) void attn_decode_cross_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                                const T* __restrict__ v, int H, int T_,
                                                                T* __restrict__ out, int rows_per_b) {
  constexpr int EPT = 16 / sizeof(T);   // elements per 16-byte chunk
  constexpr int TPK = 64 / EPT;         // lanes per key row
  constexpr int KPP = 256 / TPK;        // keys per pass
  typedef typename std::conditional<sizeof(T) == 2, uint4, float4>::type V16;
  __shared__ __attribute__((aligned(16))) float red[16][64];
  __shared__ float rowmax[16], rsum[16];
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int part = tid % TPK, kg = tid / TPK;
  float qreg[EPT];
  {
    const T* qp = q + ((long)b * H + h) * 64 + part * EPT;
#pragma unroll
    for (int i = 0; i < EPT; ++i) qreg[i] = Act<T>::cvt(qp[i]) * (0.125f * LOG2E);  // scores in base-2 units
  }
  const long head = ((long)(b / rows_per_b) * H + h) * T_ * 64 + part * EPT;  // K/V of the query row's batch row
  const T* K = k + head;
  const T* V = v + head;
  float m = -INFINITY, l = 0.f, acc[EPT];
#pragma unroll
  for (int i = 0; i < EPT; ++i) acc[i] = 0.f;
  for (int base = 0; base < T_; base += KPP * CROSS_NB) {
    V16 ck[CROSS_NB], cv[CROSS_NB];
#pragma unroll
    for (int i = 0; i < CROSS_NB; ++i) {
      const long j = min(base + kg + KPP * i, T_ - 1);
      ck[i] = *(const V16*)(K + j * 64);
      cv[i] = *(const V16*)(V + j * 64);
    }
    __builtin_amdgcn_sched_barrier(0);
    float sj[CROSS_NB];
    float bm = -INFINITY;
#pragma unroll
    for (int i = 0; i < CROSS_NB; ++i) {
      float kk[EPT];
      unpack16(ck[i], kk);
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < EPT; ++e) d = fmaf(qreg[e], kk[e], d);
      if constexpr (TPK == 8) d = sum8_lanes(d);
      else if constexpr (TPK == 4) d = sum4_lanes(d);
      else {
#pragma unroll
        for (int o = 1; o < TPK; o <<= 1) d += __shfl_xor(d, o, 64);
      }
      sj[i] = (base + kg + KPP * i < T_) ? d : -INFINITY;
      bm = fmaxf(bm, sj[i]);
    }
    const float mn = fmaxf(m, bm);
    const float alpha = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - mn);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < EPT; ++e) acc[e] *= alpha;
#pragma unroll
    for (int i = 0; i < CROSS_NB; ++i) {
      const float p = (sj[i] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sj[i] - mn);
      l += p;
      float vv[EPT];
      unpack16(cv[i], vv);
#pragma unroll
      for (int e = 0; e < EPT; ++e) acc[e] = fmaf(p, vv[e], acc[e]);
    }
    m = mn;
  }
  // merge: each 16-lane row (16 / TPK key groups of TPK parts) takes its max
  // and its sums over key groups of equal part with DPP row rotations; the 16
  // rows of the block meet in LDS once, each output dim rescaling the rows'
  // sums to the block max as it adds them
  static_assert(TPK == 8 || TPK == 16, "a 16-lane row holds whole key groups");
  const int rrow = wave * 4 + (lane >> 4);
  float rm = m;
  rm = fmaxf(rm, dpp_f<0x128>(rm));  // row_ror:8
  rm = fmaxf(rm, dpp_f<0x124>(rm));  // row_ror:4
  rm = fmaxf(rm, dpp_f<0x122>(rm));  // row_ror:2
  rm = fmaxf(rm, dpp_f<0x121>(rm));  // row_ror:1
  const float f = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - rm);
  float ls = l * f;
#pragma unroll
  for (int e = 0; e < EPT; ++e) acc[e] *= f;
  if constexpr (TPK == 8) {
    ls += dpp_f<0x128>(ls);
#pragma unroll
    for (int e = 0; e < EPT; ++e) acc[e] += dpp_f<0x128>(acc[e]);
  }
  if ((lane & 15) < TPK) {
#pragma unroll
    for (int e = 0; e < EPT; e += 4)
      *(float4*)&red[rrow][part * EPT + e] = make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
    if ((lane & 15) == 0) {
      rsum[rrow] = ls;
      rowmax[rrow] = rm;
    }
  }
  __syncthreads();
  if (tid < 64) {
    float mx = rowmax[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, rowmax[r]);
    float sum = 0.f, sacc = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float w = rowmax[r] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(rowmax[r] - mx);
      sum = fmaf(rsum[r], w, sum);
      sacc = fmaf(red[r][tid], w, sacc);
    }
    out[((long)b * H + h) * 64 + tid] = Act<T>::st(T_ > 0 ? sacc / sum : 0.f);
  }
}

hipError_t launch_attn_decode_cross(ActType t, const void* q, const void* k, const void* v, int B, int H, int T,
                                    void* out, hipStream_t s, int rows_per_b) {
  if (T <= 0 || rows_per_b < 1 || B % rows_per_b) return hipErrorInvalidValue;
  const dim3 grid(H, B);
  if (t == ACT_BF16)
    hipLaunchKernelGGL(attn_decode_cross_kernel<u16>, grid, dim3(256), 0, s, (const u16*)q, (const u16*)k,
                       (const u16*)v, H, T, (u16*)out, rows_per_b);
  else
    hipLaunchKernelGGL(attn_decode_cross_kernel<float>, grid, dim3(256), 0, s, (const float*)q, (const float*)k,
                       (const float*)v, H, T, (float*)out, rows_per_b);
  return hipGetLastError();
}

}  // namespace wh
