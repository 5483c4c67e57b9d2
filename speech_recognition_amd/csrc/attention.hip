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
// directly from registers; V is transposed once per tile on its way into LDS.
//
// Decoder self-attention reads the caller's e4m3 KV cache and dequantises on
// read (the Inference Endpoints post, "Inference Stack": K/V stored as float8,
// compute in bfloat16). Decoder cross-attention streams head-major bf16 K/V,
// split over the 1500 frames with a log-sum-exp combine.
#include "common.hpp"
#include "internal.hpp"

namespace wh {

// ------------------------------------------------------------------ encoder, bf16 MFMA
__device__ __forceinline__ int k_swz(int row, int kc) { return row * 64 + ((kc ^ (row & 7)) << 3); }
__device__ __forceinline__ int vt_swz(int e, int key) {
  return e * 64 + ((((key >> 2) ^ (e & 15))) << 2) + (key & 3);
}

__device__ __forceinline__ bf16x8 pack_bf16x8(float a0, float a1, float a2, float a3, float a4, float a5, float a6,
                                              float a7) {
  uint4 u;
  u.x = (uint32_t)f2bf(a0) | ((uint32_t)f2bf(a1) << 16);
  u.y = (uint32_t)f2bf(a2) | ((uint32_t)f2bf(a3) << 16);
  u.z = (uint32_t)f2bf(a4) | ((uint32_t)f2bf(a5) << 16);
  u.w = (uint32_t)f2bf(a6) | ((uint32_t)f2bf(a7) << 16);
  return bitcast<bf16x8>(u);
}

__global__ __launch_bounds__(256) void attn_encoder_bf16(const u16* __restrict__ qkv, int T, int H,
                                                         u16* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) u16 sK[2][64 * 64];
  __shared__ __attribute__((aligned(16))) u16 sVt[2][64 * 64];
  const int d = H * 64, ld = 3 * d;
  const int b = blockIdx.z, h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const u16* Qp = qkv + (long)b * T * ld + h * 64;
  const u16* Kp = Qp + d;
  const u16* Vp = Qp + 2 * d;
  const int q0 = blockIdx.x * 128 + wave * 32;
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
  auto vt_store = [&](int buf, const uint4 v, int key) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sVt[buf][vt_swz(kc * 8 + 2 * j, key)] = (u16)(w[j] & 0xffffu);
      sVt[buf][vt_swz(kc * 8 + 2 * j + 1, key)] = (u16)(w[j] >> 16);
    }
  };
  auto sstore = [&](int buf) {
    *(uint4*)&sK[buf][k_swz(row, kc)] = rk0;
    *(uint4*)&sK[buf][k_swz(row + 32, kc)] = rk1;
    vt_store(buf, rv0, row);
    vt_store(buf, rv1, row + 32);
  };

  f32x16 o[2];
#pragma unroll
  for (int e = 0; e < 2; ++e)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[e][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float c = 1.4426950408889634f * 0.125f;  // log2(e) / sqrt(64)
  const int nkb = (T + 63) / 64;

  gload(0);
  sstore(0);
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int cur = kb & 1;
    if (kb + 1 < nkb) gload(kb + 1);
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
    if (kb * 64 + 64 > T) {
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
    const float alpha = exp2f((m_run - m_new) * c);
    const float mc = m_new * c;
    float psum = 0.f;
#pragma unroll
    for (int j2 = 0; j2 < 2; ++j2)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = exp2f(fmaf(st[j2][i], c, -mc));
        st[j2][i] = p;
        psum += p;
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[e][i] *= alpha;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int j2 = t >> 1, hs = (t & 1) * 8;
      const bf16x8 pf = pack_bf16x8(st[j2][hs + 0], st[j2][hs + 1], st[j2][hs + 2], st[j2][hs + 3],
                                    st[j2][hs + 4], st[j2][hs + 5], st[j2][hs + 6], st[j2][hs + 7]);
#pragma unroll
      for (int eb = 0; eb < 2; ++eb) {
        const int e = eb * 32 + l32;
        const uint2 lo = *(const uint2*)&sVt[cur][vt_swz(e, t * 16 + g * 4)];
        const uint2 hi = *(const uint2*)&sVt[cur][vt_swz(e, t * 16 + 8 + g * 4)];
        const uint4 vv = make_uint4(lo.x, lo.y, hi.x, hi.y);
        o[eb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bitcast<bf16x8>(vv), pf, o[eb], 0, 0, 0);
      }
    }
    if (kb + 1 < nkb) sstore(cur ^ 1);
    __syncthreads();
  }
  const float l = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.0f / l;
  const int q = q0 + l32;
  if (q < T) {
    u16* op = out + ((long)b * T + q) * d + h * 64;
#pragma unroll
    for (int eb = 0; eb < 2; ++eb)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        uint2 u;
        u.x = (uint32_t)f2bf(o[eb][i4 * 4 + 0] * inv) | ((uint32_t)f2bf(o[eb][i4 * 4 + 1] * inv) << 16);
        u.y = (uint32_t)f2bf(o[eb][i4 * 4 + 2] * inv) | ((uint32_t)f2bf(o[eb][i4 * 4 + 3] * inv) << 16);
        *(uint2*)(op + eb * 32 + i4 * 8 + g * 4) = u;
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
    hipLaunchKernelGGL(attn_encoder_bf16, dim3((T + 127) / 128, H, B), dim3(256), 0, s, (const u16*)qkv, T, H,
                       (u16*)out);
  else
    hipLaunchKernelGGL(attn_encoder_f32, dim3((T + 63) / 64, H, B), dim3(64), 0, s, (const float*)qkv, T, H,
                       (float*)out);
  return hipGetLastError();
}

// ------------------------------------------------------------------ decoder self-attention over e4m3 codes
// One workgroup per (head, row). Keys 0..n-1 (n = lengths[b] + len_add) are
// 64-byte code rows read as 4 lanes x 16 codes. Each lane issues all of its
// loads of a batch (8 keys, 128 B) before decoding any of them, so a whole
// cache row of up to 512 keys is in flight at once; scores stay in LDS.
constexpr int DEC_MAX_CAP = 4096;
constexpr int SELF_BATCH = 8;

__device__ __forceinline__ float dot16_e4m3(const uint4 c, const float* q) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float v[4];
    e4m3x4_decode(w[i], v);
#pragma unroll
    for (int k = 0; k < 4; ++k) acc = fmaf(q[4 * i + k], v[k], acc);
  }
  return acc;
}

template <typename T>
__global__ __launch_bounds__(256) void attn_decode_self_kernel(const T* __restrict__ q, long q_stride,
                                                               const uint8_t* __restrict__ kc,
                                                               const uint8_t* __restrict__ vc,
                                                               const float* __restrict__ scales,
                                                               const int32_t* __restrict__ lengths, int len_add, int H,
                                                               int cap, T* __restrict__ out) {
  __shared__ float qs[64];
  __shared__ float sc[DEC_MAX_CAP];
  __shared__ float red[64][65];
  __shared__ float wred[8];
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int n = max(0, min(lengths[b] + len_add, cap));
  const float sk = scales[0], sv = scales[1];
  if (tid < 64) qs[tid] = Act<T>::cvt(q[(long)b * q_stride + h * 64 + tid]);
  __syncthreads();
  const long head = ((long)b * H + h) * cap * 64;
  const uint8_t* K = kc + head;
  const uint8_t* V = vc + head;
  const int part = tid & 3, kg = tid >> 2;
  float qreg[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) qreg[i] = qs[part * 16 + i];
  const float sscale = sk * 0.125f;
  for (int base = 0; base < n; base += 64 * SELF_BATCH) {
    uint4 c[SELF_BATCH];
#pragma unroll
    for (int i = 0; i < SELF_BATCH; ++i) {
      const int j = base + kg + 64 * i;
      c[i] = j < n ? *(const uint4*)(K + (long)j * 64 + part * 16) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < SELF_BATCH; ++i) {
      const int j = base + kg + 64 * i;
      float acc = dot16_e4m3(c[i], qreg);
      acc += __shfl_xor(acc, 1, 64);
      acc += __shfl_xor(acc, 2, 64);
      if (part == 0 && j < n) sc[j] = acc * sscale;
    }
  }
  __syncthreads();
  float mx = -INFINITY;
  for (int j = tid; j < n; j += 256) mx = fmaxf(mx, sc[j]);
  mx = wave_max(mx);
  if ((tid & 63) == 0) wred[tid >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(wred[0], wred[1]), fmaxf(wred[2], wred[3]));
  float sum = 0.f;
  for (int j = tid; j < n; j += 256) { const float p = expf(sc[j] - mx); sc[j] = p; sum += p; }
  sum = wave_sum(sum);
  if ((tid & 63) == 0) wred[4 + (tid >> 6)] = sum;
  __syncthreads();
  sum = wred[4] + wred[5] + wred[6] + wred[7];
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  for (int base = 0; base < n; base += 64 * SELF_BATCH) {
    uint4 c[SELF_BATCH];
#pragma unroll
    for (int i = 0; i < SELF_BATCH; ++i) {
      const int j = base + kg + 64 * i;
      c[i] = j < n ? *(const uint4*)(V + (long)j * 64 + part * 16) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < SELF_BATCH; ++i) {
      const int j = base + kg + 64 * i;
      const float p = j < n ? sc[j] : 0.f;
      const uint32_t w[4] = {c[i].x, c[i].y, c[i].z, c[i].w};
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        float v[4];
        e4m3x4_decode(w[e4], v);
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[4 * e4 + k] = fmaf(p, v[k], acc[4 * e4 + k]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) red[kg][part * 16 + i] = acc[i];
  __syncthreads();
  if (tid < 64) {
    float s = 0.f;
    for (int r = 0; r < 64; ++r) s += red[r][tid];
    const float v = (n > 0) ? s * sv / sum : 0.f;
    out[(long)b * H * 64 + h * 64 + tid] = Act<T>::st(v);
  }
}

hipError_t launch_attn_decode_self(ActType t, const void* q, long q_stride, const uint8_t* k_codes,
                                   const uint8_t* v_codes, const float* scales, const int32_t* lengths, int len_add,
                                   int B, int H, int cap, void* out, hipStream_t s) {
  if (cap > DEC_MAX_CAP) return hipErrorInvalidValue;
  dim3 grid(H, B);
  if (t == ACT_BF16)
    hipLaunchKernelGGL(attn_decode_self_kernel<u16>, grid, dim3(256), 0, s, (const u16*)q, q_stride, k_codes,
                       v_codes, scales, lengths, len_add, H, cap, (u16*)out);
  else
    hipLaunchKernelGGL(attn_decode_self_kernel<float>, grid, dim3(256), 0, s, (const float*)q, q_stride, k_codes,
                       v_codes, scales, lengths, len_add, H, cap, (float*)out);
  return hipGetLastError();
}

// ------------------------------------------------------------------ decoder cross-attention
// Grid (split, head, row). Each split handles a contiguous range of frames,
// keeps its scores in LDS and writes an unnormalised partial output with its
// local max and sum; the combine kernel merges the splits.
constexpr int CROSS_SPLIT = 4;
constexpr int CROSS_MAX_CHUNK = 1024;

size_t attn_decode_cross_ws(int B, int H, int T) { return (size_t)B * H * CROSS_SPLIT * 66 * sizeof(float); }

template <typename T>
__global__ __launch_bounds__(256) void attn_decode_cross_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                                const T* __restrict__ v, int H, int T_,
                                                                float* __restrict__ ws) {
  constexpr int EPT = 16 / sizeof(T);   // elements per 16-byte chunk
  constexpr int TPK = 64 / EPT;         // threads per key row
  constexpr int KPP = 256 / TPK;        // keys per pass
  __shared__ float qs[64];
  __shared__ float sc[CROSS_MAX_CHUNK];
  __shared__ float red[KPP][65];
  __shared__ float wred[8];
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int chunk = (T_ + CROSS_SPLIT - 1) / CROSS_SPLIT;
  const int t0 = split * chunk, t1 = min(T_, t0 + chunk), n = max(0, t1 - t0);
  if (tid < 64) qs[tid] = Act<T>::cvt(q[((long)b * H + h) * 64 + tid]);
  __syncthreads();
  const long head = (((long)b * H + h) * T_ + t0) * 64;
  const T* K = k + head;
  const T* V = v + head;
  const int part = tid % TPK, kg = tid / TPK;
  float qreg[EPT];
#pragma unroll
  for (int i = 0; i < EPT; ++i) qreg[i] = qs[part * EPT + i];
#pragma unroll 4
  for (int j = kg; j < n; j += KPP) {
    const uint4 c = *(const uint4*)(K + (long)j * 64 + part * EPT);
    const T* e = (const T*)&c;
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < EPT; ++i) acc = fmaf(qreg[i], Act<T>::cvt(e[i]), acc);
#pragma unroll
    for (int o = 1; o < TPK; o <<= 1) acc += __shfl_xor(acc, o, 64);
    if (part == 0) sc[j] = acc * 0.125f;
  }
  __syncthreads();
  float mx = -INFINITY;
  for (int j = tid; j < n; j += 256) mx = fmaxf(mx, sc[j]);
  mx = wave_max(mx);
  if ((tid & 63) == 0) wred[tid >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(wred[0], wred[1]), fmaxf(wred[2], wred[3]));
  float sum = 0.f;
  for (int j = tid; j < n; j += 256) { const float p = expf(sc[j] - mx); sc[j] = p; sum += p; }
  sum = wave_sum(sum);
  __syncthreads();
  if ((tid & 63) == 0) wred[4 + (tid >> 6)] = sum;
  __syncthreads();
  sum = wred[4] + wred[5] + wred[6] + wred[7];
  float acc[EPT];
#pragma unroll
  for (int i = 0; i < EPT; ++i) acc[i] = 0.f;
#pragma unroll 4
  for (int j = kg; j < n; j += KPP) {
    const uint4 c = *(const uint4*)(V + (long)j * 64 + part * EPT);
    const T* e = (const T*)&c;
    const float p = sc[j];
#pragma unroll
    for (int i = 0; i < EPT; ++i) acc[i] = fmaf(p, Act<T>::cvt(e[i]), acc[i]);
  }
#pragma unroll
  for (int i = 0; i < EPT; ++i) red[kg][part * EPT + i] = acc[i];
  __syncthreads();
  float* w = ws + (((long)b * H + h) * CROSS_SPLIT + split) * 66;
  if (tid < 64) {
    float s = 0.f;
    for (int r = 0; r < KPP; ++r) s += red[r][tid];
    w[tid] = s;
  }
  if (tid == 0) { w[64] = (n > 0) ? mx : -INFINITY; w[65] = (n > 0) ? sum : 0.f; }
}

template <typename T>
__global__ __launch_bounds__(64) void attn_decode_cross_combine(const float* __restrict__ ws, int H,
                                                                T* __restrict__ out) {
  const int h = blockIdx.x, b = blockIdx.y, e = threadIdx.x;
  const float* w = ws + ((long)b * H + h) * CROSS_SPLIT * 66;
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < CROSS_SPLIT; ++s) M = fmaxf(M, w[s * 66 + 64]);
  float num = 0.f, den = 0.f;
#pragma unroll
  for (int s = 0; s < CROSS_SPLIT; ++s) {
    const float ms = w[s * 66 + 64];
    const float f = (ms == -INFINITY) ? 0.f : expf(ms - M);
    num += w[s * 66 + e] * f;
    den += w[s * 66 + 65] * f;
  }
  out[((long)b * H + h) * 64 + e] = Act<T>::st(num / den);
}

hipError_t launch_attn_decode_cross_partial(ActType t, const void* q, const void* k, const void* v, int B, int H,
                                            int T, float* ws, hipStream_t s) {
  if ((T + CROSS_SPLIT - 1) / CROSS_SPLIT > CROSS_MAX_CHUNK) return hipErrorInvalidValue;
  dim3 grid(CROSS_SPLIT, H, B);
  if (t == ACT_BF16)
    hipLaunchKernelGGL(attn_decode_cross_kernel<u16>, grid, dim3(256), 0, s, (const u16*)q, (const u16*)k,
                       (const u16*)v, H, T, ws);
  else
    hipLaunchKernelGGL(attn_decode_cross_kernel<float>, grid, dim3(256), 0, s, (const float*)q, (const float*)k,
                       (const float*)v, H, T, ws);
  return hipGetLastError();
}

hipError_t launch_attn_decode_cross_combine(ActType t, const float* ws, int B, int H, void* out, hipStream_t s) {
  if (t == ACT_BF16)
    hipLaunchKernelGGL(attn_decode_cross_combine<u16>, dim3(H, B), dim3(64), 0, s, ws, H, (u16*)out);
  else
    hipLaunchKernelGGL(attn_decode_cross_combine<float>, dim3(H, B), dim3(64), 0, s, ws, H, (float*)out);
  return hipGetLastError();
}

hipError_t launch_attn_decode_cross(ActType t, const void* q, const void* k, const void* v, int B, int H, int T,
                                    void* out, float* ws, hipStream_t s) {
  hipError_t e = launch_attn_decode_cross_partial(t, q, k, v, B, H, T, ws, s);
  if (e != hipSuccess) return e;
  return launch_attn_decode_cross_combine(t, ws, B, H, out, s);
}

}  // namespace wh
