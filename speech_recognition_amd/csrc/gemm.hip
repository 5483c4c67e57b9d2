// GEMMs of the hot path: C = epilogue(A . B^T + bias) with A [M,K] (rows may
// overlap for the implicit-GEMM convolutions) and B the weight in [N,K]
// layout, both K-contiguous. This is the projection GEMM of the whisper_blaze
// showcase page ("The Solution", gemm_hopper.cu card) rebuilt for gfx950:
// bf16 MFMA 16x16x32 tiles, LDS double buffering with an XOR swizzle, and a
// skinny variant for the decoder's batch-row GEMMs that streams each weight
// once. fp32 activations (the tiny fp32 config) take a plain SIMT kernel.
#include "common.hpp"
#include "internal.hpp"

namespace wh {

// ------------------------------------------------------------------ epilogues
template <typename T, int EPI>
__device__ __forceinline__ void epi_store(const GemmParams& p, int z, int m, int n, float acc) {
  if (m >= p.M || n >= p.N) return;
  float v = acc + (p.bias ? p.bias[n] : 0.0f);
  if constexpr (EPI == EPI_STORE) {
    ((T*)p.C)[(long)z * p.strideC + (long)m * p.ldc + n] = Act<T>::st(v);
  } else if constexpr (EPI == EPI_GELU) {
    ((T*)p.C)[(long)z * p.strideC + (long)m * p.ldc + n] = Act<T>::st(gelu_erf(v));
  } else if constexpr (EPI == EPI_GELU_PE) {
    ((float*)p.C)[(long)z * p.strideC + (long)m * p.ldc + n] = gelu_erf(v) + p.pe[(long)m * p.N + n];
  } else if constexpr (EPI == EPI_F32) {
    ((float*)p.C)[(long)z * p.strideC + (long)m * p.ldc + n] = v;
  } else if constexpr (EPI == EPI_CROSSKV) {
    const int d = p.ckv_d, T_ = p.ckv_T;
    const int b = m / T_, t = m - b * T_;
    const int l = n / (2 * d), r = n - l * 2 * d;
    const int kv = r / d, c = r - kv * d;
    const int h = c >> 6, e = c & 63;
    const long idx = ((((long)(l * 2 + kv) * p.ckv_B + b) * p.ckv_H + h) * T_ + t) * 64 + e;
    ((T*)p.C)[idx] = Act<T>::st(v);
  } else if constexpr (EPI == EPI_DEC_QKV) {
    const int d = p.d_model;
    if (n < d) {
      ((T*)p.C)[(long)m * d + n] = Act<T>::st(v);
    } else {
      const int kv = (n - d) / d, c = (n - d) - kv * d;
      const int h = c >> 6, e = c & 63;
      const int pos = p.lengths[m];
      if (pos >= 0 && pos < p.kv_cap) {
        const float inv = 1.0f / p.kv_scales[p.kv_layer * 2 + kv];
        const long idx = ((((long)(p.kv_layer * 2 + kv) * p.kv_B + m) * p.kv_H + h) * p.kv_cap + pos) * 64 + e;
        p.kv_cache[idx] = (uint8_t)e4m3_encode(v * inv);
      } else if (p.dev_error && n == d) {
        *p.dev_error = 6;  // capacity exceeded: the write is skipped
      }
    }
  }
}

// ------------------------------------------------------------------ bf16 MFMA, 128x128x64
constexpr int TB = 128, TK = 64;

__device__ __forceinline__ int swz(int row, int kc) { return row * TK + ((kc ^ (row & 7)) << 3); }

template <int EPI>
__global__ __launch_bounds__(256) void gemm_bf16_128(GemmParams p) {
  __shared__ __attribute__((aligned(16))) u16 sA[2][TB * TK];
  __shared__ __attribute__((aligned(16))) u16 sB[2][TB * TK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int tiles_n = (p.N + TB - 1) / TB;
  const int tiles_m = (p.M + TB - 1) / TB;
  // XCD-aware order: blocks are dispatched round-robin over 8 XCDs, so give
  // each XCD a contiguous run of tiles (neighbours share A rows in that L2).
  const int nblk = tiles_m * tiles_n;
  int bid = blockIdx.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int tm = bid / tiles_n, tn = bid - tm * tiles_n;
  const int z = blockIdx.z;
  const u16* A = (const u16*)p.A + (long)z * p.strideA;
  const u16* B = (const u16*)p.B;
  const int m0 = tm * TB, n0 = tn * TB;

  const u16* a_ptr[4];
  const u16* b_ptr[4];
  int lds_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + i * 256, row = c >> 3, kc = c & 7;
    const int ar = min(m0 + row, p.M - 1), br = min(n0 + row, p.N - 1);
    a_ptr[i] = A + (long)ar * p.lda + kc * 8;
    b_ptr[i] = B + (long)br * p.ldb + kc * 8;
    lds_off[i] = swz(row, kc);
  }
  uint4 ra[4], rb[4];
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = p.K / TK;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ra[i] = *(const uint4*)a_ptr[i];
    rb[i] = *(const uint4*)b_ptr[i];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    *(uint4*)&sA[0][lds_off[i]] = ra[i];
    *(uint4*)&sB[0][lds_off[i]] = rb[i];
  }
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ra[i] = *(const uint4*)(a_ptr[i] + (kt + 1) * TK);
        rb[i] = *(const uint4*)(b_ptr[i] + (kt + 1) * TK);
      }
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x8 af[4], bfr[4];
      const int kc = s * 4 + (lane >> 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        af[i] = bitcast<bf16x8>(*(const uint4*)&sA[cur][swz(wm * 64 + i * 16 + (lane & 15), kc)]);
        bfr[i] = bitcast<bf16x8>(*(const uint4*)&sB[cur][swz(wn * 64 + i * 16 + (lane & 15), kc)]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        *(uint4*)&sA[cur ^ 1][lds_off[i]] = ra[i];
        *(uint4*)&sB[cur ^ 1][lds_off[i]] = rb[i];
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * 64 + i * 16 + (lane >> 4) * 4 + r;
        const int n = n0 + wn * 64 + j * 16 + (lane & 15);
        epi_store<u16, EPI>(p, z, m, n, acc[i][j][r]);
      }
}

// ------------------------------------------------------------------ bf16 skinny (decode rows)
// One workgroup owns 16 output columns; its KS waves split K into contiguous
// ranges and stream that slice of the weight exactly once; the activation
// rows (<= 16*MB) are re-read from L2. Partials are summed through LDS.
template <int EPI, int MB, int KS>
__global__ __launch_bounds__(KS * 64) void gemm_bf16_skinny(GemmParams p) {
  __shared__ float red[KS][MB * 16][17];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * 16;
  const int kper = p.K / KS;
  const int kb = wave * kper;
  const int nrow = min(n0 + (lane & 15), p.N - 1);
  const u16* wp = (const u16*)p.B + (long)nrow * p.ldb + kb + (lane >> 4) * 8;
  const u16* ap[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int row = min(mb * 16 + (lane & 15), p.M - 1);
    ap[mb] = (const u16*)p.A + (long)row * p.lda + kb + (lane >> 4) * 8;
  }
  f32x4 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int k = 0; k < kper; k += 32) {
    const bf16x8 b = bitcast<bf16x8>(*(const uint4*)(wp + k));
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const bf16x8 a = bitcast<bf16x8>(*(const uint4*)(ap[mb] + k));
      acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[mb], 0, 0, 0);
    }
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][mb * 16 + (lane >> 4) * 4 + r][lane & 15] = acc[mb][r];
  __syncthreads();
  for (int o = tid; o < MB * 16 * 16; o += KS * 64) {
    const int m = o >> 4, c = o & 15;
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < KS; ++w) s += red[w][m][c];
    epi_store<u16, EPI>(p, 0, m, n0 + c, s);
  }
}

// ------------------------------------------------------------------ fp32 SIMT (tiny fp32 config)
template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_simt(GemmParams p) {
  __shared__ float sA[16][64 + 4];
  __shared__ float sB[16][64 + 4];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int tiles_n = (p.N + 63) / 64;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x - tm * tiles_n;
  const int z = blockIdx.z;
  const float* A = (const float*)p.A + (long)z * p.strideA;
  const float* B = (const float*)p.B;
  const int m0 = tm * 64, n0 = tn * 64;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < p.K; k0 += 16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = ty + 16 * i, kk = tx;
      const int m = m0 + row, n = n0 + row, k = k0 + kk;
      sA[kk][row] = (m < p.M && k < p.K) ? A[(long)m * p.lda + k] : 0.f;
      sB[kk][row] = (n < p.N && k < p.K) ? B[(long)n * p.ldb + k] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { a[i] = sA[kk][ty * 4 + i]; b[i] = sB[kk][tx * 4 + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) epi_store<float, EPI>(p, z, m0 + ty * 4 + i, n0 + tx * 4 + j, acc[i][j]);
}

// ------------------------------------------------------------------ launchers
#define WH_EPI_SWITCH(epi, CALL)                    \
  switch (epi) {                                    \
    case EPI_STORE: CALL(EPI_STORE); break;         \
    case EPI_GELU: CALL(EPI_GELU); break;           \
    case EPI_GELU_PE: CALL(EPI_GELU_PE); break;     \
    case EPI_F32: CALL(EPI_F32); break;             \
    case EPI_CROSSKV: CALL(EPI_CROSSKV); break;     \
    case EPI_DEC_QKV: CALL(EPI_DEC_QKV); break;     \
    default: return hipErrorInvalidValue;           \
  }

hipError_t launch_gemm(ActType t, Epi epi, const GemmParams& p, hipStream_t s) {
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
  if (t == ACT_BF16) {
    const int tiles = ((p.M + TB - 1) / TB) * ((p.N + TB - 1) / TB);
    dim3 grid(tiles, 1, p.batch);
#define CALL(E) hipLaunchKernelGGL(gemm_bf16_128<E>, grid, dim3(256), 0, s, p)
    WH_EPI_SWITCH(epi, CALL)
#undef CALL
  } else {
    const int tiles = ((p.M + 63) / 64) * ((p.N + 63) / 64);
    dim3 grid(tiles, 1, p.batch);
#define CALL(E) hipLaunchKernelGGL(gemm_f32_simt<E>, grid, dim3(256), 0, s, p)
    WH_EPI_SWITCH(epi, CALL)
#undef CALL
  }
  return hipGetLastError();
}

template <int EPI, int KS>
static void skinny_mb(const GemmParams& p, hipStream_t s) {
  dim3 grid((p.N + 15) / 16);
  const int mb = (p.M + 15) / 16;
  if (mb <= 1) hipLaunchKernelGGL((gemm_bf16_skinny<EPI, 1, KS>), grid, dim3(KS * 64), 0, s, p);
  else if (mb <= 2) hipLaunchKernelGGL((gemm_bf16_skinny<EPI, 2, KS>), grid, dim3(KS * 64), 0, s, p);
  else if (mb <= 4) hipLaunchKernelGGL((gemm_bf16_skinny<EPI, 4, KS>), grid, dim3(KS * 64), 0, s, p);
  else if (mb <= 6) hipLaunchKernelGGL((gemm_bf16_skinny<EPI, 6, KS>), grid, dim3(KS * 64), 0, s, p);
  else hipLaunchKernelGGL((gemm_bf16_skinny<EPI, 8, KS>), grid, dim3(KS * 64), 0, s, p);
}

template <int EPI>
static void skinny_ks(const GemmParams& p, hipStream_t s) {
  if (p.K % (32 * 8) == 0 && p.K >= 4096) skinny_mb<EPI, 8>(p, s);
  else skinny_mb<EPI, 4>(p, s);
}

hipError_t launch_gemm_skinny(ActType t, Epi epi, const GemmParams& p, hipStream_t s) {
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
  if (t != ACT_BF16 || p.M > 128 || p.batch != 1 || p.K % 128 != 0) return launch_gemm(t, epi, p, s);
  switch (epi) {
    case EPI_STORE: skinny_ks<EPI_STORE>(p, s); break;
    case EPI_GELU: skinny_ks<EPI_GELU>(p, s); break;
    case EPI_F32: skinny_ks<EPI_F32>(p, s); break;
    case EPI_DEC_QKV: skinny_ks<EPI_DEC_QKV>(p, s); break;
    default: return launch_gemm(t, epi, p, s);
  }
  return hipGetLastError();
}

}  // namespace wh
