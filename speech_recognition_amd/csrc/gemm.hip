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
// 256 threads = 2x2 waves, each wave a 64x64 sub-tile of 16x16x32 MFMAs with
// fp32 accumulators. A and B tiles (128 rows x 64 k) are staged through
// registers into double-buffered LDS. Rows are 128 B (8 chunks of 16 B); chunk
// c of row r is stored at c ^ ((r >> 1) & 7), so the 16 rows one MFMA fragment
// read touches (two rows per 256-byte bank line) land on distinct banks.
constexpr int TB = 128, TK = 64;

__device__ __forceinline__ int swz(int row, int kc) { return row * TK + ((kc ^ ((row >> 1) & 7)) << 3); }

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

  // this thread stages chunk (row r0 + 32 i, kc) of each tile, i = 0..3
  const int r0 = tid >> 3, kc0 = tid & 7;
  const long la = p.lda, lb = p.ldb;
  const u16* pa0 = A + (long)min(m0 + r0, p.M - 1) * la + kc0 * 8;
  const u16* pa1 = A + (long)min(m0 + r0 + 32, p.M - 1) * la + kc0 * 8;
  const u16* pa2 = A + (long)min(m0 + r0 + 64, p.M - 1) * la + kc0 * 8;
  const u16* pa3 = A + (long)min(m0 + r0 + 96, p.M - 1) * la + kc0 * 8;
  const u16* pb0 = B + (long)min(n0 + r0, p.N - 1) * lb + kc0 * 8;
  const u16* pb1 = B + (long)min(n0 + r0 + 32, p.N - 1) * lb + kc0 * 8;
  const u16* pb2 = B + (long)min(n0 + r0 + 64, p.N - 1) * lb + kc0 * 8;
  const u16* pb3 = B + (long)min(n0 + r0 + 96, p.N - 1) * lb + kc0 * 8;
  const int so = swz(r0, kc0);  // rows r0 + 32 i share the swizzle, so chunk i sits at so + 32*i*TK

  uint4 ga0, ga1, ga2, ga3, gb0, gb1, gb2, gb3;
#define WH_GLOAD(k)                                                                  \
  ga0 = *(const uint4*)(pa0 + (k)); ga1 = *(const uint4*)(pa1 + (k));                 \
  ga2 = *(const uint4*)(pa2 + (k)); ga3 = *(const uint4*)(pa3 + (k));                 \
  gb0 = *(const uint4*)(pb0 + (k)); gb1 = *(const uint4*)(pb1 + (k));                 \
  gb2 = *(const uint4*)(pb2 + (k)); gb3 = *(const uint4*)(pb3 + (k));
#define WH_SSTORE(buf)                                                               \
  *(uint4*)(&sA[buf][so]) = ga0; *(uint4*)(&sA[buf][so + 32 * TK]) = ga1;             \
  *(uint4*)(&sA[buf][so + 64 * TK]) = ga2; *(uint4*)(&sA[buf][so + 96 * TK]) = ga3;   \
  *(uint4*)(&sB[buf][so]) = gb0; *(uint4*)(&sB[buf][so + 32 * TK]) = gb1;             \
  *(uint4*)(&sB[buf][so + 64 * TK]) = gb2; *(uint4*)(&sB[buf][so + 96 * TK]) = gb3;

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = p.K / TK;
  WH_GLOAD(0)
  WH_SSTORE(0)
  __syncthreads();
  const int fr = lane & 15;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) { WH_GLOAD((kt + 1) * TK) }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int kc = s * 4 + (lane >> 4);
      bf16x8 af0 = bitcast<bf16x8>(*(const uint4*)&sA[cur][swz(wm * 64 + 0 + fr, kc)]);
      bf16x8 af1 = bitcast<bf16x8>(*(const uint4*)&sA[cur][swz(wm * 64 + 16 + fr, kc)]);
      bf16x8 af2 = bitcast<bf16x8>(*(const uint4*)&sA[cur][swz(wm * 64 + 32 + fr, kc)]);
      bf16x8 af3 = bitcast<bf16x8>(*(const uint4*)&sA[cur][swz(wm * 64 + 48 + fr, kc)]);
      bf16x8 bf0 = bitcast<bf16x8>(*(const uint4*)&sB[cur][swz(wn * 64 + 0 + fr, kc)]);
      bf16x8 bf1 = bitcast<bf16x8>(*(const uint4*)&sB[cur][swz(wn * 64 + 16 + fr, kc)]);
      bf16x8 bf2 = bitcast<bf16x8>(*(const uint4*)&sB[cur][swz(wn * 64 + 32 + fr, kc)]);
      bf16x8 bf3 = bitcast<bf16x8>(*(const uint4*)&sB[cur][swz(wn * 64 + 48 + fr, kc)]);
#define WH_MF(i, j, a, b) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[i][j], 0, 0, 0)
      WH_MF(0, 0, af0, bf0); WH_MF(0, 1, af0, bf1); WH_MF(0, 2, af0, bf2); WH_MF(0, 3, af0, bf3);
      WH_MF(1, 0, af1, bf0); WH_MF(1, 1, af1, bf1); WH_MF(1, 2, af1, bf2); WH_MF(1, 3, af1, bf3);
      WH_MF(2, 0, af2, bf0); WH_MF(2, 1, af2, bf1); WH_MF(2, 2, af2, bf2); WH_MF(2, 3, af2, bf3);
      WH_MF(3, 0, af3, bf0); WH_MF(3, 1, af3, bf1); WH_MF(3, 2, af3, bf2); WH_MF(3, 3, af3, bf3);
#undef WH_MF
    }
    if (more) { WH_SSTORE(cur ^ 1) }
    __syncthreads();
  }
#undef WH_GLOAD
#undef WH_SSTORE
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
// Decoder GEMMs have M = batch rows (<= 128) and stream their weight once, so
// they are bound by bytes in flight, not by MFMA. One workgroup owns 16*CB
// output columns; its WAVES waves split K into contiguous ranges, and each
// wave issues all loads of a batch of SKB k-steps (weights from HBM,
// activation rows from L2) before the MFMAs of that batch, so a whole
// (N/16*CB) x K weight slice is requested at once. Partials meet in LDS.
template <int EPI, int MB, int CB, int W>
__global__ __launch_bounds__(W * 64) void gemm_bf16_skinny(GemmParams p) {
  constexpr int SKB = MB >= 8 ? 3 : 5;  // k-steps whose loads are issued together
  constexpr int RW = CB * 16 + 1;
  __shared__ float red[W][MB * 16][RW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * 16 * CB;
  const int kper = p.K / W;
  const int kofs = wave * kper + (lane >> 4) * 8;
  const u16* wp[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int nrow = min(n0 + cb * 16 + (lane & 15), p.N - 1);
    wp[cb] = (const u16*)p.B + (long)nrow * p.ldb + kofs;
  }
  const u16* ap[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int row = min(mb * 16 + (lane & 15), p.M - 1);
    ap[mb] = (const u16*)p.A + (long)row * p.lda + kofs;
  }
  f32x4 acc[MB][CB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[mb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < kper; k0 += 32 * SKB) {
    uint4 wv[SKB][CB], av[SKB][MB];
#pragma unroll
    for (int j = 0; j < SKB; ++j) {
      const int k = k0 + j * 32;
      const bool ok = k < kper;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) wv[j][cb] = ok ? *(const uint4*)(wp[cb] + k) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) av[j][mb] = ok ? *(const uint4*)(ap[mb] + k) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < SKB; ++j)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
          acc[mb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8>(av[j][mb]), bitcast<bf16x8>(wv[j][cb]),
                                                                acc[mb][cb], 0, 0, 0);
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave][mb * 16 + (lane >> 4) * 4 + r][cb * 16 + (lane & 15)] = acc[mb][cb][r];
  __syncthreads();
  for (int o = tid; o < MB * 16 * CB * 16; o += W * 64) {
    const int m = o / (CB * 16), c = o - m * (CB * 16);
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) sum += red[w][m][c];
    epi_store<u16, EPI>(p, 0, m, n0 + c, sum);
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

template <int EPI, int CB, int W>
static void skinny_mb(const GemmParams& p, hipStream_t s) {
  dim3 grid((p.N + 16 * CB - 1) / (16 * CB)), block(W * 64);
  const int mb = (p.M + 15) / 16;
  if (mb <= 1) hipLaunchKernelGGL((gemm_bf16_skinny<EPI, 1, CB, W>), grid, block, 0, s, p);
  else if (mb <= 2) hipLaunchKernelGGL((gemm_bf16_skinny<EPI, 2, CB, W>), grid, block, 0, s, p);
  else if (mb <= 4) hipLaunchKernelGGL((gemm_bf16_skinny<EPI, 4, CB, W>), grid, block, 0, s, p);
  else if (mb <= 6) hipLaunchKernelGGL((gemm_bf16_skinny<EPI, 6, CB, W>), grid, block, 0, s, p);
  else hipLaunchKernelGGL((gemm_bf16_skinny<EPI, 8, CB, W>), grid, block, 0, s, p);
}

// K is split over 8 waves when it divides into 32-wide steps, else over 4.
template <int EPI, int CB>
static bool skinny_w(const GemmParams& p, hipStream_t s) {
  if (p.K % (32 * 8) == 0) { skinny_mb<EPI, CB, 8>(p, s); return true; }
  if (p.K % (32 * 4) == 0) { skinny_mb<EPI, CB, 4>(p, s); return true; }
  return false;
}

hipError_t launch_gemm_skinny(ActType t, Epi epi, const GemmParams& p, hipStream_t s) {
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
  if (t != ACT_BF16 || p.M > 128 || p.batch != 1) return launch_gemm(t, epi, p, s);
  bool ok = false;
  switch (epi) {
    case EPI_STORE: ok = skinny_w<EPI_STORE, 1>(p, s); break;
    case EPI_GELU: ok = skinny_w<EPI_GELU, 1>(p, s); break;
    case EPI_DEC_QKV: ok = skinny_w<EPI_DEC_QKV, 1>(p, s); break;
    // the vocabulary projection: two column blocks per wave halve activation re-reads
    case EPI_F32: ok = p.N >= 16384 ? skinny_w<EPI_F32, 2>(p, s) : skinny_w<EPI_F32, 1>(p, s); break;
    default: break;
  }
  if (!ok) return launch_gemm(t, epi, p, s);
  return hipGetLastError();
}

}  // namespace wh
