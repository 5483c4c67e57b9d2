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
      const long dbg = ((long)(p.kv_layer * 2 + kv) * p.M + m) * d + c;
      if (p.kv_pre) p.kv_pre[dbg] = v;
      if (pos >= 0 && pos < p.kv_cap) {
        const float inv = 1.0f / p.kv_scales[p.kv_layer * 2 + kv];
        const long idx = ((((long)(p.kv_layer * 2 + kv) * p.kv_B + m) * p.kv_H + h) * p.kv_cap + pos) * 64 + e;
        uint32_t code = e4m3_encode(v * inv);
        if (p.kv_force && p.kv_force[dbg] >= 0) code = (uint32_t)p.kv_force[dbg];
        p.kv_cache[idx] = (uint8_t)code;
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

// ------------------------------------------------------------------ bf16 MFMA, 256x256x64
// Large-M variant (the encoder projections, conv stem and cross K/V): 512
// threads = 2x4 waves, each wave a 128x64 sub-tile (8x4 MFMA 16x16x32 tiles,
// 128 fp32 accumulators), so each fragment read from LDS feeds twice as many
// MFMAs as in the 64x64 sub-tile. 2 x (32 KB A + 32 KB B) of LDS per block;
// same row swizzle and XCD-aware tile order as above.
constexpr int TB2 = 256;

template <int EPI>
__global__ __launch_bounds__(512) void gemm_bf16_256(GemmParams p) {
  __shared__ __attribute__((aligned(16))) u16 sA[2][TB2 * TK];
  __shared__ __attribute__((aligned(16))) u16 sB[2][TB2 * TK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int tiles_n = (p.N + TB2 - 1) / TB2;
  const int tiles_m = (p.M + TB2 - 1) / TB2;
  const int nblk = tiles_m * tiles_n;
  int bid = blockIdx.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int tm = bid / tiles_n, tn = bid - tm * tiles_n;
  const int z = blockIdx.z;
  const u16* A = (const u16*)p.A + (long)z * p.strideA;
  const u16* B = (const u16*)p.B;
  const int m0 = tm * TB2, n0 = tn * TB2;

  // this thread stages chunk (row r0 + 64 i, kc0) of each tile, i = 0..3
  const int r0 = tid >> 3, kc0 = tid & 7;
  const long la = p.lda, lb = p.ldb;
  const u16* pa0 = A + (long)min(m0 + r0, p.M - 1) * la + kc0 * 8;
  const u16* pa1 = A + (long)min(m0 + r0 + 64, p.M - 1) * la + kc0 * 8;
  const u16* pa2 = A + (long)min(m0 + r0 + 128, p.M - 1) * la + kc0 * 8;
  const u16* pa3 = A + (long)min(m0 + r0 + 192, p.M - 1) * la + kc0 * 8;
  const u16* pb0 = B + (long)min(n0 + r0, p.N - 1) * lb + kc0 * 8;
  const u16* pb1 = B + (long)min(n0 + r0 + 64, p.N - 1) * lb + kc0 * 8;
  const u16* pb2 = B + (long)min(n0 + r0 + 128, p.N - 1) * lb + kc0 * 8;
  const u16* pb3 = B + (long)min(n0 + r0 + 192, p.N - 1) * lb + kc0 * 8;
  const int so = swz(r0, kc0);  // rows r0 + 64 i share the swizzle

  uint4 ga0, ga1, ga2, ga3, gb0, gb1, gb2, gb3;
#define WH_GLOAD(k)                                                                  \
  ga0 = *(const uint4*)(pa0 + (k)); ga1 = *(const uint4*)(pa1 + (k));                 \
  ga2 = *(const uint4*)(pa2 + (k)); ga3 = *(const uint4*)(pa3 + (k));                 \
  gb0 = *(const uint4*)(pb0 + (k)); gb1 = *(const uint4*)(pb1 + (k));                 \
  gb2 = *(const uint4*)(pb2 + (k)); gb3 = *(const uint4*)(pb3 + (k));
#define WH_SSTORE(buf)                                                                 \
  *(uint4*)(&sA[buf][so]) = ga0; *(uint4*)(&sA[buf][so + 64 * TK]) = ga1;               \
  *(uint4*)(&sA[buf][so + 128 * TK]) = ga2; *(uint4*)(&sA[buf][so + 192 * TK]) = ga3;   \
  *(uint4*)(&sB[buf][so]) = gb0; *(uint4*)(&sB[buf][so + 64 * TK]) = gb1;               \
  *(uint4*)(&sB[buf][so + 128 * TK]) = gb2; *(uint4*)(&sB[buf][so + 192 * TK]) = gb3;

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
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
      bf16x8 bf[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) bf[j] = bitcast<bf16x8>(*(const uint4*)&sB[cur][swz(wn * 64 + j * 16 + fr, kc)]);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bf16x8 af = bitcast<bf16x8>(*(const uint4*)&sA[cur][swz(wm * 128 + i * 16 + fr, kc)]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[j], acc[i][j], 0, 0, 0);
      }
    }
    if (more) { WH_SSTORE(cur ^ 1) }
    __syncthreads();
  }
#undef WH_GLOAD
#undef WH_SSTORE
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * 128 + i * 16 + (lane >> 4) * 4 + r;
        const int n = n0 + wn * 64 + j * 16 + (lane & 15);
        epi_store<u16, EPI>(p, z, m, n, acc[i][j][r]);
      }
}

// ------------------------------------------------------------------ vectorised epilogue
// Eight consecutive columns n..n+7 of row m (n % 8 == 0, all < N) in one go:
// bias read as two float4, one 16-byte store for bf16 outputs.
template <int EPI>
__device__ __forceinline__ void epi_store8(const GemmParams& p, int z, int m, int n, float v[8]) {
  if (p.bias) {
    const float4 b0 = *(const float4*)(p.bias + n), b1 = *(const float4*)(p.bias + n + 4);
    v[0] += b0.x; v[1] += b0.y; v[2] += b0.z; v[3] += b0.w;
    v[4] += b1.x; v[5] += b1.y; v[6] += b1.z; v[7] += b1.w;
  }
  if constexpr (EPI == EPI_GELU || EPI == EPI_GELU_PE) {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = gelu_erf(v[i]);
  }
  if constexpr (EPI == EPI_GELU_PE) {
    const float* pe = p.pe + (long)m * p.N + n;
    const float4 q0 = *(const float4*)pe, q1 = *(const float4*)(pe + 4);
    float* c = (float*)p.C + (long)z * p.strideC + (long)m * p.ldc + n;
    *(float4*)c = make_float4(v[0] + q0.x, v[1] + q0.y, v[2] + q0.z, v[3] + q0.w);
    *(float4*)(c + 4) = make_float4(v[4] + q1.x, v[5] + q1.y, v[6] + q1.z, v[7] + q1.w);
    return;
  }
  uint4 u;
  u.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
  u.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
  u.z = (uint32_t)f2bf(v[4]) | ((uint32_t)f2bf(v[5]) << 16);
  u.w = (uint32_t)f2bf(v[6]) | ((uint32_t)f2bf(v[7]) << 16);
  if constexpr (EPI == EPI_CROSSKV) {
    const int d = p.ckv_d, T_ = p.ckv_T;
    const int b = m / T_, t = m - b * T_;
    const int l = n / (2 * d), r = n - l * 2 * d;
    const int kv = r / d, c = r - kv * d;
    const long idx = ((((long)(l * 2 + kv) * p.ckv_B + b) * p.ckv_H + (c >> 6)) * T_ + t) * 64 + (c & 63);
    *(uint4*)((u16*)p.C + idx) = u;
  } else {
    *(uint4*)((u16*)p.C + (long)z * p.strideC + (long)m * p.ldc + n) = u;
  }
}

// Four consecutive columns n..n+3 of row m (n % 4 == 0, all < N): bias as one
// float4, one 8-byte store for bf16 outputs (16 bytes for the fp32 stream).
template <int EPI>
__device__ __forceinline__ void epi_store4(const GemmParams& p, int z, int m, int n, float v[4]) {
  if (p.bias) {
    const float4 b = *(const float4*)(p.bias + n);
    v[0] += b.x; v[1] += b.y; v[2] += b.z; v[3] += b.w;
  }
  if constexpr (EPI == EPI_GELU || EPI == EPI_GELU_PE) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = gelu_erf(v[i]);
  }
  if constexpr (EPI == EPI_GELU_PE) {
    const float4 q = *(const float4*)(p.pe + (long)m * p.N + n);
    *(float4*)((float*)p.C + (long)z * p.strideC + (long)m * p.ldc + n) =
        make_float4(v[0] + q.x, v[1] + q.y, v[2] + q.z, v[3] + q.w);
    return;
  }
  uint2 u;
  u.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
  u.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
  if constexpr (EPI == EPI_CROSSKV) {
    const int d = p.ckv_d, T_ = p.ckv_T;
    const int b = m / T_, t = m - b * T_;
    const int l = n / (2 * d), r = n - l * 2 * d;
    const int kv = r / d, c = r - kv * d;
    const long idx = ((((long)(l * 2 + kv) * p.ckv_B + b) * p.ckv_H + (c >> 6)) * T_ + t) * 64 + (c & 63);
    *(uint2*)((u16*)p.C + idx) = u;
  } else {
    *(uint2*)((u16*)p.C + (long)z * p.strideC + (long)m * p.ldc + n) = u;
  }
}

// ------------------------------------------------------------------ bf16 MFMA, 256x256x64, 4 waves
// 256 threads = 2x2 waves, each wave a 128x128 sub-tile (8x8 MFMA 16x16x32
// tiles, 256 fp32 accumulators held in AGPRs), one wave per SIMD: per MFMA,
// half the LDS fragment bytes of the 64x64 sub-tile. The accumulators leave
// through LDS (bias/activation applied, packed to bf16) so C is written with
// 16-byte row-contiguous stores.
template <int EPI>
__global__ __launch_bounds__(256) void gemm_bf16_256w4(GemmParams p) {
  __shared__ __attribute__((aligned(16))) u16 smem[2 * 2 * TB2 * TK];  // [buf][A|B][256][64]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int tiles_n = (p.N + TB2 - 1) / TB2;
  const int tiles_m = (p.M + TB2 - 1) / TB2;
  const int nblk = tiles_m * tiles_n;
  int bid = blockIdx.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int tm = bid / tiles_n, tn = bid - tm * tiles_n;
  const int z = blockIdx.z;
  const u16* A = (const u16*)p.A + (long)z * p.strideA;
  const u16* B = (const u16*)p.B;
  const int m0 = tm * TB2, n0 = tn * TB2;
  u16* sA0 = smem;
  u16* sB0 = smem + TB2 * TK;
  constexpr int BUF = 2 * TB2 * TK;

  // staging: rows r0 + 32 i (i = 0..7) of A and of B, chunk kc0
  const int r0 = tid >> 3, kc0 = tid & 7;
  const long la = p.lda, lb = p.ldb;
  const u16* pa = A + (long)min(m0 + r0, p.M - 1) * la + kc0 * 8;
  const u16* pb = B + (long)min(n0 + r0, p.N - 1) * lb + kc0 * 8;
  long oa[8], ob[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    oa[i] = ((long)min(m0 + r0 + 32 * i, p.M - 1) - min(m0 + r0, p.M - 1)) * la;
    ob[i] = ((long)min(n0 + r0 + 32 * i, p.N - 1) - min(n0 + r0, p.N - 1)) * lb;
  }
  const int so = swz(r0, kc0);
  uint4 ga[8], gb[8];

  f32x4 acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = p.K / TK;
#pragma unroll
  for (int i = 0; i < 8; ++i) { ga[i] = *(const uint4*)(pa + oa[i]); gb[i] = *(const uint4*)(pb + ob[i]); }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    *(uint4*)(sA0 + so + 32 * i * TK) = ga[i];
    *(uint4*)(sB0 + so + 32 * i * TK) = gb[i];
  }
  __syncthreads();
  const int fr = lane & 15;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    // next tile (the last iteration re-reads the last tile: in bounds, unused)
    const int kn = min(kt + 1, nk - 1) * TK;
#pragma unroll
    for (int i = 0; i < 8; ++i) { ga[i] = *(const uint4*)(pa + oa[i] + kn); gb[i] = *(const uint4*)(pb + ob[i] + kn); }
    const u16* cA = sA0 + cur * BUF;
    const u16* cB = sB0 + cur * BUF;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int kc = s * 4 + (lane >> 4);
      bf16x8 bf[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) bf[j] = bitcast<bf16x8>(*(const uint4*)(cB + swz(wn * 128 + j * 16 + fr, kc)));
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bf16x8 af = bitcast<bf16x8>(*(const uint4*)(cA + swz(wm * 128 + i * 16 + fr, kc)));
#pragma unroll
        for (int j = 0; j < 8; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[j], acc[i][j], 0, 0, 0);
      }
    }
    u16* nA = sA0 + (cur ^ 1) * BUF;
    u16* nB = sB0 + (cur ^ 1) * BUF;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      *(uint4*)(nA + so + 32 * i * TK) = ga[i];
      *(uint4*)(nB + so + 32 * i * TK) = gb[i];
    }
    __syncthreads();
  }
  // epilogue: each wave parks its fp32 128x128 sub-tile in LDS in two 64-row
  // halves (32 KB each), then reads 8 consecutive columns per lane
  float* wbuf = (float*)smem + wave * (64 * 128);
  constexpr int WR = 128;  // row stride in floats
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    __syncthreads();
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = ii * 16 + (lane >> 4) * 4 + r;
          const int col = j * 16 + (lane & 15);
          wbuf[row * WR + (col ^ ((row & 7) << 2))] = acc[h * 4 + ii][j][r];
        }
    __syncthreads();
#pragma unroll 4
    for (int it = 0; it < 16; ++it) {
      const int c8 = it * 64 + lane;   // 64 rows x 16 eight-column chunks
      const int row = c8 >> 4, col = (c8 & 15) * 8;
      const int m = m0 + wm * 128 + h * 64 + row;
      const int n = n0 + wn * 128 + col;
      float v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = wbuf[row * WR + ((col + q) ^ ((row & 7) << 2))];
      if (m < p.M) {
        if (n + 8 <= p.N) {
          epi_store8<EPI>(p, z, m, n, v);
        } else {
#pragma unroll
          for (int q = 0; q < 8; ++q) epi_store<u16, EPI>(p, z, m, n + q, v[q]);
        }
      }
    }
  }
}

// ------------------------------------------------------------------ bf16 MFMA, 256x256, LDS DMA pipeline
// The encoder / cross-K/V GEMM at full size. Measured on the register-staged
// kernels: no LDS bank conflicts and LDS only ~17% busy, but waves spent ~45%
// of their time waiting for the next tile's global loads. Here tiles flow
// through a 4-stage LDS ring (BK = 32, 32 KB per stage) filled by direct
// global->LDS loads (16 bytes per lane, no staging registers) issued three
// stages ahead, with one barrier per stage. 512 threads = 2x4 waves of 128x64
// sub-tiles (8x4 MFMA 16x16x32). Each 1 KB DMA block is 16 rows x 64 bytes;
// lane L fills row L/4, slot L%4 with global chunk (L%4) ^ ((L/8)%4), the
// swizzle of dswz() below, so fragment reads are free of bank conflicts.
// The stages are separate LDS objects so the compiler's wait insertion can
// tell a stage being read from the stages being filled.
constexpr int DBK = 32;

// Tile order for the large kernels. Blocks are dispatched round-robin over
// the 8 XCDs, so XCD x runs blocks x, x+8, ...: each XCD gets a contiguous
// run of logical tiles (tile-columns fastest), so tiles running together on
// one XCD share A row-panels in its L2. (Grouping 8 tile-columns with
// tile-rows fastest measured no better at these shapes.)
__device__ __forceinline__ void tile_order(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int nblk = tiles_m * tiles_n;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  tm = bid / tiles_n;
  tn = bid - tm * tiles_n;
}

// Grouped order: each XCD walks a group of GN tile-columns down the tile-rows
// before moving to the next group, so the GN weight panels it reads stay in
// its L2 (the whole weight, 3-13 MB, does not fit in one XCD's 4 MB) while
// the activation panels stream past once per group.
template <int GN>
__device__ __forceinline__ void tile_order_grouped(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int nblk = tiles_m * tiles_n;
  if ((nblk & 7) != 0) { tile_order(bid, tiles_m, tiles_n, tm, tn); return; }
  const int t = (bid & 7) * (nblk >> 3) + (bid >> 3);  // contiguous logical range per XCD, as above
  const int gsz = GN * tiles_m;                         // tiles per full column group
  const int grp = t / gsz, r = t - grp * gsz;
  const int gn = min(GN, tiles_n - grp * GN);           // width of this (possibly last, narrower) group
  tm = r / gn;
  tn = grp * GN + (r - tm * gn);
}
constexpr int DSTAGE = 2 * TB2 * DBK;  // u16 elements per stage (A then B)

// LDS serves a 16-byte-per-lane read in groups of 8 lanes over a 128-byte
// bank window (32 banks), so the 8 rows one group reads (64 B apart: two per
// window) must land on 8 distinct 16-byte slots: chunk kc of row r is stored
// at slot kc ^ ((r >> 1) & 3).
__device__ __forceinline__ int dswz(int row, int kc) { return row * DBK + ((kc ^ ((row >> 1) & 3)) << 3); }

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] at [15:14])
#define WH_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))
// the same, and lgkmcnt(0): this wave's LDS reads have completed
#define WH_WAIT_VM_LGKM0(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4))

// One 16-byte-per-lane direct global->LDS load into the 1 KB block at LDS
// byte offset `lds` (wave-uniform): M0 holds the LDS base; one wait state is
// required between writing M0 and the LDS-DMA load. Issued as inline assembly
// so that the compiler's wait insertion leaves the ring's counting to us.
typedef __attribute__((address_space(3))) u16* lds_u16_ptr;
__device__ __forceinline__ uint32_t lds_addr(const u16* p) { return (uint32_t)(uintptr_t)(lds_u16_ptr)(p); }
__device__ __forceinline__ void dma16(const u16* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(g) : "memory", "m0");
}

template <int EPI, int ORDER>
__global__ __launch_bounds__(512) void gemm_bf16_dma(GemmParams p) {
  __shared__ __attribute__((aligned(1024))) u16 st0[DSTAGE];
  __shared__ __attribute__((aligned(1024))) u16 st1[DSTAGE];
  __shared__ __attribute__((aligned(1024))) u16 st2[DSTAGE];
  __shared__ __attribute__((aligned(1024))) u16 st3[DSTAGE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int tiles_n = (p.N + TB2 - 1) / TB2;
  const int tiles_m = (p.M + TB2 - 1) / TB2;
  int tm, tn;
  if constexpr (ORDER == 1) tile_order_grouped<4>(blockIdx.x, tiles_m, tiles_n, tm, tn);
  else tile_order(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int z = blockIdx.z;
  const u16* A = (const u16*)p.A + (long)z * p.strideA;
  const u16* B = (const u16*)p.B;
  const int m0 = tm * TB2, n0 = tn * TB2;

  // DMA: wave w fills A blocks w, w+8 and B blocks w, w+8 (16 rows each)
  const int lr = lane >> 2, lc = (lane & 3) ^ ((lane >> 3) & 3);  // global chunk for LDS slot lane & 3 of row lr
  const u16* ga0 = A + (long)min(m0 + wave * 16 + lr, p.M - 1) * p.lda + lc * 8;
  const u16* ga1 = A + (long)min(m0 + (wave + 8) * 16 + lr, p.M - 1) * p.lda + lc * 8;
  const u16* gb0 = B + (long)min(n0 + wave * 16 + lr, p.N - 1) * p.ldb + lc * 8;
  const u16* gb1 = B + (long)min(n0 + (wave + 8) * 16 + lr, p.N - 1) * p.ldb + lc * 8;
  const int la0 = wave * 16 * DBK, la1 = (wave + 8) * 16 * DBK;
  const int lb0 = TB2 * DBK + wave * 16 * DBK, lb1 = TB2 * DBK + (wave + 8) * 16 * DBK;
#define WH_ISSUE(S, k)                                                                         \
  dma16(ga0 + (k), __builtin_amdgcn_readfirstlane(lds_addr((S) + la0)));                        \
  dma16(ga1 + (k), __builtin_amdgcn_readfirstlane(lds_addr((S) + la1)));                        \
  dma16(gb0 + (k), __builtin_amdgcn_readfirstlane(lds_addr((S) + lb0)));                        \
  dma16(gb1 + (k), __builtin_amdgcn_readfirstlane(lds_addr((S) + lb1)));

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int fr = lane & 15, kc = lane >> 4;
  const int nk = p.K / DBK;
  // fragment registers, two sets: stage t+1's fragments are read while stage
  // t's MFMAs run from the other set
  bf16x8 a0[8], b0[4], a1[8], b1[4];
#define WH_READ(S, AF, BF)                                                                    \
  _Pragma("unroll") for (int j = 0; j < 4; ++j)                                               \
    BF[j] = bitcast<bf16x8>(*(const uint4*)((S) + TB2 * DBK + dswz(wn * 64 + j * 16 + fr, kc))); \
  _Pragma("unroll") for (int i = 0; i < 8; ++i)                                               \
    AF[i] = bitcast<bf16x8>(*(const uint4*)((S) + dswz(wm * 128 + i * 16 + fr, kc)));
#define WH_MFMA(AF, BF)                                                                       \
  _Pragma("unroll") for (int i = 0; i < 8; ++i)                                               \
    _Pragma("unroll") for (int j = 0; j < 4; ++j)                                             \
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(BF[j], AF[i], acc[i][j], 0, 0, 0);
  // Straight-line pipeline (K % 128 == 0): every wait is static, so the
  // compiler keeps the two fragment sets in place and waits for LDS reads
  // only where their registers are used. WH_SYNC(n): this wave's DMA loads of
  // the stage being waited for have landed (n later loads may still be in
  // flight) and its LDS reads are complete, then all waves meet.
#define WH_SYNC(n)                                                                             \
  {                                                                                            \
    WH_WAIT_VM_LGKM0(n);                                                                       \
    __builtin_amdgcn_s_barrier();                                                              \
  }
  // one k-step: make the next stage ready, optionally refill the buffer the
  // current stage came from, read the next stage's fragments, then run the
  // current stage's MFMAs
#define WH_STEP(WAITN, REFILL, SREFILL, KREFILL, SN, AC, BC, AN, BN)                           \
  WH_SYNC(WAITN)                                                                               \
  if (REFILL) { WH_ISSUE(SREFILL, KREFILL) }                                                   \
  WH_READ(SN, AN, BN)                                                                          \
  WH_MFMA(AC, BC)

  WH_ISSUE(st0, 0)
  WH_ISSUE(st1, DBK)
  WH_ISSUE(st2, 2 * DBK)
  WH_SYNC(8)
  WH_ISSUE(st3, 3 * DBK)
  WH_READ(st0, a0, b0)
  int kt = 0;
  for (; kt + 8 <= nk; kt += 4) {
    WH_STEP(8, true, st0, (kt + 4) * DBK, st1, a0, b0, a1, b1)
    WH_STEP(8, true, st1, (kt + 5) * DBK, st2, a1, b1, a0, b0)
    WH_STEP(8, true, st2, (kt + 6) * DBK, st3, a0, b0, a1, b1)
    WH_STEP(8, true, st3, (kt + 7) * DBK, st0, a1, b1, a0, b0)
  }
  // last four k-steps (stages nk-4 .. nk-1 live in buffers 0 .. 3)
  WH_STEP(8, false, st0, 0, st1, a0, b0, a1, b1)
  WH_STEP(4, false, st0, 0, st2, a1, b1, a0, b0)
  WH_STEP(0, false, st0, 0, st3, a0, b0, a1, b1)
  WH_MFMA(a1, b1)
#undef WH_READ
#undef WH_MFMA
#undef WH_SYNC
#undef WH_STEP
#undef WH_ISSUE
  // epilogue straight from registers: with B as the first MFMA operand each
  // lane holds C[m][n..n+3] for m = its fragment row, so it writes 4
  // consecutive columns (the 4 lanes of a row cover 16 contiguous columns)
  const int em = m0 + wm * 128 + (lane & 15), en = n0 + wn * 64 + (lane >> 4) * 4;
  if constexpr (EPI == EPI_CROSSKV) {
    // head-major scatter: destination offset = column part + row part
    const int d = p.ckv_d, T_ = p.ckv_T, H_ = p.ckv_H;
    long coff[4];
    float4 cb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = min(en + j * 16, p.N - 4);
      const int l = n / (2 * d), r = n - l * 2 * d;
      const int kv = r / d, c = r - kv * d;
      coff[j] = (((long)(l * 2 + kv) * p.ckv_B * H_ + (c >> 6)) * T_) * 64 + (c & 63);
      cb[j] = p.bias ? *(const float4*)(p.bias + n) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int m = em + i * 16;
      if (m >= p.M) continue;
      const int b = m / T_, t = m - b * T_;
      const long roff = ((long)b * H_ * T_ + t) * 64;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (en + j * 16 + 4 > p.N) continue;
        uint2 u;
        u.x = (uint32_t)f2bf(acc[i][j][0] + cb[j].x) | ((uint32_t)f2bf(acc[i][j][1] + cb[j].y) << 16);
        u.y = (uint32_t)f2bf(acc[i][j][2] + cb[j].z) | ((uint32_t)f2bf(acc[i][j][3] + cb[j].w) << 16);
        *(uint2*)((u16*)p.C + coff[j] + roff) = u;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int m = em + i * 16;
      if (m >= p.M) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = en + j * 16;
        float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
        if (n + 4 <= p.N) {
          epi_store4<EPI>(p, z, m, n, v);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) epi_store<u16, EPI>(p, z, m, n + q, v[q]);
        }
      }
    }
  }
}
// ------------------------------------------------------------------ bf16 MFMA, 256x256, LDS DMA pipeline, persistent
// The 8-wave LDS-DMA kernel above, run as one workgroup per CU that walks a
// share of the tiles. The 4-stage ring runs on across tile boundaries: the
// last four k-steps of a tile load the first four stages of the next one (and
// its bias), so a tile's 16 stores per lane are issued with the next tile's
// loads already in flight. Loads use buffer addressing (scalar resource and k
// offset, one 32-bit VGPR offset per stream); stores use the buffer range
// check to drop rows past M. Every wave issues the same, fixed number of loads
// per tile, and each vmcnt wait allows exactly the loads issued after the
// awaited stage to stay in flight. Loads retire in order among themselves,
// but stores may retire before older loads (a dropped store at once), so a
// pending store must never be counted as one of the operations allowed to
// remain outstanding; the waits count loads only:
//   in-tile wait for stage s+1: the 2 younger stages (8 loads);
//   tail waits: also the next tile's bias load (9);
//   tile head (next tile's bias and stage 0): its stages 1-3 (12).
// With the previous tile's stores younger than those loads, the head wait also
// holds until most of those stores have retired.
// Requirements (checked by the launcher): batch 1, N % 256 == 0, K % 128 == 0,
// K >= 256, ldc % 8 == 0, operands and output under 2 GB.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 buf_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  i32x4 r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));  // stride 0
  r.z = __builtin_amdgcn_readfirstlane((int)bytes);                             // range in bytes
  r.w = 0x00020000;                                                             // gfx9 raw-buffer format word
  return r;
}
// One 16-byte-per-lane buffer load straight into the 1 KB LDS block at `lds`
// (lane L writes bytes 16L..16L+15): address = resource base + voff + soff.
__device__ __forceinline__ void dma16_buf(i32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(lds), "v"(voff), "s"(rsrc),
               "s"(soff)
               : "memory", "m0");
}

// logical tile t -> (tm, tn) in column groups of 4 tile-columns, tile-rows within a group
__device__ __forceinline__ void grouped_coords(int t, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int gsz = 4 * tiles_m, grp = t / gsz, r = t - grp * gsz;
  const int gn = min(4, tiles_n - grp * 4);
  tm = r / gn;
  tn = grp * 4 + (r - tm * gn);
}

template <int EPI>
__global__ __launch_bounds__(512) void gemm_bf16_persist(GemmParams p) {
  __shared__ __attribute__((aligned(1024))) u16 st0[DSTAGE];
  __shared__ __attribute__((aligned(1024))) u16 st1[DSTAGE];
  __shared__ __attribute__((aligned(1024))) u16 st2[DSTAGE];
  __shared__ __attribute__((aligned(1024))) u16 st3[DSTAGE];
  __shared__ __attribute__((aligned(1024))) float bsl[2][TB2];  // bias of the current / next tile
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int tiles_m = (p.M + TB2 - 1) / TB2, tiles_n = p.N / TB2, T = tiles_m * tiles_n;
  // XCD x (= blockIdx.x % 8) owns the logical tiles [lo, hi); its workgroups
  // take every nslot-th one, so the tiles running together on one XCD are
  // consecutive in the grouped order and share weight and activation panels.
  const int x = blockIdx.x & 7, nslot = (gridDim.x - x + 7) >> 3;
  const int lo = (int)(((long)T * x) >> 3), hi = (int)(((long)T * (x + 1)) >> 3);
  int L = lo + (blockIdx.x >> 3);
  if (L >= hi) return;
  int tm, tn;
  grouped_coords(L, tiles_m, tiles_n, tm, tn);

  const i32x4 ra = buf_rsrc(p.A, (uint32_t)(((long)(p.M - 1) * p.lda + p.K) * 2));
  const i32x4 rb = buf_rsrc(p.B, (uint32_t)(((long)(p.N - 1) * p.ldb + p.K) * 2));
  const i32x4 rbias = buf_rsrc(p.bias ? (const void*)p.bias : p.A, p.bias ? (uint32_t)p.N * 4 : 0u);
  const int lr = lane >> 2, lc = (lane & 3) ^ ((lane >> 3) & 3);  // global chunk for LDS slot lane & 3 of row lr
  const uint32_t la0 = wave * 16 * DBK, la1 = (wave + 8) * 16 * DBK;
  const uint32_t lb0 = TB2 * DBK + wave * 16 * DBK, lb1 = TB2 * DBK + (wave + 8) * 16 * DBK;
  uint32_t oa0, oa1, ob0, ob1;  // byte offsets of this lane's 16-byte chunk in its four DMA rows
#define WH_OFFS(TM, TN)                                                                              \
  oa0 = ((uint32_t)min((TM) * TB2 + wave * 16 + lr, p.M - 1) * (uint32_t)p.lda + lc * 8) * 2;        \
  oa1 = ((uint32_t)min((TM) * TB2 + (wave + 8) * 16 + lr, p.M - 1) * (uint32_t)p.lda + lc * 8) * 2;  \
  ob0 = ((uint32_t)((TN) * TB2 + wave * 16 + lr) * (uint32_t)p.ldb + lc * 8) * 2;                    \
  ob1 = ((uint32_t)((TN) * TB2 + (wave + 8) * 16 + lr) * (uint32_t)p.ldb + lc * 8) * 2;
  WH_OFFS(tm, tn)
#define WH_ISSUE(S, k)                                       \
  dma16_buf(ra, oa0, (k) * 2, lds_addr((S) + la0));          \
  dma16_buf(ra, oa1, (k) * 2, lds_addr((S) + la1));          \
  dma16_buf(rb, ob0, (k) * 2, lds_addr((S) + lb0));          \
  dma16_buf(rb, ob1, (k) * 2, lds_addr((S) + lb1));
  // every wave loads the whole 1 KB bias row (identical bytes), so each
  // wave's own wait covers it
#define WH_BIAS(SLOT, TN) \
  dma16_buf(rbias, lane * 16, (TN) * TB2 * 4, (uint32_t)(uintptr_t)(__attribute__((address_space(3))) float*)(bsl[SLOT]));

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int fr = lane & 15, kc = lane >> 4;
  const int nk = p.K / DBK;
  bf16x8 a0[8], b0[4], a1[8], b1[4];
  // B fragment slot s of block j holds tile row 32 (j / 2) + 8 (s / 4) + 4 (j % 2) + s % 4, so a
  // lane's outputs in blocks 2h and 2h+1 are 8 consecutive columns (one 16-byte store)
#define WH_READ(S, AF, BF)                                                                    \
  _Pragma("unroll") for (int j = 0; j < 4; ++j)                                               \
    BF[j] = bitcast<bf16x8>(*(const uint4*)((S) + TB2 * DBK + dswz(wn * 64 + 32 * (j >> 1) + 8 * (fr >> 2) + 4 * (j & 1) + (fr & 3), kc))); \
  _Pragma("unroll") for (int i = 0; i < 8; ++i)                                               \
    AF[i] = bitcast<bf16x8>(*(const uint4*)((S) + dswz(wm * 128 + i * 16 + fr, kc)));
#define WH_MFMA(AF, BF)                                                                       \
  _Pragma("unroll") for (int i = 0; i < 8; ++i)                                               \
    _Pragma("unroll") for (int j = 0; j < 4; ++j)                                             \
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(BF[j], AF[i], acc[i][j], 0, 0, 0);
#define WH_SYNC(n)             \
  {                            \
    WH_WAIT_VM_LGKM0(n);       \
    __builtin_amdgcn_s_barrier(); \
  }
  // one k-step: wait for the stage whose fragments are read next, refill the
  // buffer the current stage came from, read the next fragments, then the
  // current stage's MFMAs
#define WH_STEP(WAITN, SREFILL, KREFILL, SN, AC, BC, AN, BN) \
  WH_SYNC(WAITN)                                             \
  WH_ISSUE(SREFILL, KREFILL)                                 \
  WH_READ(SN, AN, BN)                                        \
  WH_MFMA(AC, BC)
#define WH_ROUND(W0, W1, W2, W3, KT)                                \
  WH_STEP(W0, st0, ((KT) + 4) * DBK, st1, a0, b0, a1, b1)           \
  WH_STEP(W1, st1, ((KT) + 5) * DBK, st2, a1, b1, a0, b0)           \
  WH_STEP(W2, st2, ((KT) + 6) * DBK, st3, a0, b0, a1, b1)           \
  WH_STEP(W3, st3, ((KT) + 7) * DBK, st0, a1, b1, a0, b0)

  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(p.C, (short)0, (int)((long)p.M * p.ldc * 2), 0x00020000);
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  // the first tile starts like every later one: bias and stages 0-3 in flight
  WH_BIAS(0, tn)
  WH_ISSUE(st0, 0)
  WH_ISSUE(st1, DBK)
  WH_ISSUE(st2, 2 * DBK)
  WH_ISSUE(st3, 3 * DBK)
  asm volatile("" ::: "memory");
  int par = 0;
  for (;;) {
    WH_SYNC(12)  // this tile's bias and stage 0 have landed (stages 1-3 may be in flight)
    WH_READ(st0, a0, b0)
    WH_ROUND(8, 8, 8, 8, 0)
    for (int kt = 4; kt + 8 <= nk; kt += 4) {
      WH_ROUND(8, 8, 8, 8, kt)
    }
    // tail: the next tile's bias and stages 0-3 (when there is no next tile,
    // the same tile's are loaded again so that the wait counts stay exact)
    const int Ln = L + nslot;
    const bool more = Ln < hi;
    int tmn = tm, tnn = tn;
    if (more) grouped_coords(Ln, tiles_m, tiles_n, tmn, tnn);
    const int m0 = tm * TB2, n0 = tn * TB2;
    WH_OFFS(tmn, tnn)
    WH_SYNC(8)
    WH_BIAS(par ^ 1, tnn)
    WH_ISSUE(st0, 0)
    WH_READ(st1, a1, b1)
    WH_MFMA(a0, b0)
    WH_STEP(9, st1, DBK, st2, a1, b1, a0, b0)
    WH_STEP(9, st2, 2 * DBK, st3, a0, b0, a1, b1)
    WH_SYNC(63)  // all waves are done reading buffer 3; nothing to wait for in vmcnt
    WH_ISSUE(st3, 3 * DBK)
    WH_MFMA(a1, b1)
    // epilogue: bias from LDS, activation, bf16, 16 buffer stores of 16 bytes per
    // lane (each instruction writes 64 contiguous bytes of 16 rows); rows past M
    // get an offset beyond the range and are dropped
    {
      // lane columns: en + 32 h + 0..7 come from blocks 2h (first 4) and 2h + 1
      const int en = wn * 64 + (lane >> 4) * 8;
      float4 bj[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bj[j] = p.bias ? *(const float4*)(&bsl[par][en + 32 * (j >> 1) + 4 * (j & 1)]) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int m = m0 + wm * 128 + i * 16 + (lane & 15);
        const uint32_t roff = m < p.M ? ((uint32_t)m * (uint32_t)p.ldc + (uint32_t)(n0 + en)) * 2 : 0x80000000u;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float v[8];
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int j = 2 * h + q;
            v[4 * q + 0] = acc[i][j][0] + bj[j].x; v[4 * q + 1] = acc[i][j][1] + bj[j].y;
            v[4 * q + 2] = acc[i][j][2] + bj[j].z; v[4 * q + 3] = acc[i][j][3] + bj[j].w;
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
          if constexpr (EPI == EPI_GELU) {
#pragma unroll
            for (int q = 0; q < 8; ++q) v[q] = gelu_erf(v[q]);
          }
          const u32x4 u = {f2bf2(v[0], v[1]), f2bf2(v[2], v[3]), f2bf2(v[4], v[5]), f2bf2(v[6], v[7])};
          __builtin_amdgcn_raw_buffer_store_b128(u, rc, roff + h * 64, 0, 0);
        }
      }
    }
    // the stores stay ahead of the next tile's waits in program order
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    if (!more) break;
    L = Ln; tm = tmn; tn = tnn; par ^= 1;
  }
  WH_WAIT_VM(0);  // no LDS-DMA write may still be in flight when the workgroup ends
#undef WH_READ
#undef WH_MFMA
#undef WH_SYNC
#undef WH_STEP
#undef WH_ROUND
#undef WH_ISSUE
#undef WH_BIAS
#undef WH_OFFS
}

// ------------------------------------------------------------------ fp8 E4M3 MFMA, 256x256, LDS DMA pipeline
// The mixed_fp8 sites (showcase page, precision.py card: encoder QKV and FFN
// in fp8 E4M3; gemm_hopper.cu card: FP8 E4M3 GEMM). A [M, K] and B [N, K] are
// E4M3 codes, K-contiguous; C = epi(acc * sa[m / a_rows_per_scale] * sb + bias)
// in bf16. The memory pipeline is the bf16 LDS-DMA kernel's byte for byte
// (one 256x256 tile per workgroup, 8 waves, 4-stage ring): a stage holds 64
// bytes of every tile row, which is 64 fp8 values instead of 32 bf16, and one
// 32x32x64 fp8 MFMA per 32x32 block consumes exactly one stage in the MFMA
// time the bf16 kernel spends on one stage, so the same traffic feeds twice
// the FLOPs. The launcher passes K and the row strides in 2-byte units
// (bytes / 2) so that the address computations are the bf16 kernel's.
// A lane's MFMA operand is 32 bytes of one row: chunks 2g, 2g+1 (g = lane / 32)
// of row lane % 32, for A and B alike; the K order inside the MFMA is the same
// for both operands, so any K permutation it applies cancels in the products.
// B row slot i of a 32-row block holds tile column 16 ((i / 4) % 2) + 4 (i / 8)
// + i % 4, so the 16 outputs a lane holds (rows 8 (v / 4) + 4 g + v % 4 of the
// MFMA result) are 16 consecutive columns g*16 .. g*16 + 15: two 16-byte stores.
// Requirements (checked by the launcher): K % 256 == 0, K >= 512, N % 256 == 0,
// lda, ldb % 2 == 0, ldc % 8 == 0, a_rows_per_scale >= 256.
typedef int i32x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ int fp8_bcol(int i) { return ((i >> 2) & 1) * 16 + (i >> 3) * 4 + (i & 3); }

template <int EPI>
__global__ __launch_bounds__(512) void gemm_fp8_dma(GemmParams p) {
  __shared__ __attribute__((aligned(1024))) u16 st0[DSTAGE];
  __shared__ __attribute__((aligned(1024))) u16 st1[DSTAGE];
  __shared__ __attribute__((aligned(1024))) u16 st2[DSTAGE];
  __shared__ __attribute__((aligned(1024))) u16 st3[DSTAGE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int tiles_n = p.N / TB2;
  const int tiles_m = (p.M + TB2 - 1) / TB2;
  int tm, tn;
  tile_order_grouped<4>(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const u16* A = (const u16*)p.A;
  const u16* B = (const u16*)p.B;
  const int m0 = tm * TB2, n0 = tn * TB2;

  const int lr = lane >> 2, lc = (lane & 3) ^ ((lane >> 3) & 3);
  const u16* ga0 = A + (long)min(m0 + wave * 16 + lr, p.M - 1) * p.lda + lc * 8;
  const u16* ga1 = A + (long)min(m0 + (wave + 8) * 16 + lr, p.M - 1) * p.lda + lc * 8;
  const u16* gb0 = B + (long)(n0 + wave * 16 + lr) * p.ldb + lc * 8;
  const u16* gb1 = B + (long)(n0 + (wave + 8) * 16 + lr) * p.ldb + lc * 8;
  const int la0 = wave * 16 * DBK, la1 = (wave + 8) * 16 * DBK;
  const int lb0 = TB2 * DBK + wave * 16 * DBK, lb1 = TB2 * DBK + (wave + 8) * 16 * DBK;
#define WH_ISSUE(S, k)                                                                         \
  dma16(ga0 + (k), __builtin_amdgcn_readfirstlane(lds_addr((S) + la0)));                        \
  dma16(ga1 + (k), __builtin_amdgcn_readfirstlane(lds_addr((S) + la1)));                        \
  dma16(gb0 + (k), __builtin_amdgcn_readfirstlane(lds_addr((S) + lb0)));                        \
  dma16(gb1 + (k), __builtin_amdgcn_readfirstlane(lds_addr((S) + lb1)));

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int fr = lane & 31, g = lane >> 5;
  const int nk = p.K / DBK;
  i32x8 a0[4], b0[2], a1[4], b1[2];
#define WH_FRAG(S, ROW, DST)                                                       \
  {                                                                                \
    const uint4 lo_ = *(const uint4*)((S) + dswz((ROW), 2 * g));                   \
    const uint4 hi_ = *(const uint4*)((S) + dswz((ROW), 2 * g + 1));               \
    DST = i32x8{(int)lo_.x, (int)lo_.y, (int)lo_.z, (int)lo_.w,                     \
                (int)hi_.x, (int)hi_.y, (int)hi_.z, (int)hi_.w};                    \
  }
#define WH_READ(S, AF, BF)                                                                 \
  _Pragma("unroll") for (int j = 0; j < 2; ++j)                                            \
    WH_FRAG((S) + TB2 * DBK, wn * 64 + 32 * j + fp8_bcol(fr), BF[j])                        \
  _Pragma("unroll") for (int i = 0; i < 4; ++i)                                            \
    WH_FRAG((S), wm * 128 + i * 32 + fr, AF[i])
  // E4M3 both operands (format 0), unit block scales (E8M0 127 = 2^0)
#define WH_MFMA(AF, BF)                                                                    \
  _Pragma("unroll") for (int i = 0; i < 4; ++i)                                            \
    _Pragma("unroll") for (int j = 0; j < 2; ++j)                                          \
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(BF[j], AF[i], acc[i][j], 0, 0, 0, 127, 0, 127);
#define WH_SYNC(n)                                                                             \
  {                                                                                            \
    WH_WAIT_VM_LGKM0(n);                                                                       \
    __builtin_amdgcn_s_barrier();                                                              \
  }
#define WH_STEP(WAITN, REFILL, SREFILL, KREFILL, SN, AC, BC, AN, BN)                           \
  WH_SYNC(WAITN)                                                                               \
  if (REFILL) { WH_ISSUE(SREFILL, KREFILL) }                                                   \
  WH_READ(SN, AN, BN)                                                                          \
  WH_MFMA(AC, BC)

  WH_ISSUE(st0, 0)
  WH_ISSUE(st1, DBK)
  WH_ISSUE(st2, 2 * DBK)
  WH_SYNC(8)
  WH_ISSUE(st3, 3 * DBK)
  WH_READ(st0, a0, b0)
  int kt = 0;
  for (; kt + 8 <= nk; kt += 4) {
    WH_STEP(8, true, st0, (kt + 4) * DBK, st1, a0, b0, a1, b1)
    WH_STEP(8, true, st1, (kt + 5) * DBK, st2, a1, b1, a0, b0)
    WH_STEP(8, true, st2, (kt + 6) * DBK, st3, a0, b0, a1, b1)
    WH_STEP(8, true, st3, (kt + 7) * DBK, st0, a1, b1, a0, b0)
  }
  WH_STEP(8, false, st0, 0, st1, a0, b0, a1, b1)
  WH_STEP(4, false, st0, 0, st2, a1, b1, a0, b0)
  WH_STEP(0, false, st0, 0, st3, a0, b0, a1, b1)
  WH_MFMA(a1, b1)
#undef WH_FRAG
#undef WH_READ
#undef WH_MFMA
#undef WH_SYNC
#undef WH_STEP
#undef WH_ISSUE
  // epilogue: per-row activation scale (a tile spans at most two scale
  // groups), weight scale, bias, activation, bf16, two 16-byte stores per
  // 32x32 block
  const int rps = p.a_rows_per_scale;
  const int c0 = m0 / rps, c1 = min(m0 + TB2 - 1, p.M - 1) / rps, mb = (c0 + 1) * rps;
  const float s_w = p.b_scale[0], s_lo = p.a_scale[c0] * s_w, s_hi = p.a_scale[c1] * s_w;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + wm * 128 + i * 32 + fr;
    if (m >= p.M) continue;
    const float sm = (m >= mb) ? s_hi : s_lo;
    u16* crow = (u16*)p.C + (long)m * p.ldc + n0;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int cl = wn * 64 + 32 * j + 16 * g;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float v[8];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const float4 bq = p.bias ? *(const float4*)(p.bias + n0 + cl + 8 * h + 4 * q) : make_float4(0.f, 0.f, 0.f, 0.f);
          v[4 * q + 0] = acc[i][j][8 * h + 4 * q + 0] * sm + bq.x;
          v[4 * q + 1] = acc[i][j][8 * h + 4 * q + 1] * sm + bq.y;
          v[4 * q + 2] = acc[i][j][8 * h + 4 * q + 2] * sm + bq.z;
          v[4 * q + 3] = acc[i][j][8 * h + 4 * q + 3] * sm + bq.w;
        }
        if constexpr (EPI == EPI_GELU) {
#pragma unroll
          for (int q = 0; q < 8; ++q) v[q] = gelu_erf(v[q]);
        }
        *(uint4*)(crow + cl + 8 * h) = uint4{f2bf2(v[0], v[1]), f2bf2(v[2], v[3]), f2bf2(v[4], v[5]), f2bf2(v[6], v[7])};
      }
    }
  }
}

hipError_t launch_gemm_fp8(Epi epi, const GemmParams& q, hipStream_t s) {
  // K and strides in bytes here; the kernel takes them in 2-byte units
  if (q.K % 256 || q.K < 512 || q.N % TB2 || q.lda % 2 || q.ldb % 2 || q.ldc % 8 || q.batch != 1 ||
      q.a_rows_per_scale < TB2 || !q.a_scale || !q.b_scale || q.M <= 0)
    return hipErrorInvalidValue;
  if ((long)q.M * q.lda > (1L << 31) || (long)q.N * q.ldb > (1L << 31) || (long)q.M * q.ldc * 2 > (1L << 31))
    return hipErrorInvalidValue;
  if (epi != EPI_STORE && epi != EPI_GELU) return hipErrorInvalidValue;
  GemmParams p = q;
  p.K = q.K / 2; p.lda = q.lda / 2; p.ldb = q.ldb / 2;
  dim3 grid(((p.M + TB2 - 1) / TB2) * (p.N / TB2));
  if (epi == EPI_GELU) hipLaunchKernelGGL(gemm_fp8_dma<EPI_GELU>, grid, dim3(512), 0, s, p);
  else hipLaunchKernelGGL(gemm_fp8_dma<EPI_STORE>, grid, dim3(512), 0, s, p);
  return hipGetLastError();
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

// compute units of the current device (one persistent workgroup each)
static int num_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

hipError_t launch_gemm(ActType t, Epi epi, const GemmParams& p, hipStream_t s) {
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
  if (t == ACT_BF16) {
    const int tiles2 = ((p.M + TB2 - 1) / TB2) * ((p.N + TB2 - 1) / TB2);
    const bool w4_ok = p.N % 8 == 0 &&
                       (epi == EPI_STORE || epi == EPI_GELU || epi == EPI_GELU_PE || epi == EPI_CROSSKV);
    const bool dma_ok = w4_ok && p.K % (4 * DBK) == 0;  // the LDS-DMA kernels run whole 4-stage rounds
    // persistent variant: whole 256-column tiles, one workgroup per CU
    const bool pers_ok = dma_ok && p.batch == 1 && p.N % TB2 == 0 && p.K >= 8 * DBK && (epi == EPI_STORE || epi == EPI_GELU) &&
                         (long)p.M * p.ldc * 2 < (1L << 31) && ((long)(p.M - 1) * p.lda + p.K) * 2 < (1L << 32) &&
                         ((long)(p.N - 1) * p.ldb + p.K) * 2 < (1L << 32) && p.ldc >= p.N && p.ldc % 8 == 0;
    int v = p.variant;
    if (v == 0) v = (tiles2 * p.batch >= 192 && epi != EPI_DEC_QKV) ? (pers_ok ? 9 : dma_ok ? 4 : 2) : 1;
    if ((v == 3 && !w4_ok) || (v == 4 && !dma_ok)) v = 1;
    if (v == 5) v = 6;  // the 4-wave 256x256 form is retired (its 256 accumulators per lane do not fit)
    if (v == 9 && !pers_ok) v = dma_ok ? 4 : 1;
    if (v == 9) {
      dim3 grid(min(num_cus(), ((p.M + TB2 - 1) / TB2) * (p.N / TB2) + 7));
      if (epi == EPI_GELU) hipLaunchKernelGGL(gemm_bf16_persist<EPI_GELU>, grid, dim3(512), 0, s, p);
      else hipLaunchKernelGGL(gemm_bf16_persist<EPI_STORE>, grid, dim3(512), 0, s, p);
      return hipGetLastError();
    }
    if (v == 6 && !dma_ok) v = 1;
    if (v == 6) {  // plain (ungrouped) tile order, for comparison
      dim3 grid(tiles2, 1, p.batch);
#define CALL(E) hipLaunchKernelGGL((gemm_bf16_dma<E, 0>), grid, dim3(512), 0, s, p)
      switch (epi) {
        case EPI_STORE: CALL(EPI_STORE); break;
        case EPI_GELU: CALL(EPI_GELU); break;
        case EPI_GELU_PE: CALL(EPI_GELU_PE); break;
        default: CALL(EPI_CROSSKV); break;
      }
#undef CALL
      return hipGetLastError();
    }
    if (v == 4) {
      dim3 grid(tiles2, 1, p.batch);
#define CALL(E) hipLaunchKernelGGL((gemm_bf16_dma<E, 1>), grid, dim3(512), 0, s, p)
      switch (epi) {
        case EPI_STORE: CALL(EPI_STORE); break;
        case EPI_GELU: CALL(EPI_GELU); break;
        case EPI_GELU_PE: CALL(EPI_GELU_PE); break;
        default: CALL(EPI_CROSSKV); break;
      }
#undef CALL
      return hipGetLastError();
    }
    if (v == 2 && epi == EPI_DEC_QKV) v = 1;
    if (v == 3) {
      dim3 grid(tiles2, 1, p.batch);
#define CALL(E) hipLaunchKernelGGL(gemm_bf16_256w4<E>, grid, dim3(256), 0, s, p)
      switch (epi) {
        case EPI_STORE: CALL(EPI_STORE); break;
        case EPI_GELU: CALL(EPI_GELU); break;
        case EPI_GELU_PE: CALL(EPI_GELU_PE); break;
        default: CALL(EPI_CROSSKV); break;
      }
#undef CALL
    } else if (v == 2) {
      dim3 grid(tiles2, 1, p.batch);
#define CALL(E) hipLaunchKernelGGL(gemm_bf16_256<E>, grid, dim3(512), 0, s, p)
      switch (epi) {
        case EPI_STORE: CALL(EPI_STORE); break;
        case EPI_GELU: CALL(EPI_GELU); break;
        case EPI_GELU_PE: CALL(EPI_GELU_PE); break;
        case EPI_F32: CALL(EPI_F32); break;
        case EPI_CROSSKV: CALL(EPI_CROSSKV); break;
        default: return hipErrorInvalidValue;
      }
#undef CALL
    } else {
      const int tiles = ((p.M + TB - 1) / TB) * ((p.N + TB - 1) / TB);
      dim3 grid(tiles, 1, p.batch);
#define CALL(E) hipLaunchKernelGGL(gemm_bf16_128<E>, grid, dim3(256), 0, s, p)
      WH_EPI_SWITCH(epi, CALL)
#undef CALL
    }
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
