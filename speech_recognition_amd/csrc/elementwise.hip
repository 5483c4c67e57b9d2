// Memory-bound kernels of the hot path: fused residual + LayerNorm (the
// whisper_blaze showcase page's layernorm_fused.cu card: residual add and
// LayerNorm in one pass; the project page's "Direct Kernel API" returns both
// the normalised value and the pre-norm sum), the fp8 codec (E4M3, and E5M2
// for range) with a per-tensor scale (fp8_quantize.cu card; project page
// quantise_e4m3 / dequantise_e4m3), weight packing, decoder embeddings and the greedy argmax.
#include "common.hpp"
#include "internal.hpp"

namespace wh {

// ------------------------------------------------------------------ vector IO
template <typename T> struct Vec4;
template <> struct Vec4<u16> {
  static __device__ __forceinline__ void ld(const u16* p, float v[4]) {
    const uint2 u = *(const uint2*)p;
    v[0] = __uint_as_float(u.x << 16); v[1] = __uint_as_float(u.x & 0xffff0000u);
    v[2] = __uint_as_float(u.y << 16); v[3] = __uint_as_float(u.y & 0xffff0000u);
  }
  static __device__ __forceinline__ void st(u16* p, const float v[4]) {
    uint2 u;
    u.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
    u.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
    *(uint2*)p = u;
  }
};
template <> struct Vec4<float> {
  static __device__ __forceinline__ void ld(const float* p, float v[4]) {
    const float4 u = *(const float4*)p; v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
  }
  static __device__ __forceinline__ void st(float* p, const float v[4]) {
    *(float4*)p = make_float4(v[0], v[1], v[2], v[3]);
  }
};

// ------------------------------------------------------------------ residual + LayerNorm
// One wave64 per row; each lane holds up to 8 groups of 4 elements (d <= 2048)
// in registers, so the row is read once and written once. The residual
// stream is fp32: total = fl32(h + residual) (h alone if there is no
// residual); statistics in fp32 over total (two passes over registers: mean,
// then mean squared deviation); normed is stored in the activation type.
template <typename TH, typename T>
__global__ __launch_bounds__(256) void layernorm_kernel(const TH* h, const float* res, const float* g,
                                                        const float* b, float eps, int M, int d, T* normed,
                                                        float* total, float* row_amax) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= M) return;
  const int nc = d >> 2;
  const long off = (long)row * d;
  float v[8][4];
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = lane + i * 64;
    if (c < nc) {
      Vec4<TH>::ld(h + off + c * 4, v[i]);
      if (res) {
        const float4 r = *(const float4*)(res + off + c * 4);
        v[i][0] += r.x; v[i][1] += r.y; v[i][2] += r.z; v[i][3] += r.w;
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) sum += v[i][k];
    }
  }
  const float mean = wave_sum(sum) / (float)d;
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (lane + i * 64 < nc)
#pragma unroll
      for (int k = 0; k < 4; ++k) { const float t = v[i][k] - mean; sq += t * t; }
  const float var = wave_sum(sq) / (float)d;
  const float rstd = 1.0f / sqrtf(var + eps);
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = lane + i * 64;
    if (c < nc) {
      if (total) *(float4*)(total + off + c * 4) = make_float4(v[i][0], v[i][1], v[i][2], v[i][3]);
      if (normed) {
        const float4 gg = *(const float4*)(g + c * 4), bb = *(const float4*)(b + c * 4);
        float o[4] = {(v[i][0] - mean) * rstd * gg.x + bb.x, (v[i][1] - mean) * rstd * gg.y + bb.y,
                      (v[i][2] - mean) * rstd * gg.z + bb.z, (v[i][3] - mean) * rstd * gg.w + bb.w};
        Vec4<T>::st(normed + off + c * 4, o);
#pragma unroll
        for (int k = 0; k < 4; ++k) amax = fmaxf(amax, fabsf(Act<T>::round(o[k])));  // as stored
      }
    }
  }
  if (row_amax) {
    amax = wave_max(amax);
    if (lane == 0) row_amax[row] = amax;
  }
}

hipError_t launch_layernorm(ActType t, bool h_f32, const void* h, const float* res, const float* g, const float* b,
                            float eps, int M, int d, void* normed, float* total, hipStream_t s, float* row_amax) {
  if (M <= 0) return hipSuccess;
  if (row_amax && !normed) return hipErrorInvalidValue;
  dim3 grid((M + 3) / 4);
  if (t == ACT_BF16 && !h_f32)
    hipLaunchKernelGGL((layernorm_kernel<u16, u16>), grid, dim3(256), 0, s, (const u16*)h, res, g, b, eps, M, d,
                       (u16*)normed, total, row_amax);
  else if (t == ACT_BF16)
    hipLaunchKernelGGL((layernorm_kernel<float, u16>), grid, dim3(256), 0, s, (const float*)h, res, g, b, eps, M, d,
                       (u16*)normed, total, row_amax);
  else
    hipLaunchKernelGGL((layernorm_kernel<float, float>), grid, dim3(256), 0, s, (const float*)h, res, g, b, eps, M,
                       d, (float*)normed, total, row_amax);
  return hipGetLastError();
}

// ------------------------------------------------------------------ fp8 codec (E4M3, E5M2)
// 8 consecutive elements (16-byte aligned group) as fp32
__device__ __forceinline__ void load8(const u16* p, float v[8]) {
  const uint4 w = *(const uint4*)p;
  const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(a[i] << 16);
    v[2 * i + 1] = __uint_as_float(a[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float v[8]) {
  const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

template <typename T>
__global__ __launch_bounds__(256) void amax_partial(const T* x, size_t n, float* partial) {
  float m = 0.f;
  // 8 elements per lane per iteration from 16-byte-aligned groups (x is 16-byte
  // aligned), then the tail one by one
  const size_t n8 = n / 8, stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += stride) {
    float v[8];
    load8(x + i * 8, v);
#pragma unroll
    for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(v[k]));
  }
  for (size_t i = n8 * 8 + (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride)
    m = fmaxf(m, fabsf(Act<T>::cvt(x[i])));
  m = wave_max(m);
  __shared__ float sm[4];
  if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) partial[blockIdx.x] = fmaxf(fmaxf(sm[0], sm[1]), fmaxf(sm[2], sm[3]));
}

// scale = fl32(amax) / (largest finite magnitude of the format), 1 for amax 0
__global__ __launch_bounds__(64) void amax_final(const float* partial, int n, float fmax, float* scale_out) {
  float m = 0.f;
  for (int i = threadIdx.x; i < n; i += 64) m = fmaxf(m, partial[i]);
  m = wave_max(m);
  if (threadIdx.x == 0) scale_out[0] = (m > 0.f) ? m / fmax : 1.0f;
}

hipError_t launch_amax(ActType t, int fmt, const void* x, size_t n, float* partial, int n_partial, float* scale_out,
                       hipStream_t s) {
  if (t == ACT_BF16)
    hipLaunchKernelGGL(amax_partial<u16>, dim3(n_partial), dim3(256), 0, s, (const u16*)x, n, partial);
  else
    hipLaunchKernelGGL(amax_partial<float>, dim3(n_partial), dim3(256), 0, s, (const float*)x, n, partial);
  const float fmax = fmt == FP8_E5M2 ? fp8_max<FP8_E5M2>() : fp8_max<FP8_E4M3>();
  hipLaunchKernelGGL(amax_final, dim3(1), dim3(64), 0, s, partial, n_partial, fmax, scale_out);
  return hipGetLastError();
}

template <typename T, int FMT>
__global__ __launch_bounds__(256) void fp8_quantize_kernel(const T* x, size_t n, const float* scale, uint8_t* codes) {
  const float inv = 1.0f / scale[0];
  // 8 elements per lane per iteration (x 16-byte and codes 8-byte aligned per
  // group), then the tail one by one
  const size_t n8 = n / 8, stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += stride) {
    float v[8];
    load8(x + i * 8, v);
    uint32_t c[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) c[k] = fp8_encode<FMT>(v[k] * inv);
    *(uint2*)(codes + i * 8) = uint2{c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24),
                                     c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24)};
  }
  for (size_t i = n8 * 8 + (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride)
    codes[i] = (uint8_t)fp8_encode<FMT>(Act<T>::cvt(x[i]) * inv);
}

template <typename T, int FMT>
__global__ __launch_bounds__(256) void fp8_dequantize_kernel(const uint8_t* codes, size_t n, const float* scale, T* y) {
  const float s = scale[0];
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    float v[4];
    fp8x4_decode<FMT>(codes[i], v);
    y[i] = Act<T>::st(v[0] * s);
  }
}

// ------------------------------------------------------------------ per-chunk activation quantisation
// The activation entering an fp8 GEMM site, bf16 [rows, K] with rows in
// chunks of rows_per_chunk (one 30 s clip each), becomes E4M3 codes with one
// scale per chunk: scale = fl32(amax of the chunk) / 448 (1 if the chunk is
// all zero), code = e4m3(fl32(x * fl32(1 / scale))). Pass 1 writes CQ_PARTS
// partial maxima per chunk; pass 2 reduces them in every workgroup, quantises
// its slice and the chunk's first workgroup stores the scale.
constexpr int CQ_PARTS = 64;

__global__ __launch_bounds__(256) void chunk_amax_kernel(const u16* __restrict__ x, long chunk_elems, long total,
                                                         float* __restrict__ partial) {
  const int c = blockIdx.y;
  const long begin = (long)c * chunk_elems, end = min(begin + chunk_elems, total);
  const long n8 = (end - begin) / 8;
  float m = 0.f;
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n8; i += (long)CQ_PARTS * 256) {
    float v[8];
    load8(x + begin + i * 8, v);
#pragma unroll
    for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(v[k]));
  }
  m = wave_max(m);
  __shared__ float sm[4];
  if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) partial[c * CQ_PARTS + blockIdx.x] = fmaxf(fmaxf(sm[0], sm[1]), fmaxf(sm[2], sm[3]));
}

__global__ __launch_bounds__(256) void chunk_quant_kernel(const u16* __restrict__ x, long chunk_elems, long total,
                                                          const float* __restrict__ partial,
                                                          float* __restrict__ scales, uint8_t* __restrict__ codes) {
  const int c = blockIdx.y;
  __shared__ float s_inv;
  if (threadIdx.x < 64) {
    const float m = wave_max(partial[c * CQ_PARTS + threadIdx.x]);
    if (threadIdx.x == 0) {
      const float sc = (m > 0.f) ? m / 448.0f : 1.0f;
      s_inv = 1.0f / sc;
      if (blockIdx.x == 0) scales[c] = sc;
    }
  }
  __syncthreads();
  const float inv = s_inv;
  const long begin = (long)c * chunk_elems, end = min(begin + chunk_elems, total);
  const long n8 = (end - begin) / 8;
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n8; i += (long)CQ_PARTS * 256) {
    float v[8];
    load8(x + begin + i * 8, v);
    uint32_t q[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) q[k] = e4m3_encode(v[k] * inv);
    *(uint2*)(codes + begin + i * 8) = uint2{q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24),
                                             q[4] | (q[5] << 8) | (q[6] << 16) | (q[7] << 24)};
  }
}

// The same quantisation of a bf16 activation whose rows' maxima |x| are
// already known (row_amax[m], as the LayerNorm kernel leaves them): each
// workgroup reduces its chunk's row maxima, so no amax pass over x is needed.
__global__ __launch_bounds__(256) void chunk_quant_rows_kernel(const u16* __restrict__ x, int K, long rows,
                                                               int rows_per_chunk, const float* __restrict__ row_amax,
                                                               float* __restrict__ scales,
                                                               uint8_t* __restrict__ codes) {
  const int c = blockIdx.y;
  const long r0 = (long)c * rows_per_chunk, r1 = min(r0 + rows_per_chunk, rows);
  float m = 0.f;
  for (long r = r0 + threadIdx.x; r < r1; r += 256) m = fmaxf(m, row_amax[r]);
  m = wave_max(m);
  __shared__ float sm[4];
  __shared__ float s_inv;
  if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float mx = fmaxf(fmaxf(sm[0], sm[1]), fmaxf(sm[2], sm[3]));
    const float sc = (mx > 0.f) ? mx / 448.0f : 1.0f;
    s_inv = 1.0f / sc;
    if (blockIdx.x == 0) scales[c] = sc;
  }
  __syncthreads();
  const float inv = s_inv;
  const long begin = r0 * K, n8 = (r1 - r0) * K / 8;
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n8; i += (long)CQ_PARTS * 256) {
    float v[8];
    load8(x + begin + i * 8, v);
    uint32_t q[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) q[k] = e4m3_encode(v[k] * inv);
    *(uint2*)(codes + begin + i * 8) = uint2{q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24),
                                             q[4] | (q[5] << 8) | (q[6] << 16) | (q[7] << 24)};
  }
}

hipError_t launch_chunk_quant_rows_fp8(const void* x, long rows, int K, int rows_per_chunk, const float* row_amax,
                                       float* scales, uint8_t* codes, hipStream_t s) {
  if (rows <= 0 || K % 8 || rows_per_chunk <= 0 || !row_amax) return hipErrorInvalidValue;
  const int n_chunks = (int)((rows + rows_per_chunk - 1) / rows_per_chunk);
  hipLaunchKernelGGL(chunk_quant_rows_kernel, dim3(CQ_PARTS, n_chunks), dim3(256), 0, s, (const u16*)x, K, rows,
                     rows_per_chunk, row_amax, scales, codes);
  return hipGetLastError();
}

hipError_t launch_chunk_quant_fp8(const void* x, long rows, int K, int rows_per_chunk, float* partial,
                                  float* scales, uint8_t* codes, hipStream_t s) {
  if (rows <= 0 || K % 8 || rows_per_chunk <= 0) return hipErrorInvalidValue;
  const int n_chunks = (int)((rows + rows_per_chunk - 1) / rows_per_chunk);
  const long chunk_elems = (long)rows_per_chunk * K, total = rows * K;
  dim3 grid(CQ_PARTS, n_chunks);
  hipLaunchKernelGGL(chunk_amax_kernel, grid, dim3(256), 0, s, (const u16*)x, chunk_elems, total, partial);
  hipLaunchKernelGGL(chunk_quant_kernel, grid, dim3(256), 0, s, (const u16*)x, chunk_elems, total, partial, scales,
                     codes);
  return hipGetLastError();
}

static int grid_for(size_t n) {
  size_t g = (n + 255) / 256;
  return (int)(g > 8192 ? 8192 : (g < 1 ? 1 : g));
}

template <int FMT>
static void quantize_fmt(ActType t, const void* x, size_t n, const float* scale, uint8_t* codes, hipStream_t s) {
  if (t == ACT_BF16)
    hipLaunchKernelGGL((fp8_quantize_kernel<u16, FMT>), dim3(grid_for(n)), dim3(256), 0, s, (const u16*)x, n, scale,
                       codes);
  else
    hipLaunchKernelGGL((fp8_quantize_kernel<float, FMT>), dim3(grid_for(n)), dim3(256), 0, s, (const float*)x, n,
                       scale, codes);
}

hipError_t launch_fp8_quantize(ActType t, int fmt, const void* x, size_t n, const float* scale, uint8_t* codes,
                               hipStream_t s) {
  if (!n) return hipSuccess;
  if (fmt == FP8_E5M2) quantize_fmt<FP8_E5M2>(t, x, n, scale, codes, s);
  else quantize_fmt<FP8_E4M3>(t, x, n, scale, codes, s);
  return hipGetLastError();
}

template <int FMT>
static void dequantize_fmt(ActType t, const uint8_t* codes, size_t n, const float* scale, void* y, hipStream_t s) {
  if (t == ACT_BF16)
    hipLaunchKernelGGL((fp8_dequantize_kernel<u16, FMT>), dim3(grid_for(n)), dim3(256), 0, s, codes, n, scale,
                       (u16*)y);
  else
    hipLaunchKernelGGL((fp8_dequantize_kernel<float, FMT>), dim3(grid_for(n)), dim3(256), 0, s, codes, n, scale,
                       (float*)y);
}

hipError_t launch_fp8_dequantize(ActType t, int fmt, const uint8_t* codes, size_t n, const float* scale, void* y,
                                 hipStream_t s) {
  if (!n) return hipSuccess;
  if (fmt == FP8_E5M2) dequantize_fmt<FP8_E5M2>(t, codes, n, scale, y, s);
  else dequantize_fmt<FP8_E4M3>(t, codes, n, scale, y, s);
  return hipGetLastError();
}

// ------------------------------------------------------------------ packing / layout
template <typename T>
__global__ __launch_bounds__(256) void convert_kernel(const float* src, T* dst, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
    dst[i] = Act<T>::st(src[i]);
}

hipError_t launch_convert(ActType t, const float* src, void* dst, size_t n, hipStream_t s) {
  if (!n) return hipSuccess;
  if (t == ACT_BF16) hipLaunchKernelGGL(convert_kernel<u16>, dim3(grid_for(n)), dim3(256), 0, s, src, (u16*)dst, n);
  else hipLaunchKernelGGL(convert_kernel<float>, dim3(grid_for(n)), dim3(256), 0, s, src, (float*)dst, n);
  return hipGetLastError();
}

// conv weight [c_out][c_in][k] -> implicit-GEMM layout [c_out][k * c_in] (tap-major)
template <typename T>
__global__ __launch_bounds__(256) void pack_conv_kernel(const float* w, int c_out, int c_in, int k, T* dst) {
  const size_t n = (size_t)c_out * c_in * k;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    const int o = (int)(i / ((size_t)c_in * k));
    const int r = (int)(i - (size_t)o * c_in * k);
    const int j = r / c_in, ci = r - j * c_in;
    dst[i] = Act<T>::st(w[((size_t)o * c_in + ci) * k + j]);
  }
}

hipError_t launch_pack_conv(ActType t, const float* w, int c_out, int c_in, int k, void* dst, hipStream_t s) {
  const size_t n = (size_t)c_out * c_in * k;
  if (t == ACT_BF16) hipLaunchKernelGGL(pack_conv_kernel<u16>, dim3(grid_for(n)), dim3(256), 0, s, w, c_out, c_in, k, (u16*)dst);
  else hipLaunchKernelGGL(pack_conv_kernel<float>, dim3(grid_for(n)), dim3(256), 0, s, w, c_out, c_in, k, (float*)dst);
  return hipGetLastError();
}

// Fixed encoder positions: channel c < C/2 holds sin(t * 10000^(-c/(C/2-1))),
// channel C/2 + c the matching cosine; evaluated in double.
__global__ __launch_bounds__(256) void sinusoids_kernel(float* pe, int T, int C) {
  const int half = C / 2;
  const double inc = log(10000.0) / (double)(half - 1);
  const size_t n = (size_t)T * C;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    const int t = (int)(i / C), c = (int)(i - (size_t)t * C);
    const int cc = c < half ? c : c - half;
    const double a = (double)t * exp(-inc * (double)cc);
    pe[i] = (float)(c < half ? sin(a) : cos(a));
  }
}

hipError_t launch_sinusoids(float* pe, int T, int C, hipStream_t s) {
  hipLaunchKernelGGL(sinusoids_kernel, dim3(grid_for((size_t)T * C)), dim3(256), 0, s, pe, T, C);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void fill_f32_kernel(float* dst, float v, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) dst[i] = v;
}
hipError_t launch_fill_f32(float* dst, float v, size_t n, hipStream_t s) {
  if (!n) return hipSuccess;
  hipLaunchKernelGGL(fill_f32_kernel, dim3(grid_for(n)), dim3(256), 0, s, dst, v, n);
  return hipGetLastError();
}
__global__ __launch_bounds__(256) void copy_f32_kernel(const float* src, float* dst, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) dst[i] = src[i];
}
hipError_t launch_copy_f32(const float* src, float* dst, size_t n, hipStream_t s) {
  if (!n) return hipSuccess;
  hipLaunchKernelGGL(copy_f32_kernel, dim3(grid_for(n)), dim3(256), 0, s, src, dst, n);
  return hipGetLastError();
}

// mel [B][n_mels][F] fp32 -> conv1 input [B][F+2][n_mels] (time-major, rows 1..F),
// through a 32x32 LDS tile so both sides stay coalesced.
template <typename T>
__global__ __launch_bounds__(256) void mel_to_conv_kernel(const float* mel, int n_mels, int F, T* x0) {
  __shared__ float tile[32][33];
  const int b = blockIdx.z, t0 = blockIdx.x * 32, m0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const float* src = mel + (size_t)b * n_mels * F;
  for (int r = ty; r < 32; r += 8) {
    const int m = m0 + r, t = t0 + tx;
    tile[r][tx] = (m < n_mels && t < F) ? src[(size_t)m * F + t] : 0.f;
  }
  __syncthreads();
  T* dst = x0 + (size_t)b * (F + 2) * n_mels;
  for (int r = ty; r < 32; r += 8) {
    const int t = t0 + r, m = m0 + tx;
    if (t < F && m < n_mels) dst[(size_t)(t + 1) * n_mels + m] = Act<T>::st(tile[tx][r]);
  }
}

hipError_t launch_mel_to_conv_input(ActType t, const float* mel, int B, int n_mels, int n_frames, void* x0,
                                    hipStream_t s) {
  dim3 grid((n_frames + 31) / 32, (n_mels + 31) / 32, B);
  if (t == ACT_BF16) hipLaunchKernelGGL(mel_to_conv_kernel<u16>, grid, dim3(256), 0, s, mel, n_mels, n_frames, (u16*)x0);
  else hipLaunchKernelGGL(mel_to_conv_kernel<float>, grid, dim3(256), 0, s, mel, n_mels, n_frames, (float*)x0);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  return launch_zero_rows(t, x0, n_mels, n_frames + 2, B, 0, n_frames + 1, s);
}

template <typename T>
__global__ __launch_bounds__(256) void zero_rows_kernel(T* base, long row_elems, long rows_per_batch, int row_a,
                                                        int row_b) {
  const int b = blockIdx.y;
  T* p0 = base + ((long)b * rows_per_batch + row_a) * row_elems;
  T* p1 = base + ((long)b * rows_per_batch + row_b) * row_elems;
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < row_elems; i += (long)gridDim.x * 256) {
    p0[i] = T(0);
    p1[i] = T(0);
  }
}

hipError_t launch_zero_rows(ActType t, void* base, long row_elems, long rows_per_batch, int B, int row_a, int row_b,
                            hipStream_t s) {
  dim3 grid((unsigned)((row_elems + 255) / 256), B);
  if (t == ACT_BF16) hipLaunchKernelGGL(zero_rows_kernel<u16>, grid, dim3(256), 0, s, (u16*)base, row_elems, rows_per_batch, row_a, row_b);
  else hipLaunchKernelGGL(zero_rows_kernel<float>, grid, dim3(256), 0, s, (float*)base, row_elems, rows_per_batch, row_a, row_b);
  return hipGetLastError();
}

// ------------------------------------------------------------------ decoder embedding / argmax
// x[b] = tok_emb[tokens[b]] + pos_emb[lengths[b]] into the fp32 residual stream
// (in a prefill of R tokens per batch row, row b is token b % R of batch row
// b / R, at position lengths[b / R] + b % R).
// Out-of-range token ids or positions write zeros and raise the device error.
// With order, each workgroup also ranks its row among all rows by cache
// length (longest first, lower row first on ties) and writes (row, length)
// at that rank: the dispatch order of the step's self-attention.
template <typename T>
__global__ __launch_bounds__(256) void embed_kernel(const T* tok_emb, const T* pos_emb, const int32_t* tokens,
                                                    const int32_t* lengths, int d, int n_vocab, int n_ctx, int cap,
                                                    float* x, int32_t* dev_error, int32_t* zero, int n_zero,
                                                    int x_tiled, int rows_per_b, int2* order) {
  const int b = blockIdx.x;
  if (b == 0)  // the step's split-K counters start at zero
    for (int i = threadIdx.x; i < n_zero; i += 256) zero[i] = 0;
  if (order) {
    // rows ranked by cache length, longest first (lower row first on ties):
    // order[rank] = (row, length), so the self-attention can dispatch the
    // longest rows first
    __shared__ int s_cnt[4];
    const int B = gridDim.x, nb = lengths[b];
    int c = 0;
    for (int j = threadIdx.x; j < B; j += 256) {
      const int nj = lengths[j];
      c += (nj > nb || (nj == nb && j < b)) ? 1 : 0;
    }
    for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o, 64);
    if ((threadIdx.x & 63) == 0) s_cnt[threadIdx.x >> 6] = c;
    __syncthreads();
    if (threadIdx.x == 0) order[s_cnt[0] + s_cnt[1] + s_cnt[2] + s_cnt[3]] = make_int2(b, nb);
  }
  const int tok = tokens[b], pos = lengths[b / rows_per_b] + b % rows_per_b;
  const bool ok = tok >= 0 && tok < n_vocab && pos >= 0 && pos < n_ctx && pos < cap;
  if (!ok && dev_error && threadIdx.x == 0) *dev_error = (pos >= cap) ? 6 : 1;
  for (int c = threadIdx.x; c < d; c += 256) {
    float v = 0.f;
    if (ok) v = Act<T>::cvt(tok_emb[(size_t)tok * d + c]) + Act<T>::cvt(pos_emb[(size_t)pos * d + c]);
    x[x_tiled ? dec_x_index(b, c, d) : (long)b * d + c] = v;
  }
}

hipError_t launch_embed(ActType t, const void* tok_emb, const void* pos_emb, const int32_t* tokens,
                        const int32_t* lengths, int B, int d, int n_vocab, int n_ctx, int cap, float* x,
                        int32_t* dev_error, hipStream_t s, int32_t* zero, int n_zero, int x_tiled,
                        int rows_per_b, int2* order) {
  if ((x_tiled && d % 32) || rows_per_b < 1 || B % rows_per_b || (order && rows_per_b != 1))
    return hipErrorInvalidValue;
  if (t == ACT_BF16)
    hipLaunchKernelGGL(embed_kernel<u16>, dim3(B), dim3(256), 0, s, (const u16*)tok_emb, (const u16*)pos_emb, tokens,
                       lengths, d, n_vocab, n_ctx, cap, x, dev_error, zero, n_zero, x_tiled, rows_per_b, order);
  else
    hipLaunchKernelGGL(embed_kernel<float>, dim3(B), dim3(256), 0, s, (const float*)tok_emb, (const float*)pos_emb,
                       tokens, lengths, d, n_vocab, n_ctx, cap, x, dev_error, zero, n_zero, x_tiled, rows_per_b,
                       order);
  return hipGetLastError();
}

// Greedy token per row: largest logit, lowest index on ties; then lengths[b] +=
// len_inc (1 per decode step, the prompt length after a prefill).
// 1024 lanes per row with 16-byte loads, so a 51866-wide row is one pass of
// ~13 independent loads per lane.
__global__ __launch_bounds__(1024) void argmax_kernel(const float* logits, int V, int32_t* out, int32_t* lengths,
                                                     int len_inc) {
  const int b = blockIdx.x, tid = threadIdx.x;
  const float* row = logits + (size_t)b * V;
  float best = -INFINITY;
  int idx = 0x7fffffff;
  const bool vec = ((((uintptr_t)row) & 15u) == 0);
  const int nv = vec ? V / 4 : 0;
  for (int i = tid; i < nv; i += 1024) {
    const float4 v = *(const float4*)(row + 4 * i);
    const float a[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (a[k] > best) { best = a[k]; idx = 4 * i + k; }
  }
  for (int i = 4 * nv + tid; i < V; i += 1024) {
    const float v = row[i];
    if (v > best || (v == best && i < idx)) { best = v; idx = i; }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(best, o, 64);
    const int oi = __shfl_xor(idx, o, 64);
    if (ov > best || (ov == best && oi < idx)) { best = ov; idx = oi; }
  }
  __shared__ float sv[16];
  __shared__ int si[16];
  if ((tid & 63) == 0) { sv[tid >> 6] = best; si[tid >> 6] = idx; }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < 16; ++w)
      if (sv[w] > best || (sv[w] == best && si[w] < idx)) { best = sv[w]; idx = si[w]; }
    out[b] = idx == 0x7fffffff ? 0 : idx;
    if (lengths) lengths[b] += len_inc;
  }
}

hipError_t launch_argmax(const float* logits, int B, int V, int32_t* argmax, int32_t* lengths, hipStream_t s,
                         int len_inc) {
  hipLaunchKernelGGL(argmax_kernel, dim3(B), dim3(1024), 0, s, logits, V, argmax, lengths, len_inc);
  return hipGetLastError();
}

// Second stage of the greedy argmax over the per-block maxima the vocabulary
// projection writes ([B][NB] as (float bits, column)): the same rule as
// argmax_kernel (largest value, lowest column on ties, NaN never chosen, 0 for
// a row with no candidate). One workgroup per row.
__global__ __launch_bounds__(1024) void argmax_part_kernel(const int2* part, int NB, int32_t* out, int32_t* lengths,
                                                           int len_inc) {
  const int b = blockIdx.x, tid = threadIdx.x;
  const int2* row = part + (size_t)b * NB;
  float best = -INFINITY;
  int idx = 0x7fffffff;
  for (int i0 = 0; i0 < NB; i0 += 4096) {
    int2 e[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {  // four loads in flight per thread
      const int i = i0 + k * 1024 + tid;
      e[k] = i < NB ? row[i] : make_int2(__float_as_int(-INFINITY), 0x7fffffff);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float v = __int_as_float(e[k].x);
      if (v > best || (v == best && e[k].y < idx)) { best = v; idx = e[k].y; }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(best, o, 64);
    const int oi = __shfl_xor(idx, o, 64);
    if (ov > best || (ov == best && oi < idx)) { best = ov; idx = oi; }
  }
  __shared__ float sv[16];
  __shared__ int si[16];
  if ((tid & 63) == 0) { sv[tid >> 6] = best; si[tid >> 6] = idx; }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < 16; ++w)
      if (sv[w] > best || (sv[w] == best && si[w] < idx)) { best = sv[w]; idx = si[w]; }
    out[b] = idx == 0x7fffffff ? 0 : idx;
    if (lengths) lengths[b] += len_inc;
  }
}

hipError_t launch_argmax_part(const int2* part, int B, int NB, int32_t* argmax, int32_t* lengths, hipStream_t s,
                              int len_inc) {
  if (B <= 0 || NB <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(argmax_part_kernel, dim3(B), dim3(1024), 0, s, part, NB, argmax, lengths, len_inc);
  return hipGetLastError();
}

// Row-major fp32 rows <-> the 16-row tiles of dec_x_index (one workgroup per row).
__global__ __launch_bounds__(256) void x_tiles_kernel(const float* src, float* dst, int d, int to_tiles) {
  const long m = blockIdx.x;
  for (int c = threadIdx.x; c < d; c += 256) {
    if (to_tiles) dst[dec_x_index(m, c, d)] = src[m * d + c];
    else dst[m * d + c] = src[dec_x_index(m, c, d)];
  }
}

hipError_t launch_x_tiles(const float* src, float* dst, int M, int d, int to_tiles, hipStream_t s) {
  if (M <= 0 || d <= 0 || d % 32) return hipErrorInvalidValue;
  hipLaunchKernelGGL(x_tiles_kernel, dim3(M), dim3(256), 0, s, src, dst, d, to_tiles);
  return hipGetLastError();
}

// Last position of each batch row of a prefill: x_dst row b = x_src row
// b * R + R - 1, both in the 16-row tiles of dec_x_index.
__global__ __launch_bounds__(256) void gather_last_rows_kernel(const float* x_src, float* x_dst, int R, int d) {
  const int b = blockIdx.x;
  for (int c = threadIdx.x; c < d; c += 256) x_dst[dec_x_index(b, c, d)] = x_src[dec_x_index((long)b * R + R - 1, c, d)];
}

hipError_t launch_gather_last_rows(const float* x_src, float* x_dst, int B, int R, int d, hipStream_t s) {
  if (B <= 0 || R < 1 || d % 32) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gather_last_rows_kernel, dim3(B), dim3(256), 0, s, x_src, x_dst, R, d);
  return hipGetLastError();
}

}  // namespace wh
