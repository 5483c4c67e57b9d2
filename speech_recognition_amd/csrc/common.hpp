// Device helpers shared by the gfx950 kernels of the Whisper hot path:
// bf16 / OCP fp8 (E4M3, E5M2) conversions done on bits, MFMA operand vector
// types and wave64 reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.hpp"

namespace wh {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint16_t u16;

constexpr int WAVE = 64;

// ------------------------------------------------------------------ bf16 storage
__device__ __forceinline__ float bf2f(u16 b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ u16 f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u16)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (u16)(u >> 16);
}

// Two fp32 -> packed bf16 pair with the gfx950 converter (round to nearest
// even, like f2bf on non-NaN inputs): low half from a, high half from b.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f2bf2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// Storage type traits: activations are bf16 (u16 bits) or fp32.
template <typename T> struct Act;
template <> struct Act<u16> {
  static __device__ __forceinline__ float ld(const u16* p) { return bf2f(*p); }
  static __device__ __forceinline__ float cvt(u16 v) { return bf2f(v); }
  static __device__ __forceinline__ u16 st(float v) { return f2bf(v); }
  static __device__ __forceinline__ float round(float v) { return bf2f(f2bf(v)); }
};
template <> struct Act<float> {
  static __device__ __forceinline__ float ld(const float* p) { return *p; }
  static __device__ __forceinline__ float cvt(float v) { return v; }
  static __device__ __forceinline__ float st(float v) { return v; }
  static __device__ __forceinline__ float round(float v) { return v; }
};

// ------------------------------------------------------------------ OCP E4M3FN
// 1 sign, 4 exponent bits (bias 7), 3 mantissa bits; no infinities; S.1111.111
// is NaN; largest finite magnitude 448. Encoding rounds to nearest even and
// saturates magnitudes >= 448 to +-448; the sign bit is always kept.
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7fu;          // NaN
  if (a >= 0x43e00000u) return sign | 0x7eu;         // |y| >= 448: saturate
  if (a < 0x3c800000u) {                             // |y| < 2^-6: subnormal, step 2^-9
    const float s = __uint_as_float(a) * 512.0f;     // exact scaling by a power of two
    return sign | (uint32_t)__builtin_rintf(s);      // 0..8 (8 is the smallest normal)
  }
  const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);  // round 23 -> 3 mantissa bits, ties to even
  uint32_t code = (((r >> 23) - 120u) << 3) | ((r >> 20) & 7u);
  return sign | (code > 0x7eu ? 0x7eu : code);
}

// Four codes packed in a word -> fp32 with the gfx950 converter (OCP E4M3FN,
// NaN for S.1111.111), two codes per instruction.
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void e4m3x4_decode(uint32_t w, float o[4]) {
  const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  o[0] = lo[0]; o[1] = lo[1]; o[2] = hi[0]; o[3] = hi[1];
}

// Scalar decode from the bit fields (reference form of the same mapping).
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
  if ((c & 0x7fu) == 0x7fu) v = __uint_as_float(0x7fc00000u);
  return (c & 0x80u) ? -v : v;
}

// ------------------------------------------------------------------ OCP E5M2
// 1 sign, 5 exponent bits (bias 15), 2 mantissa bits: IEEE binary16's top
// byte, with +-inf (S.11111.00) and NaN (S.11111.xx, xx != 0); largest finite
// magnitude 57344. Encoding rounds to nearest even and saturates magnitudes
// >= 57344, infinities included, to +-57344; the sign bit is always kept.
__device__ __forceinline__ uint32_t e5m2_encode(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7fu;          // NaN
  if (a >= 0x47600000u) return sign | 0x7bu;         // |y| >= 57344: saturate
  if (a < 0x38800000u) {                             // |y| < 2^-14: subnormal, step 2^-16
    const float s = __uint_as_float(a) * 65536.0f;   // exact scaling by a power of two
    return sign | (uint32_t)__builtin_rintf(s);      // 0..4 (4 is the smallest normal)
  }
  const uint32_t r = a + 0xfffffu + ((a >> 21) & 1u);  // round 23 -> 2 mantissa bits, ties to even
  uint32_t code = (((r >> 23) - 112u) << 2) | ((r >> 21) & 3u);
  return sign | (code > 0x7bu ? 0x7bu : code);
}

// Four E5M2 codes packed in a word -> fp32 with the gfx950 converter.
__device__ __forceinline__ void e5m2x4_decode(uint32_t w, float o[4]) {
  const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_bf8((int)w, false);
  const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_bf8((int)w, true);
  o[0] = lo[0]; o[1] = lo[1]; o[2] = hi[0]; o[3] = hi[1];
}

// The two fp8 formats as one template parameter (Fp8Fmt, internal.hpp).
template <int FMT>
__device__ __forceinline__ uint32_t fp8_encode(float y) {
  return FMT == FP8_E5M2 ? e5m2_encode(y) : e4m3_encode(y);
}
template <int FMT>
__device__ __forceinline__ void fp8x4_decode(uint32_t w, float o[4]) {
  if (FMT == FP8_E5M2) e5m2x4_decode(w, o);
  else e4m3x4_decode(w, o);
}
template <int FMT>
constexpr float fp8_max() { return FMT == FP8_E5M2 ? 57344.0f : 448.0f; }

// ------------------------------------------------------------------ decoder residual tiles
// The fused decode step keeps its fp32 residual stream x [M, d] (M padded to
// a multiple of 16, d % 32 == 0) in 16-row tiles laid out for the A operand
// of a 16x16x32 MFMA: per 16 rows and 32 columns a 2 KB block holding two
// 1 KB halves, each lane-ordered (lane = 16 * ((k % 32) / 8) + m % 16, four
// consecutive k), so a wave's operand load is one contiguous 1 KB read.
__host__ __device__ __forceinline__ long dec_x_index(long m, long k, long d) {
  return ((((m >> 4) * (d >> 5) + (k >> 5)) * 2 + ((k & 7) >> 2)) * 64 + ((k & 31) >> 3) * 16 + (m & 15)) * 4 + (k & 3);
}

// ------------------------------------------------------------------ reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// GELU(x) = x Phi(x) = 0.5 x erfc(-x / sqrt 2), with erfc(z), z >= 0, from the
// rational approximation of Abramowitz & Stegun, Handbook of Mathematical
// Functions, formula 7.1.26 (|error in erf| <= 1.5e-7): erfc(z) = t (a1 + t (a2
// + t (a3 + t (a4 + t a5)))) exp(-z^2), t = 1 / (1 + p z). Used in the
// complementary form on both sides of 0, so negative x needs no cancellation:
// x >= 0: x - 0.5 x erfc(z); x < 0: 0.5 x erfc(z), z = |x| / sqrt 2. In fp32
// the GELU's absolute error is <= 3.4e-7, far below the bf16 rounding of its
// output.
__device__ __forceinline__ float gelu_erf(float x) {
  const float z = fabsf(x) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, z, 1.0f));
  const float poly =
      t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, 1.061405429f, -1.453152027f), 1.421413741f), -0.284496736f), 0.254829592f);
  const float q = poly * __builtin_amdgcn_exp2f(-z * z * 1.4426950408889634f);
  const float hx = 0.5f * x * q;
  return x >= 0.f ? x - hx : hx;
}

template <typename To, typename From>
__device__ __forceinline__ To bitcast(const From& f) { return __builtin_bit_cast(To, f); }

}  // namespace wh
