// Measured ceilings for the roofline: the rate the part sustains for bf16
// MFMA with operands resident in registers, and for streaming reads of a
// buffer far larger than the last-level cache. The bench reports its kernel
// rates against these as well as against the vendor peaks.
#include "common.hpp"
#include "internal.hpp"

namespace wh {

// Each wave runs `iters` rounds of 16 independent MFMA 16x16x32 bf16 on
// register operands (varied bit patterns, as real data toggles the
// multipliers) and writes one float so the work stays live.
constexpr int PEAK_CHAINS = 16;

__global__ __launch_bounds__(256) void peak_mfma_kernel(int iters, float* out) {
  const int lane = threadIdx.x & 63;
  const uint32_t seed = (blockIdx.x * 256u + threadIdx.x) * 2654435761u;
  uint4 ua, ub;
  ua.x = seed ^ 0x3f1e9c4bu; ua.y = seed * 3u ^ 0x40a1b2c3u; ua.z = seed * 7u ^ 0xbf3c4d5eu; ua.w = seed * 11u ^ 0x3e8f9a0bu;
  ub.x = seed * 13u ^ 0x3fd1e2f3u; ub.y = seed * 17u ^ 0xbe04a5b6u; ub.z = seed * 19u ^ 0x3f6c7d8eu; ub.w = seed * 23u ^ 0x40192a3bu;
  // keep exponents moderate: clear the top exponent bits of every bf16
  ua.x &= 0xbfffbfffu; ua.y &= 0xbfffbfffu; ua.z &= 0xbfffbfffu; ua.w &= 0xbfffbfffu;
  ub.x &= 0xbfffbfffu; ub.y &= 0xbfffbfffu; ub.z &= 0xbfffbfffu; ub.w &= 0xbfffbfffu;
  const bf16x8 a = bitcast<bf16x8>(ua), b = bitcast<bf16x8>(ub);
  f32x4 acc[PEAK_CHAINS];
#pragma unroll
  for (int c = 0; c < PEAK_CHAINS; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < PEAK_CHAINS; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < PEAK_CHAINS; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  if (lane == 0) out[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

// Grid-stride 16-byte loads over the whole buffer; one float per workgroup.
__global__ __launch_bounds__(256) void peak_read_kernel(const uint4* __restrict__ buf, size_t n16, float* out) {
  uint32_t x = 0;
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {  // four loads in flight per lane
    const uint4 v0 = buf[i], v1 = buf[i + stride], v2 = buf[i + 2 * stride], v3 = buf[i + 3 * stride];
    x ^= v0.x ^ v0.y ^ v0.z ^ v0.w ^ v1.x ^ v1.y ^ v1.z ^ v1.w ^ v2.x ^ v2.y ^ v2.z ^ v2.w ^ v3.x ^ v3.y ^ v3.z ^ v3.w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = buf[i];
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  __shared__ uint32_t red[4];
  for (int o = 32; o > 0; o >>= 1) x ^= (uint32_t)__shfl_xor((int)x, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = (float)(red[0] ^ red[1] ^ red[2] ^ red[3]);
}

hipError_t launch_peak_mfma(int n_wg, int iters, float* out, hipStream_t s) {
  if (n_wg <= 0 || iters <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(peak_mfma_kernel, dim3(n_wg), dim3(256), 0, s, iters, out);
  return hipGetLastError();
}

hipError_t launch_peak_read(const void* buf, size_t bytes, int n_wg, float* out, hipStream_t s) {
  if (n_wg <= 0 || bytes < 16) return hipErrorInvalidValue;
  hipLaunchKernelGGL(peak_read_kernel, dim3(n_wg), dim3(256), 0, s, (const uint4*)buf, bytes / 16, out);
  return hipGetLastError();
}

double peak_mfma_flop(int n_wg, int iters) { return (double)n_wg * 4 * iters * PEAK_CHAINS * (2.0 * 16 * 16 * 32); }

}  // namespace wh
