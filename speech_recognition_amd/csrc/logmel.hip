// Log-mel front end on the GPU (whisper_blaze showcase page, "The Approach":
// the mel spectrogram moves off the CPU; "The Solution", mel_spectrogram.cu
// card: STFT, 128-bin mel filterbank). Here the STFT is a direct 400-point DFT
// in fp32: 400 = 2^4 * 5^2 is not a power of two, and at 16 frames per
// workgroup every twiddle read from LDS feeds 32 FMAs. The twiddle index
// (k * n) mod 400 is tracked exactly in integers, so no phase error builds up.
//
// Reading of the parameters (the pages give none): 16 kHz, 400-sample
// periodic Hann frames, hop 160, centre framing with reflect padding of 200,
// 3000 frames per 30 s chunk (the 3001st dropped); 201-bin power spectrum;
// Slaney mel filters 0-8 kHz with area normalisation; log10 with a 1e-10
// floor; values clamped to (chunk maximum - 8) and mapped by (x + 4) / 4.
#include "common.hpp"
#include "internal.hpp"

namespace wh {

constexpr int NFFT = 400, HOPL = 160, NBIN = 201, NFR = 3000, NSAMP = 480000, FT = 16;
constexpr int NBLK = (NFR + FT - 1) / FT;

// workspace (floats): cos[400] sin[400] win[400] fb[n_mels][201] lo[n_mels] hi[n_mels] blockmax[B][NBLK]
__host__ __device__ static size_t fb_off() { return 3 * NFFT; }
__host__ __device__ static size_t lohi_off(int n_mels) { return fb_off() + (size_t)n_mels * NBIN; }
__host__ __device__ static size_t bmax_off(int n_mels) { return lohi_off(n_mels) + 2 * (size_t)n_mels; }
size_t logmel_ws(int B, int n_mels) { return (bmax_off(n_mels) + (size_t)B * NBLK) * sizeof(float); }

__device__ double hz_to_mel_d(double f) {
  const double f_sp = 200.0 / 3.0, min_log_hz = 1000.0, min_log_mel = min_log_hz / f_sp;
  const double logstep = log(6.4) / 27.0;
  return f >= min_log_hz ? min_log_mel + log(f / min_log_hz) / logstep : f / f_sp;
}
__device__ double mel_to_hz_d(double m) {
  const double f_sp = 200.0 / 3.0, min_log_hz = 1000.0, min_log_mel = min_log_hz / f_sp;
  const double logstep = log(6.4) / 27.0;
  return m >= min_log_mel ? min_log_hz * exp(logstep * (m - min_log_mel)) : f_sp * m;
}

// Tables in double, stored as fp32: twiddles, periodic Hann window, and the
// triangular Slaney filters with each filter's non-zero bin range.
__global__ __launch_bounds__(256) void logmel_setup(float* ws, int n_mels) {
  const int tid = blockIdx.x * 256 + threadIdx.x;
  const double two_pi = 6.283185307179586476925;
  if (tid < NFFT) {
    const double a = two_pi * tid / NFFT;
    ws[tid] = (float)cos(a);
    ws[NFFT + tid] = (float)sin(a);
    ws[2 * NFFT + tid] = (float)(0.5 - 0.5 * cos(a));
  }
  if (tid < n_mels) {
    const int m = tid;
    const double mmax = hz_to_mel_d(8000.0);
    const double lo = mel_to_hz_d(mmax * m / (n_mels + 1));
    const double c = mel_to_hz_d(mmax * (m + 1) / (n_mels + 1));
    const double hi = mel_to_hz_d(mmax * (m + 2) / (n_mels + 1));
    const double norm = 2.0 / (hi - lo);
    int klo = NBIN, khi = -1;
    float* fb = ws + fb_off() + (size_t)m * NBIN;
    for (int k = 0; k < NBIN; ++k) {
      const double f = k * 16000.0 / NFFT;
      double w = fmin((f - lo) / (c - lo), (hi - f) / (hi - c));
      w = w > 0.0 ? w * norm : 0.0;
      fb[k] = (float)w;
      if (w > 0.0) { klo = min(klo, k); khi = max(khi, k); }
    }
    int* lohi = (int*)(ws + lohi_off(n_mels));
    lohi[2 * m] = klo;
    lohi[2 * m + 1] = khi;
  }
}

// Chunk b starts at audio + b * row_stride and holds n_valid(b) = min(n_samples,
// total - b * row_stride) samples, zero beyond (row_stride = n_samples, total =
// B * n_samples for separate clips; a stride below 30 s for overlapping chunks
// of one long recording).
__global__ __launch_bounds__(256) void logmel_frames(const float* __restrict__ audio, int n_samples, long row_stride,
                                                     long total, int n_mels, const float* __restrict__ ws,
                                                     float* __restrict__ mel_out, float* __restrict__ bmax) {
  __shared__ float xs[FT][NFFT];
  __shared__ float cs[NFFT], sn[NFFT];
  __shared__ float pw[FT][NBIN + 3];
  __shared__ float wm[4];
  const int b = blockIdx.y, f0 = blockIdx.x * FT, tid = threadIdx.x;
  const float* a = audio + (size_t)b * row_stride;
  const long n_valid = min((long)n_samples, total - (long)b * row_stride);
  for (int i = tid; i < NFFT; i += 256) { cs[i] = ws[i]; sn[i] = ws[NFFT + i]; }
  for (int i = tid; i < FT * NFFT; i += 256) {
    const int f = i / NFFT, n = i - f * NFFT;
    int s = (f0 + f) * HOPL + n - NFFT / 2;
    if (s < 0) s = -s;
    if (s >= NSAMP) s = 2 * (NSAMP - 1) - s;
    const float v = (s < n_valid) ? a[s] : 0.f;
    xs[f][n] = v * ws[2 * NFFT + n];
  }
  __syncthreads();
  if (tid < NBIN) {
    const int k = tid;
    float re[FT], im[FT];
#pragma unroll
    for (int f = 0; f < FT; ++f) { re[f] = 0.f; im[f] = 0.f; }
    int idx = 0;
    for (int n = 0; n < NFFT; ++n) {
      const float c = cs[idx], s = sn[idx];
#pragma unroll
      for (int f = 0; f < FT; ++f) {
        const float x = xs[f][n];
        re[f] = fmaf(x, c, re[f]);
        im[f] = fmaf(-x, s, im[f]);
      }
      idx += k;
      if (idx >= NFFT) idx -= NFFT;
    }
#pragma unroll
    for (int f = 0; f < FT; ++f) pw[f][k] = re[f] * re[f] + im[f] * im[f];
  }
  __syncthreads();
  const float* fb = ws + fb_off();
  const int* lohi = (const int*)(ws + lohi_off(n_mels));
  float lmax = -INFINITY;
  for (int o = tid; o < FT * n_mels; o += 256) {
    const int m = o / FT, f = o - m * FT;
    const int t = f0 + f;
    if (t >= NFR) continue;
    const int klo = lohi[2 * m], khi = lohi[2 * m + 1];
    float acc = 0.f;
    for (int k = klo; k <= khi; ++k) acc = fmaf(fb[(size_t)m * NBIN + k], pw[f][k], acc);
    const float v = log10f(fmaxf(acc, 1e-10f));
    mel_out[((size_t)b * n_mels + m) * NFR + t] = v;
    lmax = fmaxf(lmax, v);
  }
  lmax = wave_max(lmax);
  if ((tid & 63) == 0) wm[tid >> 6] = lmax;
  __syncthreads();
  if (tid == 0) bmax[(size_t)b * NBLK + blockIdx.x] = fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3]));
}

__global__ __launch_bounds__(256) void logmel_finalize(float* __restrict__ mel_out, const float* __restrict__ bmax,
                                                       int n_mels) {
  __shared__ float wm[4];
  const int b = blockIdx.y, tid = threadIdx.x;
  float mx = -INFINITY;
  for (int i = tid; i < NBLK; i += 256) mx = fmaxf(mx, bmax[(size_t)b * NBLK + i]);
  mx = wave_max(mx);
  if ((tid & 63) == 0) wm[tid >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3]));
  const float floor_ = mx - 8.0f;
  const size_t n = (size_t)n_mels * NFR;
  float* p = mel_out + (size_t)b * n;
  for (size_t i = (size_t)blockIdx.x * 256 + tid; i < n; i += (size_t)gridDim.x * 256)
    p[i] = (fmaxf(p[i], floor_) + 4.0f) * 0.25f;
}

hipError_t launch_logmel(const float* audio, int B, int n_samples, int n_mels, float* mel_out, void* ws_,
                         hipStream_t s, long row_stride, long total) {
  float* ws = (float*)ws_;
  if (row_stride <= 0) { row_stride = n_samples; total = (long)B * n_samples; }
  hipLaunchKernelGGL(logmel_setup, dim3((NFFT + 255) / 256), dim3(256), 0, s, ws, n_mels);
  hipLaunchKernelGGL(logmel_frames, dim3(NBLK, B), dim3(256), 0, s, audio, n_samples, row_stride, total, n_mels, ws,
                     mel_out, ws + bmax_off(n_mels));
  hipLaunchKernelGGL(logmel_finalize, dim3(64, B), dim3(256), 0, s, mel_out, ws + bmax_off(n_mels), n_mels);
  return hipGetLastError();
}

}  // namespace wh
