// Resampling to 16 kHz on gfx950 (MI355X): band-limited interpolation with a
// Kaiser-windowed sinc. Output sample n of a clip sits at input position
// p = n R / 16000 = q + phi / L (R / 16000 = M / L in lowest terms, q integer,
// 0 <= phi < L), and is the dot product of the clip's samples
// x[q - J .. q + J] (zero outside the clip) with the phi-th row of taps,
// taps[phi][j] = h(phi / L + J - j). The host builds the taps (fp64 math,
// rounded once to fp32); see logmel_api.cpp.
//
// logmel_resample_kernel: a persistent grid of 1024-thread workgroups, one
// per compute unit. A workgroup copies the taps table into LDS once, then
// walks blocks of 1024 consecutive outputs of the packed batch, one output
// per thread. For each block it stages the input samples the block's
// windows cover (one coalesced pass; int16 PCM is converted to s / 32768 on
// the way) and every thread forms its dot product from LDS, in fp32 with
// four partial sums. Clips are packed back to back, so the block's windows
// always cover one contiguous range of the batch even when the block spans
// clips; a thread whose window crosses its clip's edge masks the samples
// outside the clip.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "logmel_launch.h"

namespace logmel {

static constexpr int kResThreads = kResThreadsHost;

__device__ __forceinline__ float res_sample(const float* p, int64_t k) { return p[k]; }
__device__ __forceinline__ float res_sample(const int16_t* p, int64_t k) {
  return (float)p[k] * (1.0f / 32768.0f);
}

// Last index c in [0, n) with a[c] <= v (a non-decreasing, a[0] <= v).
__device__ __forceinline__ int64_t last_le(const int64_t* __restrict__ a, int64_t n, int64_t v) {
  int64_t lo = 0, hi = n;   // answer in [lo, hi)
  while (hi - lo > 1) {
    const int64_t mid = lo + ((hi - lo) >> 1);
    if (a[mid] <= v) lo = mid; else hi = mid;
  }
  return lo;
}

template <typename In>
__device__ __forceinline__ void resample_body(const In* __restrict__ x,
                                              const int64_t* __restrict__ in_off,
                                              const int64_t* __restrict__ out_off,
                                              int64_t n_clips, int64_t total_out,
                                              float* __restrict__ y,
                                              const float* __restrict__ taps, int L, int M, int J,
                                              int span_cap, float* lds, int64_t* bounds) {
  const int tid = threadIdx.x;
  const int T = 2 * J + 1;
  const int tab_len = L * T;
  float* tab = lds;
  float* span = lds + ((tab_len + 3) & ~3);
  for (int i = tid; i < tab_len; i += kResThreads) tab[i] = taps[i];
  const int64_t total_in = in_off[n_clips];

  for (int64_t g0 = (int64_t)blockIdx.x * kResThreads; g0 < total_out;
       g0 += (int64_t)gridDim.x * kResThreads) {
    const int64_t g = g0 + tid;
    const bool active = g < total_out;
    const int64_t gq = active ? g : total_out - 1;
    // the output's clip (clips without samples have no outputs and are
    // skipped: their out_off entry equals the next one)
    const int64_t c = last_le(out_off, n_clips, gq);
    const int64_t n = gq - out_off[c];
    const int64_t nm = n * M;
    const int64_t q = nm / L;
    const int phi = (int)(nm - q * L);
    const int64_t lo = in_off[c], hi = in_off[c + 1];
    const int64_t k0 = lo + q - J;            // global index of tap 0's sample
    // The block's windows: from thread 0's first sample to the last active
    // thread's last (window starts never decrease along the packed outputs).
    const int last = (int)min((int64_t)kResThreads, total_out - g0) - 1;
    __syncthreads();                          // the previous block's span is consumed
    if (tid == 0) bounds[0] = k0;
    if (tid == last) bounds[1] = k0 + T;
    __syncthreads();
    const int64_t s0 = bounds[0];
    const int span_len = (int)min(bounds[1] - s0, (int64_t)span_cap);
    for (int i = tid; i < span_len; i += kResThreads) {
      const int64_t k = s0 + i;
      span[i] = (k >= 0 && k < total_in) ? res_sample(x, k) : 0.0f;
    }
    __syncthreads();
    if (!active) continue;
    const int64_t off = k0 - s0;
    const float* tp = tab + phi * T;
    float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
    if (off >= 0 && off + T <= span_len) {
      const float* sp = span + off;
      if (k0 >= lo && k0 + T <= hi) {
        // the whole window inside the clip
        int j = 0;
        for (; j + 4 <= T; j += 4) {
          a0 = __builtin_fmaf(tp[j], sp[j], a0);
          a1 = __builtin_fmaf(tp[j + 1], sp[j + 1], a1);
          a2 = __builtin_fmaf(tp[j + 2], sp[j + 2], a2);
          a3 = __builtin_fmaf(tp[j + 3], sp[j + 3], a3);
        }
        for (; j < T; ++j) a0 = __builtin_fmaf(tp[j], sp[j], a0);
      } else {
        // a clip edge inside the window: samples outside the clip are zero
        const int jlo = (int)max((int64_t)0, lo - k0);
        const int jhi = (int)min((int64_t)T, hi - k0);
        for (int j = jlo; j < jhi; ++j) a0 = __builtin_fmaf(tp[j], sp[j], a0);
      }
    } else {
      // not reached for packed offsets (the span covers every window); kept
      // as a correct path from global memory
      const int jlo = (int)max((int64_t)0, lo - k0);
      const int jhi = (int)min((int64_t)T, hi - k0);
      for (int j = jlo; j < jhi; ++j) a0 = __builtin_fmaf(tp[j], res_sample(x, k0 + j), a0);
    }
    y[g] = (a0 + a1) + (a2 + a3);
  }
}

#define LOGMEL_RESAMPLE_KERNEL(NAME, IN)                                                         \
  extern "C" __global__ void __launch_bounds__(kResThreads)                                      \
  NAME(const IN* __restrict__ x, const int64_t* __restrict__ in_off,                             \
       const int64_t* __restrict__ out_off, int64_t n_clips, int64_t total_out,                   \
       float* __restrict__ y, const float* __restrict__ taps, int L, int M, int J,                \
       int span_cap) {                                                                           \
    __shared__ float lds[kResLdsFloats];                                                         \
    __shared__ int64_t bounds[2];                                                                \
    resample_body<IN>(x, in_off, out_off, n_clips, total_out, y, taps, L, M, J, span_cap, lds,   \
                      bounds);                                                                   \
  }

LOGMEL_RESAMPLE_KERNEL(logmel_resample_kernel, float)
LOGMEL_RESAMPLE_KERNEL(logmel_resample_i16_kernel, int16_t)

}  // namespace logmel

hipError_t logmel_launch_resample(const void* x, int in_i16, const int64_t* in_off,
                                  const int64_t* out_off, int64_t n_clips, int64_t total_out,
                                  float* y, const float* taps, int L, int M, int J, int span_cap,
                                  int grid, hipStream_t stream) {
  if (total_out <= 0) return hipSuccess;
  const int64_t blocks = (total_out + logmel::kResThreads - 1) / logmel::kResThreads;
  const int g = (int)(blocks < grid ? blocks : grid);
  if (in_i16)
    hipLaunchKernelGGL(logmel::logmel_resample_i16_kernel, dim3(g), dim3(logmel::kResThreads), 0,
                       stream, static_cast<const int16_t*>(x), in_off, out_off, n_clips,
                       total_out, y, taps, L, M, J, span_cap);
  else
    hipLaunchKernelGGL(logmel::logmel_resample_kernel, dim3(g), dim3(logmel::kResThreads), 0,
                       stream, static_cast<const float*>(x), in_off, out_off, n_clips, total_out,
                       y, taps, L, M, J, span_cap);
  return hipGetLastError();
}
