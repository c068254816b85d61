// The streaming push, step 1 (gfx950), and the same for streams that are
// resampled to 16 kHz first (logmel_rstream_prep_kernel, below).
//
// logmel_stream_prep_kernel moves each stream's carry (the
// samples of its next, not yet complete frame) to sit right before the new
// samples in the stream's workspace row, and appends the new samples
// (fp32, or int16 PCM converted to s / 32768, exact). The frames are then
// computed by logmel_tiles_kernel over the per-stream segments, so a
// streamed frame is bit-for-bit the offline frame of the same samples.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "logmel_launch.h"
#include "logmel_resample_launch.h"

namespace logmel {

__device__ __forceinline__ float stream_sample(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float stream_sample(const int16_t* p, int64_t i) {
  return (float)p[i] * (1.0f / 32768.0f);
}

// One workgroup per stream. meta (int64, n = n_streams) is the host's
// staging slot, read by the device in place (pinned host memory):
//   [0n, 1n)  carry source index in ws (absolute)
//   [1n, 2n)  carry length (< 400)
//   [2n, 3n)  offset of the stream's new samples in `fresh`
//   [3n, 4n)  number of new samples
//   [4n, 5n)  segment start in ws  (= row base + 400 - carry length)
//   [5n, 6n)  segment end in ws    (= row base + 400 + new samples)
//   [6n, 7n+1) output frame offsets
// The kernel copies [4n, 7n + 1) into meta_dev, where the transform kernel
// that follows reads them.
template <typename In>
__device__ __forceinline__ void stream_prep_body(float* __restrict__ ws, int64_t row_stride,
                                                 const In* __restrict__ fresh,
                                                 const int64_t* __restrict__ meta,
                                                 int64_t* __restrict__ meta_dev,
                                                 int64_t n_streams) {
  const int64_t j = blockIdx.x;
  const int t = threadIdx.x;
  const int64_t base = j * row_stride;
  const int64_t src = meta[j];
  const int64_t clen = meta[n_streams + j];
  const int64_t noff = meta[2 * n_streams + j];
  const int64_t nlen = meta[3 * n_streams + j];
  // the transform kernel's inputs: segment start and end, frame offsets
  if (t == 0) meta_dev[4 * n_streams + j] = meta[4 * n_streams + j];
  if (t == 1) meta_dev[5 * n_streams + j] = meta[5 * n_streams + j];
  if (t == 2) meta_dev[6 * n_streams + j + 1] = meta[6 * n_streams + j + 1];
  if (t == 3 && j == 0) meta_dev[6 * n_streams] = meta[6 * n_streams];
  // The carry can overlap its destination, and the new samples land where
  // the old ones were: read the carry and the first new samples before any
  // write.
  float c0 = 0.f, c1 = 0.f;
  if (t < clen) c0 = ws[src + t];
  if (t + 256 < clen) c1 = ws[src + t + 256];
  const In* in = fresh + noff;
  constexpr int kBatch = 8;
  float v[kBatch];
#pragma unroll
  for (int u = 0; u < kBatch; ++u) {
    const int64_t i = t + 256 * u;
    v[u] = i < nlen ? stream_sample(in, i) : 0.0f;
  }
  __syncthreads();
  const int64_t dst = base + 400 - clen;
  if (t < clen) ws[dst + t] = c0;
  if (t + 256 < clen) ws[dst + t + 256] = c1;
  float* row = ws + base + 400;
#pragma unroll
  for (int u = 0; u < kBatch; ++u) {
    const int64_t i = t + 256 * u;
    if (i < nlen) row[i] = v[u];
  }
  for (int64_t i = t + 256 * kBatch; i < nlen; i += 256) row[i] = stream_sample(in, i);
}

extern "C" __global__ void __launch_bounds__(256)
logmel_stream_prep_kernel(float* __restrict__ ws, int64_t row_stride,
                          const float* __restrict__ fresh, const int64_t* __restrict__ meta,
                          int64_t* __restrict__ meta_dev, int64_t n_streams) {
  stream_prep_body(ws, row_stride, fresh, meta, meta_dev, n_streams);
}

extern "C" __global__ void __launch_bounds__(256)
logmel_stream_prep_i16_kernel(float* __restrict__ ws, int64_t row_stride,
                              const int16_t* __restrict__ fresh, const int64_t* __restrict__ meta,
                              int64_t* __restrict__ meta_dev, int64_t n_streams) {
  stream_prep_body(ws, row_stride, fresh, meta, meta_dev, n_streams);
}

// A resampling stream's push, step 1: one workgroup per stream builds its
// segment in dst: the retained input samples (from the previous push's
// buffer src), then the new ones (fp32, or int16 PCM as s / 32768). meta is
// the host's staging slot (pinned host memory, read in place), layout as in
// the host's rs_push: [0n) carry index in src, [1n) carry length, [2n)
// offset of the new samples, [3n) their number, [4n) segment start in dst,
// then [5n, 9n + 1) the resampling kernel's segment arrays, which the
// kernel copies into meta_dev.
template <typename In>
__device__ __forceinline__ void rstream_prep_body(float* __restrict__ dst,
                                                  const float* __restrict__ src,
                                                  const In* __restrict__ fresh,
                                                  const int64_t* __restrict__ meta,
                                                  int64_t* __restrict__ meta_dev,
                                                  int64_t n_streams) {
  const int64_t j = blockIdx.x;
  const int t = threadIdx.x;
  const int64_t csrc = meta[j];
  const int64_t clen = meta[n_streams + j];
  const int64_t noff = meta[2 * n_streams + j];
  const int64_t nlen = meta[3 * n_streams + j];
  // the resampling kernel's inputs: segment origin, end, first output
  // number and output offsets
  if (t == 0) meta_dev[5 * n_streams + j] = meta[5 * n_streams + j];
  if (t == 1) meta_dev[6 * n_streams + j] = meta[6 * n_streams + j];
  if (t == 2) meta_dev[7 * n_streams + j] = meta[7 * n_streams + j];
  if (t == 3) meta_dev[8 * n_streams + j + 1] = meta[8 * n_streams + j + 1];
  if (t == 4 && j == 0) meta_dev[8 * n_streams] = meta[8 * n_streams];
  float* seg = dst + meta[4 * n_streams + j];
  for (int64_t i = t; i < clen; i += 256) seg[i] = src[csrc + i];
  for (int64_t i = t; i < nlen; i += 256) seg[clen + i] = stream_sample(fresh + noff, i);
}

extern "C" __global__ void __launch_bounds__(256)
logmel_rstream_prep_kernel(float* __restrict__ dst, const float* __restrict__ src,
                           const float* __restrict__ fresh, const int64_t* __restrict__ meta,
                           int64_t* __restrict__ meta_dev, int64_t n_streams) {
  rstream_prep_body(dst, src, fresh, meta, meta_dev, n_streams);
}

extern "C" __global__ void __launch_bounds__(256)
logmel_rstream_prep_i16_kernel(float* __restrict__ dst, const float* __restrict__ src,
                               const int16_t* __restrict__ fresh,
                               const int64_t* __restrict__ meta, int64_t* __restrict__ meta_dev,
                               int64_t n_streams) {
  rstream_prep_body(dst, src, fresh, meta, meta_dev, n_streams);
}

}  // namespace logmel

hipError_t logmel_launch_rstream_prep(float* dst, const float* src, const void* fresh, int in_i16,
                                      const int64_t* meta, int64_t* meta_dev, int64_t n_streams,
                                      hipStream_t stream) {
  if (n_streams <= 0) return hipSuccess;
  if (in_i16)
    hipLaunchKernelGGL(logmel::logmel_rstream_prep_i16_kernel, dim3((unsigned)n_streams),
                       dim3(256), 0, stream, dst, src, static_cast<const int16_t*>(fresh), meta,
                       meta_dev, n_streams);
  else
    hipLaunchKernelGGL(logmel::logmel_rstream_prep_kernel, dim3((unsigned)n_streams), dim3(256),
                       0, stream, dst, src, static_cast<const float*>(fresh), meta, meta_dev,
                       n_streams);
  return hipGetLastError();
}

hipError_t logmel_launch_stream_prep(float* ws, int64_t row_stride, const void* fresh, int in_i16,
                                     const int64_t* meta, int64_t* meta_dev, int64_t n_streams,
                                     hipStream_t stream) {
  if (n_streams <= 0) return hipSuccess;
  if (in_i16)
    hipLaunchKernelGGL(logmel::logmel_stream_prep_i16_kernel, dim3((unsigned)n_streams), dim3(256),
                       0, stream, ws, row_stride, static_cast<const int16_t*>(fresh), meta,
                       meta_dev, n_streams);
  else
    hipLaunchKernelGGL(logmel::logmel_stream_prep_kernel, dim3((unsigned)n_streams), dim3(256), 0,
                       stream, ws, row_stride, static_cast<const float*>(fresh), meta, meta_dev,
                       n_streams);
  return hipGetLastError();
}
