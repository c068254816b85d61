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
#include "logmel_slots.h"

namespace logmel {

__device__ __forceinline__ float stream_sample(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float stream_sample(const int16_t* p, int64_t i) {
  return (float)p[i] * (1.0f / 32768.0f);
}

// One workgroup per stream. meta is the host's staging slot, read by the
// device in place (pinned host memory), one record of kStreamMetaRec int64
// per stream, so that a workgroup's fields come in one line (n records
// field by field would cost each workgroup a host-memory read per field):
//   0  carry source index in ws (absolute)
//   1  carry length (< 400)
//   2  offset of the stream's new samples in `fresh`
//   3  number of new samples
//   4  segment start in ws  (= row base + 400 - carry length)
//   5  segment end in ws    (= row base + 400 + new samples)
//   6  output frame offset after the stream
// The kernel copies fields 4, 5 and 6 into meta_dev ([4n, 5n), [5n, 6n),
// [6n + 1, 7n + 1), with 0 at 6n), where the transform kernel that follows
// reads them.
template <typename In>
__device__ __forceinline__ void stream_prep_body(float* __restrict__ ws, int64_t row_stride,
                                                 const In* __restrict__ fresh,
                                                 const int64_t* __restrict__ meta,
                                                 int64_t* __restrict__ meta_dev,
                                                 int64_t n_streams) {
  const int64_t j = blockIdx.x;
  const int t = threadIdx.x;
  const int64_t base = j * row_stride;
  const int64_t* rec = meta + j * kStreamMetaRec;
  const int64_t src = rec[0];
  const int64_t clen = rec[1];
  const int64_t noff = rec[2];
  const int64_t nlen = rec[3];
  // the transform kernel's inputs: segment start and end, frame offsets
  if (t == 0) meta_dev[4 * n_streams + j] = rec[4];
  if (t == 1) meta_dev[5 * n_streams + j] = rec[5];
  if (t == 2) meta_dev[6 * n_streams + j + 1] = rec[6];
  if (t == 3 && j == 0) meta_dev[6 * n_streams] = 0;
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
// the host's staging slot (pinned host memory, read in place), one record of
// kRStreamMetaRec int64 per stream (one line): 0 carry index in src,
// 1 carry length, 2 offset of the new samples, 3 their number, 4 segment
// start in dst, 5 buffer index of the clip's sample 0, 6 segment end,
// 7 number of the first output, 8 output offset after the stream. The
// kernel copies fields 5 to 8 into the resampling kernel's segment arrays in
// meta_dev ([5n, 6n), [6n, 7n), [7n, 8n), [8n + 1, 9n + 1), with 0 at 8n).
template <typename In>
__device__ __forceinline__ void rstream_prep_body(float* __restrict__ dst,
                                                  const float* __restrict__ src,
                                                  const In* __restrict__ fresh,
                                                  const int64_t* __restrict__ meta,
                                                  int64_t* __restrict__ meta_dev,
                                                  int64_t n_streams) {
  const int64_t j = blockIdx.x;
  const int t = threadIdx.x;
  const int64_t* rec = meta + j * kRStreamMetaRec;
  const int64_t csrc = rec[0];
  const int64_t clen = rec[1];
  const int64_t noff = rec[2];
  const int64_t nlen = rec[3];
  // the resampling kernel's inputs: segment origin, end, first output
  // number and output offsets
  if (t == 0) meta_dev[5 * n_streams + j] = rec[5];
  if (t == 1) meta_dev[6 * n_streams + j] = rec[6];
  if (t == 2) meta_dev[7 * n_streams + j] = rec[7];
  if (t == 3) meta_dev[8 * n_streams + j + 1] = rec[8];
  if (t == 4 && j == 0) meta_dev[8 * n_streams] = 0;
  float* seg = dst + rec[4];
  // src and dst are different buffers: eight loads per thread in flight
  // before their stores
  constexpr int kBatch = 8;
  for (int64_t i0 = 0; i0 < clen; i0 += 256 * kBatch) {
    float v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t i = i0 + t + 256 * u;
      v[u] = i < clen ? src[csrc + i] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t i = i0 + t + 256 * u;
      if (i < clen) seg[i] = v[u];
    }
  }
  const In* in = fresh + noff;
  float* row = seg + clen;
  for (int64_t i0 = 0; i0 < nlen; i0 += 256 * kBatch) {
    float v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t i = i0 + t + 256 * u;
      v[u] = i < nlen ? stream_sample(in, i) : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t i = i0 + t + 256 * u;
      if (i < nlen) row[i] = v[u];
    }
  }
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
