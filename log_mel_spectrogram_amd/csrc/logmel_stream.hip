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
// A uniform push (see StreamUniform) takes every field from the kernel's
// arguments and reads no host memory.
template <typename In>
__device__ __forceinline__ void stream_prep_body(float* __restrict__ ws, int64_t row_stride,
                                                 const In* __restrict__ fresh,
                                                 const int64_t* __restrict__ meta,
                                                 int64_t* __restrict__ meta_dev,
                                                 int64_t n_streams, StreamUniform u) {
  const int64_t j = blockIdx.x;
  const int t = threadIdx.x;
  const int64_t base = j * row_stride;
  int64_t src, clen, noff, nlen, seg0, seg1, fo1;
  if (u.on) {
    src = base + u.d;
    clen = u.c;
    noff = j * u.P;
    nlen = u.P;
    seg0 = base + 400 - u.c;
    seg1 = base + 400 + u.P;
    fo1 = (j + 1) * u.F;
  } else {
    const int64_t* rec = meta + j * kStreamMetaRec;
    src = rec[0];
    clen = rec[1];
    noff = rec[2];
    nlen = rec[3];
    seg0 = rec[4];
    seg1 = rec[5];
    fo1 = rec[6];
  }
  // the transform kernel's inputs: segment start and end, frame offsets
  if (t == 0) meta_dev[4 * n_streams + j] = seg0;
  if (t == 1) meta_dev[5 * n_streams + j] = seg1;
  if (t == 2) meta_dev[6 * n_streams + j + 1] = fo1;
  if (t == 3 && j == 0) meta_dev[6 * n_streams] = 0;
  // The carry can overlap its destination, and the new samples land where
  // the old ones were: read the carry and the first new samples (4,096: a
  // whole push at the 80, 120 and 160 ms clocks) before any write.
  float c0 = 0.f, c1 = 0.f;
  if (t < clen) c0 = ws[src + t];
  if (t + 256 < clen) c1 = ws[src + t + 256];
  const In* in = fresh + noff;
  constexpr int kBatch = 16;
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
                          int64_t* __restrict__ meta_dev, int64_t n_streams, StreamUniform u) {
  stream_prep_body(ws, row_stride, fresh, meta, meta_dev, n_streams, u);
}

extern "C" __global__ void __launch_bounds__(256)
logmel_stream_prep_i16_kernel(float* __restrict__ ws, int64_t row_stride,
                              const int16_t* __restrict__ fresh, const int64_t* __restrict__ meta,
                              int64_t* __restrict__ meta_dev, int64_t n_streams, StreamUniform u) {
  stream_prep_body(ws, row_stride, fresh, meta, meta_dev, n_streams, u);
}

// A resampling stream's push, step 1: one workgroup per stream builds its
// segment in dst: the retained input samples (from the previous push's
// buffer src), then the new ones (fp32, or int16 PCM as s / 32768). It also
// moves the stream's 16 kHz carry to sit right before row base + 400 of the
// workspace ws, where the resampling kernel then writes the push's 16 kHz
// samples, so that no copy of them follows. meta is the host's staging slot
// (pinned host memory, read in place), one record of kRStreamMetaRec int64
// per stream (one line): 0 carry index in src, 1 carry length, 2 offset of
// the new samples, 3 their number, 4 segment start in dst, 5 buffer index
// of the clip's sample 0, 6 segment end, 7 number of the first output,
// 8 output offset after the stream, 9 16 kHz carry index in ws, 10 its
// length, 11 the push's 16 kHz samples, 12 frame offset after the stream.
// The kernel copies fields 5 to 8 into the resampling kernel's segment
// arrays in meta_dev ([5n, 6n), [6n, 7n), [7n, 8n), [8n + 1, 9n + 1), with
// 0 at 8n) and the transform kernel's segment starts, ends and frame
// offsets into meta16_dev as the 16 kHz prep kernel does. A uniform push
// (RStreamUniform and StreamUniform both on) reads no host memory.
template <typename In>
__device__ __forceinline__ void rstream_prep_body(float* __restrict__ dst,
                                                  const float* __restrict__ src,
                                                  const In* __restrict__ fresh,
                                                  const int64_t* __restrict__ meta,
                                                  int64_t* __restrict__ meta_dev,
                                                  int64_t n_streams, RStreamUniform u,
                                                  float* __restrict__ ws, int64_t row_stride,
                                                  int64_t* __restrict__ meta16_dev,
                                                  StreamUniform u16) {
  const int64_t j = blockIdx.x;
  const int t = threadIdx.x;
  const int64_t base = j * row_stride;
  int64_t csrc, clen, noff, nlen, seg0, f5, f6, f7, f8, src16, clen16, k16, fo1;
  if (u.on) {
    // every stream in the same state: its record from the arguments
    csrc = u.src0 + j * u.src_step;
    clen = u.c;
    noff = j * u.p;
    nlen = u.p;
    seg0 = j * (u.c + u.p);
    f5 = seg0 - (u.rs_in - u.c);
    f6 = seg0 + u.c + u.p;
    f7 = u.rs_out;
    f8 = (j + 1) * u.k;
    src16 = base + u16.d;
    clen16 = u16.c;
    k16 = u16.P;
    fo1 = (j + 1) * u16.F;
  } else {
    const int64_t* rec = meta + j * kRStreamMetaRec;
    csrc = rec[0];
    clen = rec[1];
    noff = rec[2];
    nlen = rec[3];
    seg0 = rec[4];
    f5 = rec[5];
    f6 = rec[6];
    f7 = rec[7];
    f8 = rec[8];
    src16 = rec[9];
    clen16 = rec[10];
    k16 = rec[11];
    fo1 = rec[12];
  }
  // the resampling kernel's inputs: segment origin, end, first output
  // number and output offsets
  if (t == 0) meta_dev[5 * n_streams + j] = f5;
  if (t == 1) meta_dev[6 * n_streams + j] = f6;
  if (t == 2) meta_dev[7 * n_streams + j] = f7;
  if (t == 3) meta_dev[8 * n_streams + j + 1] = f8;
  if (t == 4 && j == 0) meta_dev[8 * n_streams] = 0;
  // the transform kernel's: segment start and end in ws, frame offsets
  if (t == 5) meta16_dev[4 * n_streams + j] = base + 400 - clen16;
  if (t == 6) meta16_dev[5 * n_streams + j] = base + 400 + k16;
  if (t == 7) meta16_dev[6 * n_streams + j + 1] = fo1;
  if (t == 8 && j == 0) meta16_dev[6 * n_streams] = 0;
  // The segment is the carry (from src) followed by the new samples; src and
  // dst are different buffers, and so are ws and both. The 16 kHz carry can
  // overlap its destination: read it, and the segment's first kBatch * 256
  // values (a whole push at the usual clocks), before any write, so that one
  // round trip to memory serves them all.
  constexpr int kBatch = 16;
  const int64_t total = clen + nlen;
  const In* in = fresh + noff;
  float* seg = dst + seg0;
  float c0 = 0.f, c1 = 0.f;
  if (t < clen16) c0 = ws[src16 + t];
  if (t + 256 < clen16) c1 = ws[src16 + t + 256];
  float v[kBatch];
#pragma unroll
  for (int u = 0; u < kBatch; ++u) {
    const int64_t i = t + 256 * u;
    v[u] = i < clen ? src[csrc + i] : (i < total ? stream_sample(in, i - clen) : 0.0f);
  }
  __syncthreads();
  if (t < clen16) ws[base + 400 - clen16 + t] = c0;
  if (t + 256 < clen16) ws[base + 400 - clen16 + t + 256] = c1;
#pragma unroll
  for (int u = 0; u < kBatch; ++u) {
    const int64_t i = t + 256 * u;
    if (i < total) seg[i] = v[u];
  }
  // longer segments (large pushes, high input rates): the rest in batches
  for (int64_t i0 = 256 * kBatch; i0 < total; i0 += 256 * kBatch) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t i = i0 + t + 256 * u;
      v[u] = i < clen ? src[csrc + i] : (i < total ? stream_sample(in, i - clen) : 0.0f);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t i = i0 + t + 256 * u;
      if (i < total) seg[i] = v[u];
    }
  }
}

extern "C" __global__ void __launch_bounds__(256)
logmel_rstream_prep_kernel(float* __restrict__ dst, const float* __restrict__ src,
                           const float* __restrict__ fresh, const int64_t* __restrict__ meta,
                           int64_t* __restrict__ meta_dev, int64_t n_streams, RStreamUniform u,
                           float* __restrict__ ws, int64_t row_stride,
                           int64_t* __restrict__ meta16_dev, StreamUniform u16) {
  rstream_prep_body(dst, src, fresh, meta, meta_dev, n_streams, u, ws, row_stride, meta16_dev, u16);
}

extern "C" __global__ void __launch_bounds__(256)
logmel_rstream_prep_i16_kernel(float* __restrict__ dst, const float* __restrict__ src,
                               const int16_t* __restrict__ fresh,
                               const int64_t* __restrict__ meta, int64_t* __restrict__ meta_dev,
                               int64_t n_streams, RStreamUniform u, float* __restrict__ ws,
                               int64_t row_stride, int64_t* __restrict__ meta16_dev,
                               StreamUniform u16) {
  rstream_prep_body(dst, src, fresh, meta, meta_dev, n_streams, u, ws, row_stride, meta16_dev, u16);
}

}  // namespace logmel

hipError_t logmel_launch_rstream_prep(float* dst, const float* src, const void* fresh, int in_i16,
                                      const int64_t* meta, int64_t* meta_dev, int64_t n_streams,
                                      RStreamUniform uni, float* ws, int64_t row_stride,
                                      int64_t* meta16_dev, StreamUniform uni16,
                                      hipStream_t stream) {
  if (n_streams <= 0) return hipSuccess;
  if (in_i16)
    hipLaunchKernelGGL(logmel::logmel_rstream_prep_i16_kernel, dim3((unsigned)n_streams),
                       dim3(256), 0, stream, dst, src, static_cast<const int16_t*>(fresh), meta,
                       meta_dev, n_streams, uni, ws, row_stride, meta16_dev, uni16);
  else
    hipLaunchKernelGGL(logmel::logmel_rstream_prep_kernel, dim3((unsigned)n_streams), dim3(256),
                       0, stream, dst, src, static_cast<const float*>(fresh), meta, meta_dev,
                       n_streams, uni, ws, row_stride, meta16_dev, uni16);
  return hipGetLastError();
}

hipError_t logmel_launch_stream_prep(float* ws, int64_t row_stride, const void* fresh, int in_i16,
                                     const int64_t* meta, int64_t* meta_dev, int64_t n_streams,
                                     StreamUniform uni, hipStream_t stream) {
  if (n_streams <= 0) return hipSuccess;
  if (in_i16)
    hipLaunchKernelGGL(logmel::logmel_stream_prep_i16_kernel, dim3((unsigned)n_streams), dim3(256),
                       0, stream, ws, row_stride, static_cast<const int16_t*>(fresh), meta,
                       meta_dev, n_streams, uni);
  else
    hipLaunchKernelGGL(logmel::logmel_stream_prep_kernel, dim3((unsigned)n_streams), dim3(256), 0,
                       stream, ws, row_stride, static_cast<const float*>(fresh), meta, meta_dev,
                       n_streams, uni);
  return hipGetLastError();
}
