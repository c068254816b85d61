// HIP kernels of the log-mel front end for gfx950 (MI355X).
//
// logmel_tiles_kernel: the offline hot path over a packed ragged batch.
//   The flattened frame space [0, total_frames) is cut into tiles of 64
//   consecutive frames, one wavefront per tile, one frame per lane. A tile may
//   straddle clips. Each lane finds its clip from the int64 frame offsets,
//   loads only the first 160 samples of its frame from HBM and takes the
//   remaining 240 (the overlap of the 400/160 framing) from its two right
//   neighbours with wavefront-shift DPP moves, so every sample is read from
//   HBM once. Lanes whose neighbours are not their next frames (clip ends,
//   the tile's last two lanes) read those 240 samples themselves. Then the
//   per-frame routine of logmel_frame.h runs in registers and the lane writes
//   its 512-byte output row once.
//
// logmel_stream_prep_kernel: the streaming push, step 1. Moves each stream's
//   carry (the samples of its next, not yet complete frame) to sit right
//   before the new samples in the stream's workspace row, and appends the new
//   samples. The frames themselves are then computed by logmel_tiles_kernel
//   over the per-stream segments, so a streamed frame is bit-for-bit the
//   offline frame.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "logmel_frame.h"

namespace logmel {

static constexpr int kTile = 64;

__device__ __forceinline__ float shl1(float v) {
  // wave_shl:1 -- lane i receives lane i+1's value (lane 63 keeps its own,
  // which is never used: the tile's last lanes always reload).
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v),
                                         0x130, 0xf, 0xf, false));
}

// First index in a[0, n) whose value is > v (a non-decreasing).
__device__ __forceinline__ int64_t upper_bound_i64(const int64_t* __restrict__ a, int64_t n,
                                                   int64_t v) {
  int64_t lo = 0, hi = n;
  while (lo < hi) {
    const int64_t mid = lo + ((hi - lo) >> 1);
    if (a[mid] <= v) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// dst[0..N) = p[0..N). 16-byte loads when p is 16-byte aligned, else 4-byte
// loads (a clip may start at any sample; all frames of one clip share the
// alignment because the hop, 160 samples, is a multiple of 4).
template <int N>
__device__ __forceinline__ void load_run(const float* __restrict__ p, float* dst, bool al16) {
  if (al16) {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const float4 v = *reinterpret_cast<const float4*>(p + 4 * i);
      dst[4 * i] = v.x; dst[4 * i + 1] = v.y; dst[4 * i + 2] = v.z; dst[4 * i + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) dst[i] = p[i];
  }
}

extern "C" __global__ void __attribute__((amdgpu_flat_work_group_size(64, 64),
                                          amdgpu_waves_per_eu(1, 1)))
logmel_tiles_kernel(const float* __restrict__ samples,
                    const int64_t* __restrict__ seg_start,   // [n_clips] first sample of clip
                    const int64_t* __restrict__ seg_end,     // [n_clips] one past its last
                    const int64_t* __restrict__ frame_off,   // [n_clips + 1]
                    int64_t n_clips, int64_t total_frames,
                    float* __restrict__ out,                 // [total_frames][128]
                    int64_t first_tile)                      // tile index of blockIdx.x == 0
{
  const int lane = threadIdx.x;
  const int64_t g0 = (first_tile + (int64_t)blockIdx.x) * kTile;
  const int64_t g = g0 + lane;
  const bool in_range = g < total_frames;
  const int64_t gq = in_range ? g : total_frames - 1;   // lookup key for idle lanes

  // Clip of the tile's first frame (wave-uniform), then of every lane.
  int64_t c0 = upper_bound_i64(frame_off, n_clips + 1, g0) - 1;
  c0 = c0 < 0 ? 0 : c0;
  const int64_t bidx = c0 + 1 + lane;
  const int64_t B = bidx <= n_clips ? frame_off[bidx] : INT64_MAX;
  const int64_t B63 = __shfl(B, 63);
  int64_t c;
  if (B63 <= gq) {
    // 64 or more clip boundaries inside this tile (many empty clips).
    c = upper_bound_i64(frame_off, n_clips + 1, gq) - 1;
  } else {
    int cnt = 0;
#pragma unroll
    for (int step = 32; step >= 1; step >>= 1)
      if (__shfl(B, cnt + step - 1) <= gq) cnt += step;
    c = c0 + cnt;
  }
  c = c < 0 ? 0 : (c >= n_clips ? n_clips - 1 : c);   // only inconsistent offsets need this
  const int64_t f = gq - frame_off[c];
  const int64_t s = seg_start[c] + 160 * f;
  // A frame is only computed if all its 400 samples lie inside its clip.
  const bool valid = in_range && f >= 0 && (s + 400 <= seg_end[c]);
  // Wave-uniform: may every lane use 16-byte loads?
  const bool al16 = __all(!valid || (s & 3) == 0);

  float x[400];
  if (valid) {
    load_run<160>(samples + s, x, al16);
  } else {
#pragma unroll
    for (int i = 0; i < 160; ++i) x[i] = 0.0f;
  }
#pragma unroll
  for (int i = 0; i < 160; ++i) x[160 + i] = shl1(x[i]);
#pragma unroll
  for (int i = 0; i < 80; ++i) x[320 + i] = shl1(x[160 + i]);

  // Is lane+2 this clip's frame f+2 (then lane+1 is frame f+1)?
  const int64_t c2 = __shfl_down(c, 2);
  const bool v2 = __shfl_down((int)valid, 2) != 0;
  const bool have_next = (lane < kTile - 2) && v2 && (c2 == c);
  if (valid && !have_next) load_run<240>(samples + s + 160, x + 160, al16);
#pragma unroll
  for (int i = 0; i < 400; ++i) fence(x[i]);

  float o[128];
  logmel_frame(x, o);

  if (in_range) {
    float4* dst = reinterpret_cast<float4*>(out + g * 128);
    if (valid) {
#pragma unroll
      for (int i = 0; i < 32; ++i) dst[i] = make_float4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
    } else {
      // Offsets that promise a frame the clip cannot hold: a loud row, not a
      // silent truncation.
      const float qnan = __builtin_nanf("");
#pragma unroll
      for (int i = 0; i < 32; ++i) dst[i] = make_float4(qnan, qnan, qnan, qnan);
    }
  }
}

// One workgroup per stream. meta layout (int64, n = n_streams):
//   [0n, 1n)  carry source index in ws (absolute)
//   [1n, 2n)  carry length (< 400)
//   [2n, 3n)  offset of the stream's new samples in `fresh`
//   [3n, 4n)  number of new samples
//   [4n, 5n)  segment start in ws  (= row base + 400 - carry length)
//   [5n, 6n)  segment end in ws    (= row base + 400 + new samples)
//   [6n, 7n+1) output frame offsets
extern "C" __global__ void __launch_bounds__(256)
logmel_stream_prep_kernel(float* __restrict__ ws, int64_t row_stride,
                          const float* __restrict__ fresh,
                          const int64_t* __restrict__ meta, int64_t n_streams)
{
  const int64_t j = blockIdx.x;
  const int t = threadIdx.x;
  const int64_t base = j * row_stride;
  const int64_t src = meta[j];
  const int64_t clen = meta[n_streams + j];
  const int64_t noff = meta[2 * n_streams + j];
  const int64_t nlen = meta[3 * n_streams + j];
  // The carry can overlap its destination: read it all before any write.
  float c0 = 0.f, c1 = 0.f;
  if (t < clen) c0 = ws[src + t];
  if (t + 256 < clen) c1 = ws[src + t + 256];
  __syncthreads();
  const int64_t dst = base + 400 - clen;
  if (t < clen) ws[dst + t] = c0;
  if (t + 256 < clen) ws[dst + t + 256] = c1;
  float* row = ws + base + 400;
  const float* in = fresh + noff;
  for (int64_t i = t; i < nlen; i += 256) row[i] = in[i];
}

}  // namespace logmel

// ---------------------------------------------------------------------------
// Host-side launchers, called by the C-ABI layer.
// ---------------------------------------------------------------------------
#include "logmel_launch.h"

hipError_t logmel_launch_tiles(const float* samples, const int64_t* seg_start,
                               const int64_t* seg_end, const int64_t* frame_off,
                               int64_t n_clips, int64_t total_frames, float* out,
                               hipStream_t stream) {
  if (total_frames <= 0) return hipSuccess;
  const int64_t tiles = (total_frames + logmel::kTile - 1) / logmel::kTile;
  // A launch covers at most 2^25 workgroups (2^31 work-items).
  const int64_t chunk = (int64_t)1 << 25;
  for (int64_t t0 = 0; t0 < tiles; t0 += chunk) {
    const int64_t n = tiles - t0 < chunk ? tiles - t0 : chunk;
    hipLaunchKernelGGL(logmel::logmel_tiles_kernel, dim3((unsigned)n), dim3(logmel::kTile), 0,
                       stream, samples, seg_start, seg_end, frame_off, n_clips, total_frames,
                       out, t0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t logmel_launch_stream_prep(float* ws, int64_t row_stride, const float* fresh,
                                     const int64_t* meta, int64_t n_streams,
                                     hipStream_t stream) {
  if (n_streams <= 0) return hipSuccess;
  hipLaunchKernelGGL(logmel::logmel_stream_prep_kernel, dim3((unsigned)n_streams), dim3(256), 0,
                     stream, ws, row_stride, fresh, meta, n_streams);
  return hipGetLastError();
}
