// Internal launchers shared by the kernels and the C-ABI layer.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stdint.h>


// Device constant tables owned by a plan (fp64): the window at the even
// points in the order the transform consumes them (both lanes of a pair use
// it), then cos/sin of 2 pi k / 800 interleaved, in the order the
// transform's 8-point DFTs produce bins ([k2][k1], 13 x 8 pairs).
// After the doubles, kTabPadFloats zero floats: a readable stand-in for a
// tile's 5360-sample span.
static constexpr int kTabWindow = 0;
static constexpr int kTabRot800 = 200;
static constexpr int kTabDoubles = 408;
static constexpr int kTabPadFloats = 5360;
static constexpr size_t kTabBytes = 8 * kTabDoubles + 4 * kTabPadFloats;

// Frame f of clip i goes to row row_base[i] * row_unit + f of out (rows at or
// beyond out_rows are not written). samples are fp32, or int16 PCM (s / 32768)
// with in_i16; out is fp32, or fp16 with out_f16.
hipError_t logmel_launch_tiles(const double* tables, const void* samples, int in_i16,
                               const int64_t* seg_start, const int64_t* seg_end,
                               const int64_t* frame_off, int64_t n_clips, int64_t total_frames,
                               void* out, int out_f16, const int64_t* row_base, int64_t row_unit,
                               int64_t out_rows, int resident_waves, hipStream_t stream);

hipError_t logmel_launch_chunk_pad(void* out, int out_f16, const int64_t* frame_off,
                                   const int64_t* chunk_off, int64_t n_clips, int64_t out_rows,
                                   hipStream_t stream);

// fresh: fp32, or int16 PCM (s / 32768) with in_i16. meta: the host's
// staging slot (pinned host memory, its device-side address; records as in
// logmel_stream.hip); the kernel copies what the transform kernel reads into
// meta_dev ([4n, 7n + 1): segment starts, ends, frame offsets).
hipError_t logmel_launch_stream_prep(float* ws, int64_t row_stride, const void* fresh, int in_i16,
                                     const int64_t* meta, int64_t* meta_dev, int64_t n_streams,
                                     hipStream_t stream);

