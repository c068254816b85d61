// Internal launchers shared by the kernels and the C-ABI layer.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stdint.h>


// Device constant tables owned by a plan (fp64): the window at the even
// points in the order the transform consumes them (both lanes of a pair use
// it), then cos/sin of 2 pi k / 400 interleaved for the bins each half of a
// lane pair combines ([half][slot], 2 x 50 pairs; the kernel copies them to
// LDS).
// After the doubles, kTabPadFloats zero floats: a readable stand-in for a
// tile's 5360-sample span.
static constexpr int kTabWindow = 0;
static constexpr int kTabRot400 = 200;
static constexpr int kTabDoubles = 400;
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

// A push in which every stream has the same carry length c, its carry at
// the same place of its workspace row (stream j's at j * row_stride + d),
// and the same number P of new samples: every field of stream j's record
// follows from these, and F = frames of c + P (on = 0: read the records).
struct StreamUniform {
  int64_t on, P, c, d, F;
};

// fresh: fp32, or int16 PCM (s / 32768) with in_i16. meta: the host's
// staging slot (pinned host memory, its device-side address; records as in
// logmel_stream.hip), read only where the push is not uniform; the kernel
// writes what the transform kernel reads into meta_dev ([4n, 7n + 1):
// segment starts, ends, frame offsets).
hipError_t logmel_launch_stream_prep(float* ws, int64_t row_stride, const void* fresh, int in_i16,
                                     const int64_t* meta, int64_t* meta_dev, int64_t n_streams,
                                     StreamUniform uni, hipStream_t stream);


// The fixed device array of logmel_stream_push_static (logmel_static.hip):
// its streams' workspace rows (kStaticStride fp32 each: 400 carry slots, then
// up to kStaticMaxPush new samples, 256-byte aligned), then the per-stream
// records of a push (kStaticRecBytes), then the offsets the prep kernel
// hands the transform kernel (7 n + 1 int64).
static constexpr int kStaticMaxDevices = 16;
static constexpr int64_t kStaticMaxStreams = 512;
static constexpr int64_t kStaticMaxPush = 2560;
static constexpr int64_t kStaticStride = (400 + kStaticMaxPush + 63) / 64 * 64;
static constexpr size_t kStaticWsBytes = (size_t)kStaticMaxStreams * kStaticStride * 4;
static constexpr size_t kStaticRecBytes = (size_t)kStaticMaxStreams * 8 * 8;
static constexpr size_t kStaticMetaBytes = ((7 * (size_t)kStaticMaxStreams + 1) * 8 + 255) / 256 * 256;
static constexpr size_t kStaticScratchBytes = kStaticWsBytes + kStaticRecBytes + kStaticMetaBytes;

// Device address of `device`'s copy of that array (looked up once per
// device; the calling thread's current device must be `device`).
hipError_t logmel_static_scratch(int device, void** ptr);
