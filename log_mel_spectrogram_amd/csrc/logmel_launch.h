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

hipError_t logmel_launch_stream_prep(float* ws, int64_t row_stride, const float* fresh,
                                     const int64_t* meta, int64_t n_streams,
                                     hipStream_t stream);

// Resampling to 16 kHz: LDS floats of one workgroup's staged input span
// (one 1024-thread workgroup per compute unit).
static constexpr int kResLdsFloats = 38400;   // 150 KB of the 160 KB

// Clip i's samples [in_off[i], in_off[i + 1]) of x (fp32, or int16 PCM with
// in_i16) give outputs [out_off[i], out_off[i + 1]) of y; taps is the device
// table [L][Tp] (rows of 2J + 1 taps zero-padded to Tp, a multiple of 16);
// blocks of 64 G periods of L outputs; grid: workgroups resident at once.
hipError_t logmel_launch_resample(const void* x, int in_i16, const int64_t* in_off,
                                  const int64_t* out_off, int64_t n_clips, int64_t total_out,
                                  float* y, const float* taps, int L, int M, int J, int Tp, int G,
                                  int grid, hipStream_t stream);
