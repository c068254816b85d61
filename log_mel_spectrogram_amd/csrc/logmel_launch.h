// Internal launchers shared by the kernels and the C-ABI layer.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stdint.h>


hipError_t logmel_launch_tiles(const float* samples, const int64_t* seg_start,
                               const int64_t* seg_end, const int64_t* frame_off,
                               int64_t n_clips, int64_t total_frames, float* out,
                               hipStream_t stream);

hipError_t logmel_launch_stream_prep(float* ws, int64_t row_stride, const float* fresh,
                                     const int64_t* meta, int64_t n_streams,
                                     hipStream_t stream);
