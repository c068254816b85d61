// Internal launcher of the resampling kernel, shared with the C-ABI layer.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stdint.h>

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
