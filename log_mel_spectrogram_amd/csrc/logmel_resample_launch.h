// Internal launcher of the resampling kernel, shared with the C-ABI layer.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stdint.h>

// Resampling to 16 kHz: LDS floats of one workgroup's staged input span
// (one 1024-thread workgroup per compute unit).
static constexpr int kResLdsFloats = 38400;   // 150 KB of the 160 KB

// Segment i's samples are [seg_lo[i], seg_hi[i]) of x (fp32, or int16 PCM
// with in_i16), its clip's sample 0 at seg_lo[i]; its outputs
// [out_off[i], out_off[i + 1]) of y are the clip's outputs nfirst[i],
// nfirst[i] + 1, ... (nfirst null: from 0). The last segment ends x. An
// offline batch passes its sample offsets as seg_lo and, one further, as
// seg_hi. taps is the device table [L][Tp] (rows of 2J + 1 taps zero-padded
// to Tp, a multiple of 16); taps_blk the table [L][TpX][NB] of the shared
// path (for each first phase, the NB outputs' rows shifted by their windows'
// offsets, interleaved sample by sample);
// NB in {1, 2, 3, 4} outputs per lane, lanes Q outputs apart; blocks of 64 G
// lanes; grid: workgroups resident at once.
hipError_t logmel_launch_resample(const void* x, int in_i16, const int64_t* seg_lo,
                                  const int64_t* seg_hi, const int64_t* nfirst,
                                  const int64_t* out_off, int64_t n_segs, int64_t total_out,
                                  float* y, const float* taps, const float* taps_blk, int L, int M,
                                  int J, int Tp, int TpX, int NB, int Q, int G, int grid,
                                  hipStream_t stream);

// A resampling stream's push, step 1: segment j of dst = src[carry index,
// + carry length) followed by the new samples of stream j (fp32, or int16
// PCM with in_i16; fresh may be null when there are none); meta as in the
// host's rs_push: its staging slot (pinned host memory, its device-side
// address), of which the kernel copies the resampling kernel's part into
// meta_dev.
hipError_t logmel_launch_rstream_prep(float* dst, const float* src, const void* fresh, int in_i16,
                                      const int64_t* meta, int64_t* meta_dev, int64_t n_streams,
                                      hipStream_t stream);
