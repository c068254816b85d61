// Internal launcher of the resampling kernel, shared with the C-ABI layer.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "logmel_launch.h"

// Resampling to 16 kHz on the matrix cores (see logmel_resample.hip): the
// geometry of one input rate. Super-periods of S outputs start S_in input
// samples apart; C column groups of 16 outputs; KS MFMA steps of 4 samples
// per output (a multiple of 8); tiles of NT x 16 super-periods, TB outputs,
// worked in items of RB row blocks (RB divides NT); J: the half-width in
// input samples. In LDS a tile's super-periods start P floats apart: P =
// S_in, or S_in + 2 when 32 divides S_in (two zero floats after each
// super-period's samples, so that the 16 rows of an MFMA operand start in
// distinct banks); span: LDS floats one tile stages.
struct RsmGeometry {
  int S, S_in, C, KS, NT, RB, J, span, P;
  int64_t TB;
};

// Largest LDS span a resampling workgroup may stage (floats), and the span
// below which two or more workgroups share a compute unit.
static constexpr int kRsmLdsMax = 38400;
static constexpr int kRsmLdsSmall = 14336;

// Segment i's samples are [seg_lo[i], seg_hi[i]) of x (fp32, or int16 PCM
// with in_i16), its clip's sample 0 at seg_lo[i]; samples before
// max(seg_lo[i], seg_hi[i - 1]) and from seg_hi[i] on read as zero; its
// outputs [out_off[i], out_off[i + 1]) of y are the clip's outputs
// nfirst[i], nfirst[i] + 1, ... (nfirst null: from 0), written packed at
// y[out_off[i]] on, or with ystep > 0 at y[i ystep + ybase] on (row i of a
// strided layout; the caller makes each segment's outputs fit its row). The
// last segment ends x. An offline batch passes its sample offsets as seg_lo
// and, one further, as seg_hi. btab: [C][KS][64] fp32 (the B operand per column
// group and step over LDS floats, in the MFMA's lane layout); abase: [C]
// int32, the LDS offset, from its super-period's first float, of column
// group g's window start floor(16 g M / L).
hipError_t logmel_launch_resample(const void* x, int in_i16, const int64_t* seg_lo,
                                  const int64_t* seg_hi, const int64_t* nfirst,
                                  const int64_t* out_off, int64_t n_segs, int64_t total_out,
                                  float* y, int64_t ystep, int64_t ybase, const float* btab,
                                  const int* abase, const RsmGeometry& geo, hipStream_t stream);

// A resampling stream's push, step 1: segment j of dst = src[carry index,
// + carry length) followed by the new samples of stream j (fp32, or int16
// PCM with in_i16; fresh may be null when there are none); and stream j's
// 16 kHz carry moved in ws to end at row j's float 400 (rows row_stride
// floats apart), where the resampling kernel writes the push's 16 kHz
// samples next. meta: the host's staging slot (pinned host memory, its
// device-side address; records as in logmel_stream.hip), of which the kernel
// copies the resampling kernel's part into meta_dev ([5n, 9n + 1): clip
// origins, segment ends, first outputs, output offsets) and the transform
// kernel's into meta16_dev ([4n, 7n + 1), as the 16 kHz prep kernel).
// Where every stream is in the same state (carry length c, retained and
// produced counts rs_in, rs_out, carries spaced src_step apart from src0;
// 16 kHz carries of one length at one place in their rows) and pushes the
// same p samples for k outputs, uni.on and uni16.on are both set, every
// record follows from the two and the kernel reads no host memory.
struct RStreamUniform {
  int64_t on, c, p, src0, src_step, rs_in, rs_out, k;
};
hipError_t logmel_launch_rstream_prep(float* dst, const float* src, const void* fresh, int in_i16,
                                      const int64_t* meta, int64_t* meta_dev, int64_t n_streams,
                                      RStreamUniform uni, float* ws, int64_t row_stride,
                                      int64_t* meta16_dev, StreamUniform uni16,
                                      hipStream_t stream);
