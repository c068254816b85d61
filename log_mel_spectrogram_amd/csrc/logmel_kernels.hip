// HIP kernels of the log-mel front end for gfx950 (MI355X).
//
// logmel_tiles_kernel: the offline hot path over a packed ragged batch
//   (fp32 in, fp32 out; logmel_tiles_i16_kernel, logmel_tiles_f16out_kernel
//   and logmel_tiles_i16_f16out_kernel are the same code for int16 PCM
//   input and fp16 output).
//   The flattened frame space [0, total_frames) is cut into tiles of 32
//   consecutive frames, one frame per lane pair f, f + 32 (role 0: even
//   samples, role 1: odd samples; see logmel_frame.h). A persistent grid of one wavefront
//   per SIMD walks the tiles, each wavefront a contiguous run of them; a
//   wavefront locates and loads its next tile while it finishes the current
//   one. A tile may straddle clips: each pair
//   finds its clip from the int64 frame offsets. A tile inside one clip reads
//   its 5360-sample span once, coalesced, and shares it through LDS; a tile
//   across clips stages the spans of its clips' runs of frames in LDS the
//   same way (up to 8 runs; beyond that each lane gathers its own 200
//   samples). The pair's transform runs in registers and each lane
//   writes its 64 bands once, at the row the caller's layout gives the frame
//   (frame-major, or 30-s chunks).
//
// logmel_chunk_pad_kernel (and _f16): the padding rows of the 30-s chunk
//   layout.
//
// The streaming push's first step (moving each stream's carry and appending
// its new samples) is in logmel_stream.hip; its frames are then computed by
// logmel_tiles_kernel over the per-stream segments, so a streamed frame is
// bit-for-bit the offline frame.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "logmel_frame.h"
#include "logmel_launch.h"
#include "logmel_tile.h"

namespace logmel {

// A tile of 32 frames of one clip spans 31 * 160 + 400 = 5360 samples
// (1340 16-byte groups). It is staged in LDS split by parity, each sequence
// of 2680 values stored with 4 padding slots after every 80 (value i at
// i + 4 floor(i / 80)), so that a frame's 200 values start at a multiple of
// 84 and the 16-byte reads of the 32 frames fall on distinct bank groups.
// The even sequence holds sample 2i of the span in order; the odd one holds
// sample 2i + 1 in reverse order (value i is sample 5359 - 2i), which is the
// order role 1 of a pair consumes: frame f's even values start at 84 f, its
// reversed odd values at 84 (31 - f).
static constexpr int kSpan = (kTile - 1) * 160 + 400;
static constexpr int kSpanGroups = kSpan / 4;
static constexpr int kParityLen = 2812;   // last element 2679 sits at 2811
static constexpr int kOddBase = 2832;     // odd sequence after the even one
static_assert(kTabPadFloats >= kSpan, "the plan's pad must cover a span");

// Position in a parity array of value i (4 padding slots after every 80).
__device__ __forceinline__ int par_pos(int i) { return i + 4 * (i / 80); }

// The span of a tile inside one clip, fp32: 16-byte groups lane + 64 i;
// lanes past the span's end repeat its last group, so every load is issued
// without a branch.
static constexpr int kSpanRegs = (kSpanGroups + kWaveLanes - 1) / kWaveLanes;
struct SpanF32 {
  f4u g[kSpanRegs];
};

__device__ __forceinline__ void load_span(const float* __restrict__ base, int64_t s0, int lane,
                                          SpanF32& sp) {
  const float* src = base + s0;
#pragma unroll
  for (int i = 0; i < kSpanRegs; ++i) {
    const int j = min(lane + kWaveLanes * i, kSpanGroups - 1);
    sp.g[i] = *reinterpret_cast<const f4u*>(src + 4 * j);
  }
}

// Group j = ln + 64 i of the span (i = 0 .. kSpanRegs - 2: inside the span
// for every lane) puts its even values at par_pos(2j) and its reversed odd
// values at kOddBase + par_pos(2678 - 2j). From i to i + 1 these move by
// +132 or +136 and by -132 or -136 (the padding after every 80 values is
// crossed once or twice); bit i of the lane's masks, fixed for the kernel,
// says which, so a group's two positions cost a few instructions instead
// of two divisions by 40.
struct SpanSteps {
  uint32_t even, odd;
};
__device__ __forceinline__ SpanSteps span_steps(int ln) {
  uint32_t me = 0, mo = 0;
#pragma unroll
  for (int i = 0; i < kSpanRegs - 2; ++i) {
    me |= (uint32_t)((ln + kWaveLanes * (i + 1)) / 40 - (ln + kWaveLanes * i) / 40 - 1) << i;
    const int x0 = kSpanGroups - 1 - ln - kWaveLanes * i, x1 = x0 - kWaveLanes;
    mo |= (uint32_t)(x0 / 40 - x1 / 40 - 1) << i;
  }
  return {me, mo};
}

// Writes the even and reversed odd values of the span's groups to LDS: put(i,
// e, o) stores group i's values at positions e (even) and o (odd).
template <typename Put>
__device__ __forceinline__ void span_positions(int ln, SpanSteps st, const Put& put) {
  int e = par_pos(2 * ln), o = kOddBase + par_pos(kSpan / 2 - 2 - 2 * ln);
#pragma unroll
  for (int i = 0; i < kSpanRegs - 1; ++i) {
    put(i, e, o);
    if (i < kSpanRegs - 2) {
      e += 132 + 4 * (int)((st.even >> i) & 1u);
      o -= 132 + 4 * (int)((st.odd >> i) & 1u);
    }
  }
  // the last group: lanes past the span's end repeat its last group
  const int j = min(ln + kWaveLanes * (kSpanRegs - 1), kSpanGroups - 1);
  put(kSpanRegs - 1, par_pos(2 * j), kOddBase + par_pos(kSpan / 2 - 2 - 2 * j));
}

__device__ __forceinline__ void span_to_lds(const SpanF32& sp, int ln, SpanSteps st, float* lds) {
  // even values 2j, 2j + 1; reversed odd values 2678 - 2j (sample 4j + 3)
  // and 2679 - 2j (sample 4j + 1)
  span_positions(ln, st, [&](int i, int e, int o) {
    *reinterpret_cast<float2*>(lds + e) = make_float2(sp.g[i].x, sp.g[i].z);
    *reinterpret_cast<float2*>(lds + o) = make_float2(sp.g[i].w, sp.g[i].y);
  });
}

// The span of a tile inside one clip, int16: 8-byte groups (4 samples) from
// the 4-byte aligned sample a0 = s0 rounded down to even, group j = samples
// a0 + 4j .. a0 + 4j + 3. With an even s0 the 1340 groups are the span; with
// an odd s0 they start one sample early and the span's last sample comes as
// a separate 2-byte load, so nothing outside [s0 - 1, s0 + 5360) is read.
struct __attribute__((packed, aligned(4))) u2u {
  uint32_t x, y;
};
struct SpanI16 {
  u2u g[kSpanRegs];
  int16_t tail;
  int odd;
};

__device__ __forceinline__ void load_span(const int16_t* __restrict__ base, int64_t s0, int lane,
                                          SpanI16& sp) {
  // base is 4-byte aligned (the host checks), so sample s0's address is
  // 4-byte aligned when s0 is even
  const int odd = (int)(s0 & 1);
  const int16_t* a0 = base + (s0 - odd);
#pragma unroll
  for (int i = 0; i < kSpanRegs; ++i) {
    const int j = min(lane + kWaveLanes * i, kSpanGroups - 1);
    sp.g[i] = *reinterpret_cast<const u2u*>(a0 + 4 * j);
  }
  sp.tail = a0[odd ? kSpan : 0];
  sp.odd = odd;
}

__device__ __forceinline__ float lo16(uint32_t v) { return (float)(int16_t)(v & 0xffff) * kI16Scale; }
__device__ __forceinline__ float hi16(uint32_t v) { return (float)(int16_t)(v >> 16) * kI16Scale; }

__device__ __forceinline__ void span_to_lds(const SpanI16& sp, int ln, SpanSteps st, float* lds) {
  if (!sp.odd) {
    // samples 4j .. 4j + 3 of the span, as in the fp32 layout
    span_positions(ln, st, [&](int i, int e, int o) {
      const float f0 = lo16(sp.g[i].x), f1 = hi16(sp.g[i].x);
      const float f2 = lo16(sp.g[i].y), f3 = hi16(sp.g[i].y);
      *reinterpret_cast<float2*>(lds + e) = make_float2(f0, f2);
      *reinterpret_cast<float2*>(lds + o) = make_float2(f3, f1);
    });
  } else {
    // group j holds span samples 4j - 1 .. 4j + 2: even values 2j, 2j + 1
    // (samples 4j, 4j + 2), odd values 2j - 1 and 2j (samples 4j - 1, 4j + 1)
    // at reversed positions 2680 - 2j and 2679 - 2j; group 0's first sample
    // lies before the span and goes to a padding slot.
#pragma unroll
    for (int i = 0; i < kSpanRegs; ++i) {
      const int j = min(ln + kWaveLanes * i, kSpanGroups - 1);
      const float f0 = lo16(sp.g[i].x), f1 = hi16(sp.g[i].x);
      const float f2 = lo16(sp.g[i].y), f3 = hi16(sp.g[i].y);
      *reinterpret_cast<float2*>(lds + par_pos(2 * j)) = make_float2(f1, f3);
      lds[kOddBase + (j > 0 ? par_pos(kSpan / 2 - 2 * j) : 80)] = f0;
      lds[kOddBase + par_pos(kSpan / 2 - 1 - 2 * j)] = f2;
    }
    // span sample 5359: odd value 2679, reversed position 0
    if (ln == 0) lds[kOddBase] = (float)sp.tail * kI16Scale;
  }
}

// ---------------------------------------------------------------------------
// Tiles across clips. The valid frames of such a tile form pieces: runs
// whose starts advance by exactly one hop (frames of one clip, in order).
// They are staged in LDS like a one-clip span, in a virtual span of 160-
// sample slots: each piece takes one slot per frame plus two spare slots
// after its last frame, so frame f sits at slot f + 2 b(f), where b(f)
// counts the pieces other than the first that start at or before f. A frame
// at slot t reads virtual samples [160 t, 160 t + 400): its slot, the next
// one and 80 samples of the one after, which hold the following frames of
// its piece or the spare slots, all filled from the frame's own clip. With
// at most kMaxBreaks pieces after the first, the virtual span of kPieceT
// slots (plus half a slot) fits in LDS; tiles of more pieces, which only
// clips shorter than about 100 ms produce, gather per lane.
// ---------------------------------------------------------------------------
static constexpr int kMaxBreaks = 7;
static constexpr int kPieceT = kTile + 1 + 2 * kMaxBreaks;          // 47
static constexpr int kPieceSpan = 160 * kPieceT + 80;               // 7600 samples
static constexpr int kPieceGroups = kPieceSpan / 4;                 // 1900
static constexpr int kPieceRegs = (kPieceGroups + kWaveLanes - 1) / kWaveLanes;   // 30
static constexpr int kPieceParityLen = kPieceSpan / 2 - 1 + 4 * ((kPieceSpan / 2 - 1) / 80) + 1;
// the odd sequence starts at the same bank offset, relative to the frames'
// reads, as in the one-clip layout
static constexpr int kPieceOddBase = 4024;
static_assert(kPieceOddBase >= kPieceParityLen && kPieceOddBase % 4 == 0, "piece layout");
static_assert((kPieceOddBase + 84 * (kPieceT - 2)) % 64 == (kOddBase + 84 * (kTile - 1)) % 64,
              "piece layout banks");
static constexpr int kLdsFloats =
    (kPieceOddBase + kPieceParityLen > kOddBase + kParityLen ? kPieceOddBase + kPieceParityLen
                                                            : kOddBase + kParityLen);

template <typename In>
__device__ __forceinline__ void pieces_to_lds(const In* __restrict__ samples, const TileSrc& t,
                                              const In* __restrict__ pad, int sigma,
                                              int ln, float* lds, PieceSlot* slots) {
  // Slot table: clear, then each valid frame's spare slots, then its next
  // and its own slot, each step after the last (later writes win: within a
  // piece they give the following frames' own slots).
  if (ln <= kPieceT) slots[ln].lim = 0;
  lds_barrier();
  const bool w = ln < 32 && t.valid;
  if (w) slots[sigma + 2] = PieceSlot{t.s + 320, 80, 0};
  lds_barrier();
  if (w) slots[sigma + 1] = PieceSlot{t.s + 160, 160, 0};
  lds_barrier();
  if (w) slots[sigma] = PieceSlot{t.s, 160, 0};
  lds_barrier();
  // One 16-byte read per slot (start and count together), all issued before
  // the first is used.
  int4 sl[kPieceRegs];
#pragma unroll
  for (int i = 0; i < kPieceRegs; ++i) {
    const int j = min(ln + kWaveLanes * i, kPieceGroups - 1);
    sl[i] = *reinterpret_cast<const int4*>(slots + j / 40);
  }
#pragma unroll
  for (int i = 0; i < kPieceRegs; ++i) asm volatile("" : "+v"(sl[i].x), "+v"(sl[i].y), "+v"(sl[i].z));
  // Group j (samples 4j .. 4j + 3 of the virtual span) lies in slot j / 40;
  // positions past the slot's samples read zeros from the pad, so every
  // lane loads and none waits alone.
  const In* src[kPieceRegs];
#pragma unroll
  for (int i = 0; i < kPieceRegs; ++i) {
    const int j = min(ln + kWaveLanes * i, kPieceGroups - 1);
    const int off = 4 * j - 160 * (j / 40);
    const int64_t g = (int64_t)(((uint64_t)(uint32_t)sl[i].y << 32) | (uint32_t)sl[i].x);
    src[i] = off < sl[i].z ? samples + g + off : pad;
  }
  float4 val[kPieceRegs];
#pragma unroll
  for (int i = 0; i < kPieceRegs; ++i) val[i] = load_group(src[i]);
#pragma unroll
  for (int i = 0; i < kPieceRegs; ++i) {
    const int j = min(ln + kWaveLanes * i, kPieceGroups - 1);
    const int e = par_pos(2 * j);
    const int o = kPieceOddBase + par_pos(kPieceSpan / 2 - 2 - 2 * j);
    *reinterpret_cast<float2*>(lds + e) = make_float2(val[i].x, val[i].z);
    *reinterpret_cast<float2*>(lds + o) = make_float2(val[i].w, val[i].y);
  }
}

// ---------------------------------------------------------------------------
// Output types: fp32, or fp16 (each value rounded once to nearest).
// ---------------------------------------------------------------------------
// A lane's 64 values are the bands its role logs, in runs of kBandRun<Out>
// bands (the roles take alternate runs of the row, role 0 the first; see
// band_role in logmel_frame.h): one 16-byte piece, 4 bands of fp32 output or
// 8 of fp16.
template <typename Out> constexpr int kBandRun = 16 / (int)sizeof(Out);

// Element offset in the row of the lane's value j (the start of a 16-byte
// piece when j is a multiple of its width).
template <int U>
__device__ __forceinline__ int run_offset(int role, int j) {
  return (j / U) * 2 * U + role * U + j % U;
}

__device__ __forceinline__ void store_bands(float* __restrict__ row, int role, const float (&o)[64]) {
  constexpr int U = kBandRun<float>;
  static_assert(U % 4 == 0, "runs of whole 16-byte pieces");
#pragma unroll
  for (int i = 0; i < 16; ++i)
    *reinterpret_cast<float4*>(row + run_offset<U>(role, 4 * i)) =
        make_float4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
}

__device__ __forceinline__ void store_bands(_Float16* __restrict__ row, int role, const float (&o)[64]) {
  constexpr int U = kBandRun<_Float16>;
  static_assert(U % 8 == 0, "runs of whole 16-byte pieces");
#pragma unroll
  for (int i = 0; i < 8; ++i)
    *reinterpret_cast<uint4*>(row + run_offset<U>(role, 8 * i)) =
        make_uint4(pack_half2(o[8 * i], o[8 * i + 1]), pack_half2(o[8 * i + 2], o[8 * i + 3]),
                   pack_half2(o[8 * i + 4], o[8 * i + 5]), pack_half2(o[8 * i + 6], o[8 * i + 7]));
}

template <typename In> struct SpanOf;
template <> struct SpanOf<float> { using type = SpanF32; };
template <> struct SpanOf<int16_t> { using type = SpanI16; };

template <typename In, typename Out>
__device__ __forceinline__ void tiles_body(const In* __restrict__ samples,
                                           const int64_t* __restrict__ seg_start,
                                           const int64_t* __restrict__ seg_end,
                                           const int64_t* __restrict__ frame_off,
                                           int64_t n_clips, int64_t total_frames,
                                           Out* __restrict__ out,
                                           const int64_t* __restrict__ row_base,
                                           int64_t row_unit, int64_t out_rows,
                                           const double* __restrict__ tables,
                                           float* lds, int64_t (&row_lds)[2][kTile],
                                           PieceSlot* slots, double* rot_lds) {
  // a readable stand-in for a span when there is none to fetch (zeros)
  const In* span_pad = reinterpret_cast<const In*>(tables + kTabDoubles);
  const RowMap rows{row_base, row_unit};
  const int lane = threadIdx.x;
  __builtin_assume(lane < kWaveLanes);
  const int role = lane >> 5;
  const int fl = lane & 31;
  const int64_t n_tiles = (total_frames + kTile - 1) / kTile;

  // Wavefront w takes a contiguous run of tiles (the first n_tiles % grid
  // wavefronts one more), so that consecutive tiles usually share a clip and
  // are located from the cached clip without a lookup. While it computes one
  // tile it locates the next and loads that tile's span into registers
  // (between the transform and the filterbank, where the fewest registers
  // are live), so the loads' latency hides behind the filterbank and the log.
  const int64_t per = n_tiles / gridDim.x, extra = n_tiles % gridDim.x;
  int64_t tile = blockIdx.x * per + min((int64_t)blockIdx.x, extra);
  const int64_t tile_end = tile + per + ((int64_t)blockIdx.x < extra ? 1 : 0);
  if (tile >= tile_end) return;
  // Wavefronts that start together run their tiles in step, and the four of
  // a compute unit then issue their span loads and stores at the same time;
  // tiles run faster once the wavefronts drift apart. Where each wavefront
  // has several tiles, SIMD s of a compute unit starts s x 1920 cycles late
  // (the SIMD from the hardware-ID register), so that the four begin out of
  // step; a launch of one or a few tiles per wavefront, whose time is one
  // tile's latency, starts at once.
  if (n_tiles >= 4 * (int64_t)gridDim.x) {
    const uint32_t simd = __builtin_amdgcn_s_getreg((1 << 11) | (4 << 6) | 4) & 3u;   // HW_ID[5:4]
    for (uint32_t i = 0; i < simd; ++i) __builtin_amdgcn_s_sleep(30);
  }
  // The combine's rotations go to LDS (the two halves of a pair read
  // different ones): 100 16-byte entries, loaded now and written after the
  // first tile is located, so that the loads' latency overlaps the lookup.
  const float4* rot_src = reinterpret_cast<const float4*>(tables + kTabRot400);
  const float4 rot0 = rot_src[lane], rot1 = rot_src[min(lane + kWaveLanes, 99)];
  ClipCache cc{0, 0, 0, 0, 0};
  const SpanSteps steps = span_steps(lane);
  TileSrc cur = locate_tile(tile, lane, seg_start, seg_end, frame_off, rows, n_clips,
                            total_frames, cc);
  if (role == 0) row_lds[0][fl] = cur.row;
  typename SpanOf<In>::type span;
  if (cur.fast) load_span(samples, cur.s0, lane, span);
  reinterpret_cast<float4*>(rot_lds)[lane] = rot0;
  if (lane + kWaveLanes < 100) reinterpret_cast<float4*>(rot_lds)[lane + kWaveLanes] = rot1;
  {
    // A kernel starts with its scalar cache invalidated, and the transform
    // reads the window through it: touch every 64-byte line of the window
    // now, while the first span's loads are in flight, instead of missing on
    // them one by one inside the first transform.
    // One 4-byte load per line, in batches that are all in flight before
    // their first use (one round trip to L2 per batch).
    constexpr int kLines = (200 * 8 + 63) / 64;   // 25
    constexpr int kBatch = 13;
    const uint32_t* tl = reinterpret_cast<const uint32_t*>(tables + kTabWindow);
#pragma unroll
    for (int b = 0; b < kLines; b += kBatch) {
      uint32_t v[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) v[i] = b + i < kLines ? tl[16 * (b + i)] : 0u;
      uint32_t x = 0;
#pragma unroll
      for (int i = 0; i < kBatch; ++i) x ^= v[i];
      asm volatile("" ::"s"(x));
    }
  }

  for (int it = 0;; ++it) {
    // Lane-derived LDS addresses are formed inside the loop: hoisted out of
    // it they would stay live across the transform.
    int ln = lane;
    asm volatile("" : "+v"(ln));
    // This lane's 200 samples: x[s + 2m] for role 0, x[s + 399 - 2m] for role 1.
    float v[200];
    int sigma, breaks;
    if (cur.fast) {
      // Split the span by parity into LDS (layout above), then read back this
      // lane's 200 values.
      span_to_lds(span, ln, steps, lds);
      lds_barrier();
      const float4* a = reinterpret_cast<const float4*>(
          lds + ((ln >> 5) ? kOddBase + 84 * (kTile - 1 - (ln & 31)) : 84 * (ln & 31)));
#pragma unroll
      for (int q = 0; q < 50; ++q) {
        const float4 t = a[q + q / 20];
        v[4 * q] = t.x;
        v[4 * q + 1] = t.y;
        v[4 * q + 2] = t.z;
        v[4 * q + 3] = t.w;
      }
    } else if (piece_slot(cur, ln, sigma, breaks), breaks <= kMaxBreaks) {
      // Tiles across clips (and the batch's last, partial tile): the same
      // through the pieces layout.
      pieces_to_lds(samples, cur, span_pad, sigma, ln, lds, slots);
      lds_barrier();
      const float4* a = reinterpret_cast<const float4*>(
          lds + ((ln >> 5) ? kPieceOddBase + 84 * (kPieceT - 2 - sigma) : 84 * sigma));
#pragma unroll
      for (int q = 0; q < 50; ++q) {
        const float4 t = a[q + q / 20];
        v[4 * q] = t.x;
        v[4 * q + 1] = t.y;
        v[4 * q + 2] = t.z;
        v[4 * q + 3] = t.w;
      }
    } else if (cur.valid) {
      // Frames of more than kMaxBreaks + 1 pieces: each lane gathers its own
      // 200 samples; the caches serve the overlap.
      const In* p = samples + cur.s + (role ? 399 : 0);
      const int64_t step = role ? -2 : 2;
#pragma unroll
      for (int m = 0; m < 200; ++m) {
        v[m] = sample_value(p);
        p += step;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 200; ++i) v[i] = 0.0f;
    }
    // Offsets that promise a frame the clip cannot hold give a row of NaN (a
    // loud row, not a silent truncation): a NaN sample reaches every bin of
    // both halves, so one select here stands for 64 selects of outputs.
    if (!cur.valid) v[0] = __builtin_nanf("");
#pragma unroll
    for (int i = 0; i < 200; ++i) fence(v[i]);

    float Pp[51], Pm[51];
    pair_power(v, tables + kTabWindow, rot_lds + 100 * role, Pp, Pm);

    const int64_t next = tile + 1;
    const bool more = next < tile_end;
    TileSrc nxt = cur;
    if (more) {
      nxt = locate_tile(next, lane, seg_start, seg_end, frame_off, rows, n_clips, total_frames,
                        cc);
      if (role == 0) row_lds[(it + 1) & 1][fl] = nxt.row;
    }
    // Loaded on every path (from the plan's zero pad when there is no span
    // to fetch), so that no register merge waits for the loads here.
    load_span(more && nxt.fast ? samples : span_pad, more && nxt.fast ? nxt.s0 : 0, lane, span);

    float o[64];
    pair_logmel<kBandRun<Out>>(Pp, Pm, role, o);
    const int64_t g = tile * kTile + fl;
    const int64_t row = row_lds[it & 1][ln & 31];
    if (g < total_frames && row >= 0 && row < out_rows)
      store_bands(out + row * 128, role, o);
    if (!more) break;
    tile = next;
    cur = nxt;
  }
}

#define LOGMEL_TILES_KERNEL(NAME, IN, OUT)                                                      \
  extern "C" __global__ void __attribute__((amdgpu_flat_work_group_size(64, 64),                \
                                            amdgpu_waves_per_eu(1, 1)))                         \
  NAME(const IN* __restrict__ samples, const int64_t* __restrict__ seg_start,                   \
       const int64_t* __restrict__ seg_end, const int64_t* __restrict__ frame_off,              \
       int64_t n_clips, int64_t total_frames, OUT* __restrict__ out,                             \
       const int64_t* __restrict__ row_base, int64_t row_unit, int64_t out_rows,                \
       const double* __restrict__ tables) {                                                     \
    __shared__ float4 span_lds[(kLdsFloats + 3) / 4];                                           \
    __shared__ int64_t row_lds[2][kTile];                                                       \
    __shared__ PieceSlot slots[kPieceT + 1];                                                    \
    __shared__ float4 rot_lds[100];                                                             \
    tiles_body<IN, OUT>(samples, seg_start, seg_end, frame_off, n_clips, total_frames, out,     \
                        row_base, row_unit, out_rows, tables,                                   \
                        reinterpret_cast<float*>(span_lds), row_lds, slots,                     \
                        reinterpret_cast<double*>(rot_lds));                                    \
  }

// samples [seg_start[i], seg_end[i]) are clip i; frame f of clip i goes to
// row row_base[i] * row_unit + f of out ([out_rows][128]); tables: the plan's
// window, rotations and zero pad.
LOGMEL_TILES_KERNEL(logmel_tiles_kernel, float, float)
LOGMEL_TILES_KERNEL(logmel_tiles_i16_kernel, int16_t, float)
LOGMEL_TILES_KERNEL(logmel_tiles_f16out_kernel, float, _Float16)
LOGMEL_TILES_KERNEL(logmel_tiles_i16_f16out_kernel, int16_t, _Float16)

// Padding of the 30-s chunk layout: one workgroup per clip fills the rows of
// its last chunk past its last frame, rows [chunk_off[i] * 3000 + F_i,
// chunk_off[i + 1] * 3000), with the log of the floor (rows beyond out_rows
// are skipped). `floor` is the fp32 1e-10 passed in at run time, so the value
// comes from the same log instruction as a silent frame's and equals it (and
// rounds to the same fp16).
template <typename Out>
__device__ __forceinline__ void chunk_pad_body(Out* __restrict__ out,
                                               const int64_t* __restrict__ frame_off,
                                               const int64_t* __restrict__ chunk_off,
                                               int64_t out_rows, float floor) {
  const float pad = __builtin_amdgcn_logf(floor) * kLn2;
  const int64_t i = blockIdx.x;
  const int64_t r0 = chunk_off[i] * 3000 + (frame_off[i + 1] - frame_off[i]);
  const int64_t r1 = min(chunk_off[i + 1] * 3000, out_rows);
  if (r0 >= r1 || r0 < 0) return;
  // 16-byte stores of the value's bits (a row is 512 or 256 bytes)
  const Out v = (Out)pad;
  uint32_t w;
  if constexpr (sizeof(Out) == 4) {
    w = __builtin_bit_cast(uint32_t, v);
  } else {
    const uint32_t h = __builtin_bit_cast(uint16_t, v);
    w = h | (h << 16);
  }
  const uint4 v4 = make_uint4(w, w, w, w);
  uint4* dst = reinterpret_cast<uint4*>(out + r0 * 128);
  const int64_t n = (r1 - r0) * 128 * (int64_t)sizeof(Out) / 16;
  for (int64_t k = threadIdx.x; k < n; k += 256) dst[k] = v4;
}

extern "C" __global__ void __launch_bounds__(256)
logmel_chunk_pad_kernel(float* __restrict__ out, const int64_t* __restrict__ frame_off,
                        const int64_t* __restrict__ chunk_off, int64_t out_rows, float floor) {
  chunk_pad_body<float>(out, frame_off, chunk_off, out_rows, floor);
}

extern "C" __global__ void __launch_bounds__(256)
logmel_chunk_pad_f16_kernel(_Float16* __restrict__ out, const int64_t* __restrict__ frame_off,
                            const int64_t* __restrict__ chunk_off, int64_t out_rows, float floor) {
  chunk_pad_body<_Float16>(out, frame_off, chunk_off, out_rows, floor);
}

}  // namespace logmel

// ---------------------------------------------------------------------------
// Host-side launchers, called by the C-ABI layer.
// ---------------------------------------------------------------------------
hipError_t logmel_launch_tiles(const double* tables, const void* samples, int in_i16,
                               const int64_t* seg_start, const int64_t* seg_end,
                               const int64_t* frame_off, int64_t n_clips, int64_t total_frames,
                               void* out, int out_f16, const int64_t* row_base, int64_t row_unit,
                               int64_t out_rows, int resident_waves, hipStream_t stream) {
  if (total_frames <= 0) return hipSuccess;
  const int64_t tiles = (total_frames + logmel::kTile - 1) / logmel::kTile;
  // One wavefront per SIMD is resident at a time; the grid is that many
  // wavefronts (fewer for small batches) and each walks its share of tiles.
  const int64_t grid = tiles < resident_waves ? tiles : resident_waves;
  const dim3 g((unsigned)grid), b(logmel::kWaveLanes);
  if (!in_i16 && !out_f16) {
    hipLaunchKernelGGL(logmel::logmel_tiles_kernel, g, b, 0, stream,
                       static_cast<const float*>(samples), seg_start, seg_end, frame_off, n_clips,
                       total_frames, static_cast<float*>(out), row_base, row_unit, out_rows, tables);
  } else if (in_i16 && !out_f16) {
    hipLaunchKernelGGL(logmel::logmel_tiles_i16_kernel, g, b, 0, stream,
                       static_cast<const int16_t*>(samples), seg_start, seg_end, frame_off, n_clips,
                       total_frames, static_cast<float*>(out), row_base, row_unit, out_rows, tables);
  } else if (!in_i16) {
    hipLaunchKernelGGL(logmel::logmel_tiles_f16out_kernel, g, b, 0, stream,
                       static_cast<const float*>(samples), seg_start, seg_end, frame_off, n_clips,
                       total_frames, static_cast<_Float16*>(out), row_base, row_unit, out_rows,
                       tables);
  } else {
    hipLaunchKernelGGL(logmel::logmel_tiles_i16_f16out_kernel, g, b, 0, stream,
                       static_cast<const int16_t*>(samples), seg_start, seg_end, frame_off, n_clips,
                       total_frames, static_cast<_Float16*>(out), row_base, row_unit, out_rows,
                       tables);
  }
  return hipGetLastError();
}

hipError_t logmel_launch_chunk_pad(void* out, int out_f16, const int64_t* frame_off,
                                   const int64_t* chunk_off, int64_t n_clips, int64_t out_rows,
                                   hipStream_t stream) {
  // A launch covers at most 2^31 - 1 clips.
  const int64_t chunk = ((int64_t)1 << 31) - 1;
  for (int64_t c0 = 0; c0 < n_clips; c0 += chunk) {
    const int64_t n = n_clips - c0 < chunk ? n_clips - c0 : chunk;
    if (out_f16)
      hipLaunchKernelGGL(logmel::logmel_chunk_pad_f16_kernel, dim3((unsigned)n), dim3(256), 0,
                         stream, static_cast<_Float16*>(out), frame_off + c0, chunk_off + c0,
                         out_rows, kLogFloor);
    else
      hipLaunchKernelGGL(logmel::logmel_chunk_pad_kernel, dim3((unsigned)n), dim3(256), 0, stream,
                         static_cast<float*>(out), frame_off + c0, chunk_off + c0, out_rows,
                         kLogFloor);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}
