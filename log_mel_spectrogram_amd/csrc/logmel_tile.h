// Tile bookkeeping shared by the log-mel transform kernels (gfx950): the
// flattened frame space is cut into tiles of 32 consecutive frames; a
// wavefront's lanes f and f + 32 (lane & 31 = f) belong to frame f of its
// tile. Locating a tile's clips from the int64 frame offsets, the cached
// clip of a contiguous run of tiles, the output row map, input sample types
// and the slot records of tiles across clips.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "logmel_frame.h"

namespace logmel {

static constexpr int kTile = 32;          // frames per wavefront
static constexpr int kWaveLanes = 64;

// 16 bytes from a 4-byte aligned address (global memory allows this on the
// HSA target).
struct __attribute__((packed, aligned(4))) f4u {
  float x, y, z, w;
};

// Workgroup barrier that orders LDS accesses only: the waits before it cover
// this wavefront's LDS operations, not its global stores (a __syncthreads
// would also wait for every store of the output to be acknowledged).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
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

// Where a tile's frames come from. Per lane: the frame (g), whether it is
// inside the batch (in_range) and computable (valid), its first sample (s).
// Per wavefront: whether all 32 frames lie in one clip (fast), in which case
// the tile's span starts at sample s0.
struct TileSrc {
  int64_t g, s, s0;
  int64_t row;  // output row of the lane's frame: row_base[clip] * row_unit + frame
  bool in_range, valid, fast;
};

// Where a clip's frames go: row_base[clip] * row_unit + (frame index in the
// clip). The offline layout passes the frame offsets with unit 1; the
// 30-s chunk layout passes the chunk offsets with unit 3000.
struct RowMap {
  const int64_t* __restrict__ base;
  int64_t unit;
};

// The clip that holds a tile's first frame, kept in wave-uniform registers:
// its frames [lo, hi) of the flattened frame space, its samples' range and
// its output row base. A following tile whose 32 frames all lie in [lo, hi)
// is located from these alone, with no memory access.
struct ClipCache {
  int64_t lo, hi, ss, se, rb;
};

__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t l = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t h = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)h << 32) | l);
}

__device__ __forceinline__ TileSrc locate_tile(int64_t tile, int lane,
                                               const int64_t* __restrict__ seg_start,
                                               const int64_t* __restrict__ seg_end,
                                               const int64_t* __restrict__ frame_off,
                                               RowMap rows, int64_t n_clips,
                                               int64_t total_frames, ClipCache& cc) {
  TileSrc t;
  const int64_t g0 = tile * kTile;
  t.g = g0 + (lane & 31);
  t.in_range = t.g < total_frames;
  if (cc.lo <= g0 && g0 + kTile <= cc.hi && g0 + kTile <= total_frames) {
    // all 32 frames in the cached clip (so all inside the batch)
    const int64_t f = t.g - cc.lo;
    t.s = cc.ss + 160 * f;
    t.row = cc.rb * rows.unit + f;
    t.valid = t.s + 400 <= cc.se;
    t.s0 = cc.ss + 160 * (g0 - cc.lo);
    t.fast = t.s0 + 160 * (kTile - 1) + 400 <= cc.se;
    return t;
  }
  const int64_t gq = t.in_range ? t.g : total_frames - 1;   // lookup key for idle lanes

  // A clip at or before the tile's first frame's (wave-uniform): a 64-ary
  // search for the last c with frame_off[c] <= g0 (one load per lane and one
  // ballot per level; the entries <= g0 form a prefix), stopped once at most
  // 16 candidates remain, and not run for up to 64 clips. The boundaries
  // read next, 64 from c0 on, place the remaining candidates as well (all
  // of them for up to 64 clips), so the search costs one round of loads
  // fewer, or none.
  int64_t c0 = 0;
  for (int64_t len = n_clips + 1; len > (n_clips <= kWaveLanes ? kWaveLanes + 1 : 16);) {
    const int64_t stride = (len + kWaveLanes - 1) / kWaveLanes;
    const int64_t idx = c0 + lane * stride;
    const bool le = idx < c0 + len && frame_off[idx] <= g0;
    const int cnt = __popcll(__ballot(le));
    if (cnt == 0) break;                       // frame_off[0] > g0: inconsistent offsets
    const int64_t lo = c0 + (cnt - 1) * stride;
    len = min(stride, c0 + len - lo);
    c0 = lo;
  }
  c0 = max(min(c0, n_clips - 1), (int64_t)0);
  // Then the clip of every pair: lane j holds the j-th clip boundary after
  // c0 (and clip c0 + j's sample range), and each lane counts the boundaries
  // at or below its frame (64 or more of them, a tile among runs of empty or
  // one-frame clips, take a binary search per lane instead).
  const int64_t bidx = c0 + 1 + lane;
  const int64_t B = bidx <= n_clips ? frame_off[bidx] : INT64_MAX;
  const int64_t cl = min(c0 + lane, n_clips - 1);
  const int64_t SS = seg_start[cl], SE = seg_end[cl], RB = rows.base[cl];
  const int64_t B63 = __shfl(B, 63);
  int64_t c, fo_c, ss_c, se_c, rb_c, hi_c;
  // The cross-lane search below needs every lane (__shfl reads inactive
  // lanes as garbage), so the choice is made for the whole wavefront.
  if (__any(B63 <= gq)) {
    // 64 or more clip boundaries inside this tile (runs of empty clips).
    c = upper_bound_i64(frame_off, n_clips + 1, gq) - 1;
    c = c < 0 ? 0 : (c >= n_clips ? n_clips - 1 : c);   // only inconsistent offsets need this
    fo_c = frame_off[c];
    ss_c = seg_start[c];
    se_c = seg_end[c];
    rb_c = rows.base[c];
    hi_c = fo_c;          // an empty cache: the next tile is looked up
  } else {
    int cnt = 0;
#pragma unroll
    for (int step = 32; step >= 1; step >>= 1)
      if (__shfl(B, cnt + step - 1) <= gq) cnt += step;
    c = min(c0 + cnt, n_clips - 1);            // only inconsistent offsets need the clamp
    const int j = (int)(c - c0);
    const int64_t fo_prev = __shfl(B, j > 0 ? j - 1 : 0);
    fo_c = j > 0 ? fo_prev : frame_off[c0];
    ss_c = __shfl(SS, j);
    se_c = __shfl(SE, j);
    rb_c = __shfl(RB, j);
    hi_c = __shfl(B, j);  // frame_off[c + 1], the end of the lane's clip
  }
  const int64_t f = gq - fo_c;
  t.s = ss_c + 160 * f;
  t.row = rb_c * rows.unit + f;
  // lane 0's clip is the first frame's: cache it
  cc.lo = uniform64(fo_c);
  cc.hi = uniform64(hi_c);
  cc.ss = uniform64(ss_c);
  cc.se = uniform64(se_c);
  cc.rb = uniform64(rb_c);
  // A frame is only computed if all its 400 samples lie inside its clip.
  t.valid = t.in_range && f >= 0 && (t.s + 400 <= se_c);
  t.fast = __all(t.valid && c == __shfl(c, 0));
  t.s0 = __shfl(t.s, 0);
  return t;
}


// Input types. fp32 samples as given; int16 PCM samples s mean s / 32768
// (full scale to [-1, 1), exact in fp32), so an int16 batch gives the fp32
// batch's result bit for bit.
static constexpr float kI16Scale = 1.0f / 32768.0f;

__device__ __forceinline__ float sample_value(const float* p) { return *p; }
__device__ __forceinline__ float sample_value(const int16_t* p) { return (float)*p * kI16Scale; }

// Slot t of the virtual span: samples [g, g + lim) of the batch fill its
// first lim positions (lim = 0: nothing to fetch).
struct __attribute__((aligned(16))) PieceSlot {
  int64_t g;
  int lim, pad;
};

__device__ __forceinline__ float4 load_group(const float* p) {
  const f4u t = *reinterpret_cast<const f4u*>(p);
  return make_float4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ float4 load_group(const int16_t* p) {
  return make_float4(sample_value(p), sample_value(p + 1), sample_value(p + 2), sample_value(p + 3));
}

// Slot of each lane's frame in the pieces layout, and the number of pieces
// after the first (wave-uniform). Frame f's lanes are f and f + 32, so lane
// ln - 1 holds the previous frame (for ln & 31 >= 1) and the lower 32 bits of
// a ballot hold one bit per frame.
__device__ __forceinline__ void piece_slot(const TileSrc& t, int ln, int& sigma, int& breaks) {
  const int f = ln & 31;
  const int64_t s_prev = __shfl(t.s, ln - 1);
  const bool v_prev = __shfl((int)t.valid, ln - 1) != 0;
  const bool brk = t.valid && f >= 1 && !(v_prev && t.s == s_prev + 160);
  const uint64_t bm = __ballot(brk) & 0xffffffffull;
  breaks = __popcll(bm);
  sigma = f + 2 * __popcll(bm & ((2ull << f) - 1));
}

// The fp32 value is fenced first, so that the conversion rounds the fp32
// result (the compiler would otherwise fuse the log's last multiply into a
// mixed-precision FMA rounding straight to fp16, which differs at ties).
__device__ __forceinline__ uint32_t pack_half2(float a, float b) {
  fence(a);
  fence(b);
  const _Float16 ha = (_Float16)a, hb = (_Float16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

}  // namespace logmel
