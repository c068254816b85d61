// Resampling to 16 kHz on gfx950 (MI355X): band-limited interpolation with a
// Kaiser-windowed sinc. Output sample n of a clip sits at input position
// p = n R / 16000 = q + phi / L (R / 16000 = M / L in lowest terms, q integer,
// 0 <= phi < L), and is the dot product of the clip's samples
// x[q - J .. q + J] (zero outside the clip) with the phi-th row of taps,
// taps[phi][j] = h(phi / L + J - j). The host builds the taps (fp64 math,
// rounded once to fp32, rows zero-padded to Tp, a multiple of 16); see
// logmel_api.cpp.
//
// logmel_resample_kernel: a persistent grid of one 1024-thread workgroup per
// compute unit. The outputs of the packed batch are cut into blocks of
// 64 G periods of L outputs each (a period's outputs have the L different
// phases; inside one clip, output r of every period has the same phase). A
// workgroup stages the input samples a block's windows cover in LDS (one
// coalesced pass; int16 PCM is converted to s / 32768 on the way), then its
// 16 wavefronts take the block's (period group, phase) items in turn: lane l
// of a wavefront forms output r of period 64 g + l. All lanes of an item
// share their taps, which the wavefront reads with scalar loads straight
// into scalar registers; each lane's window starts M samples after its left
// neighbour's, so with M odd the 64 lanes' LDS reads of one tap fall on 64
// different banks. Per multiply-add: one LDS read.
// Clips are packed back to back, so a block's windows cover one contiguous
// range of the batch even when the block spans clips. A lane whose window
// crosses its clip's edge or lies beyond the staged span (blocks of many
// tiny clips) forms its output alone, masked to its clip, with its own row
// of taps; lanes of one item in different clips (different phases) take one
// pass of the shared-tap loop per phase.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "logmel_resample_launch.h"

namespace logmel {

static constexpr int kResChunk = 16;   // taps per unrolled step

__device__ __forceinline__ float res_sample(const float* p, int64_t k) { return p[k]; }
__device__ __forceinline__ float res_sample(const int16_t* p, int64_t k) {
  return (float)p[k] * (1.0f / 32768.0f);
}

// Last index c in [0, n) with a[c] <= v (a non-decreasing, a[0] <= v).
__device__ __forceinline__ int64_t last_le(const int64_t* __restrict__ a, int64_t n, int64_t v) {
  int64_t lo = 0, hi = n;   // answer in [lo, hi)
  while (hi - lo > 1) {
    const int64_t mid = lo + ((hi - lo) >> 1);
    if (a[mid] <= v) lo = mid; else hi = mid;
  }
  return lo;
}

// floor(a / L) for 0 <= a: an fp64 estimate off by at most one below 2^52,
// corrected; larger values divide exactly.
__device__ __forceinline__ int64_t div_by(int64_t a, int L, double inv_L) {
  if (a >= (int64_t(1) << 52)) return a / L;
  int64_t q = (int64_t)((double)a * inv_L);
  const int64_t rem = a - q * L;
  if (rem < 0) q -= 1;
  else if (rem >= L) q += 1;
  return q;
}

// Segment c of the batch: its samples lie at [lo[c], hi[c]) of x, sample 0
// of its clip at lo[c] (zero before lo and from hi on), and its outputs,
// [out_off[c], out_off[c + 1]) of y, are the clip's outputs nfirst[c],
// nfirst[c] + 1, ... (nfirst null: from 0). An offline batch passes its
// sample offsets as lo (and, shifted by one, as hi); a stream passes the
// segment of each stream's retained and new samples.
struct ResSegs {
  const int64_t* __restrict__ lo;
  const int64_t* __restrict__ hi;
  const int64_t* __restrict__ nfirst;
  const int64_t* __restrict__ out_off;
  int64_t n;
};

// A lane's current segment: its index, output range [o_lo, o_hi), first
// output number nf and sample range [lo, hi). A lane's successive outputs
// usually stay in one segment, so it is looked up again only when an output
// leaves it.
struct ResClip {
  int64_t c, o_lo, o_hi, nf, lo, hi;
};

__device__ __forceinline__ ResClip res_clip(int64_t g, const ResSegs& sg) {
  ResClip r;
  r.c = last_le(sg.out_off, sg.n, g);
  r.o_lo = sg.out_off[r.c];
  r.o_hi = sg.out_off[r.c + 1];
  r.nf = sg.nfirst ? sg.nfirst[r.c] : 0;
  r.lo = sg.lo[r.c];
  r.hi = sg.hi[r.c];
  return r;
}

// Where output g (inside clip cl) comes from: the global index k0 of its
// window's first sample, and its phase.
struct ResSrc {
  int64_t c, lo, hi, k0;
  int phi;
};

__device__ __forceinline__ ResSrc res_pos(int64_t g, const ResClip& cl, int L, int M, int J,
                                          double inv_L) {
  ResSrc s;
  s.c = cl.c;
  s.lo = cl.lo;
  s.hi = cl.hi;
  const int64_t nm = (cl.nf + g - cl.o_lo) * M;
  const int64_t q = div_by(nm, L, inv_L);
  s.phi = (int)(nm - q * L);
  s.k0 = cl.lo + q - J;
  return s;
}

// The same lookup by a whole wavefront (g uniform): a 64-ary search, one
// load per lane and one ballot per level. Returns the last c in [0, n)
// with a[c] <= g.
__device__ __forceinline__ int64_t wave_last_le(const int64_t* __restrict__ a, int64_t n,
                                                int64_t v, int lane) {
  int64_t c0 = 0, len = n;   // answer in [c0, c0 + len); a[c0] <= v
  while (len > 1) {
    const int64_t stride = (len + 63) / 64;
    const int64_t idx = c0 + lane * stride;
    const bool le = idx < c0 + len && a[idx] <= v;
    const int cnt = __popcll(__ballot(le));
    const int64_t lo = c0 + (int64_t)(cnt - 1) * stride;
    len = min(stride, c0 + len - lo);
    c0 = lo;
  }
  return c0;
}

__device__ __forceinline__ int64_t wave_k0(int64_t g, const ResSegs& sg, int L, int M, int J,
                                           double inv_L, int lane) {
  const int64_t c = wave_last_le(sg.out_off, sg.n, g, lane);
  const int64_t nm = ((sg.nfirst ? sg.nfirst[c] : 0) + g - sg.out_off[c]) * M;
  return sg.lo[c] + div_by(nm, L, inv_L) - J;
}

// One output alone, with its own row of taps; samples outside [lo, hi) are
// zero; from the staged span when it holds the window, else from memory.
// The sums run in the order of the shared-tap loop (odd taps of whole
// 16-tap chunks in a second sum), so a whole window gives the same bits on
// either path.
template <typename In>
__device__ __forceinline__ float res_one(const ResSrc& s, const float* __restrict__ taps, int Tp,
                                         int T, const float* span, int64_t s0, int span_len,
                                         const In* __restrict__ x) {
  const float* tp = taps + (int64_t)s.phi * Tp;
  const int jlo = (int)max((int64_t)0, s.lo - s.k0);
  const int jhi = (int)min((int64_t)T, s.hi - s.k0);
  const int whole = (T / kResChunk) * kResChunk;
  const int64_t off = s.k0 - s0;
  const bool staged = off + jlo >= 0 && off + jhi <= span_len;
  float a0 = 0.0f, a1 = 0.0f;
  for (int j = jlo; j < jhi; ++j) {
    const float v = staged ? span[off + j] : res_sample(x, s.k0 + j);
    if (j < whole && (j & 1)) a1 = __builtin_fmaf(tp[j], v, a1);
    else a0 = __builtin_fmaf(tp[j], v, a0);
  }
  return a0 + a1;
}

// 16 taps (scalar registers) and 16 samples (vector registers) of a chunk.
struct ResChunk {
  float t[kResChunk];
  float v[kResChunk];
};

__device__ __forceinline__ void res_load(const __attribute__((address_space(4))) float* trow,
                                         const float* sp, int ch, ResChunk& c) {
#pragma unroll
  for (int j = 0; j < kResChunk; ++j) {
    c.t[j] = trow[ch * kResChunk + j];
    c.v[j] = sp[ch * kResChunk + j];
  }
}

// Ties every value of a chunk to this point, so that its loads are all
// issued before and waited here, in one wait.
__device__ __forceinline__ void res_wait(ResChunk& c) {
#pragma unroll
  for (int j = 0; j < kResChunk; j += 4)
    asm volatile("" : "+s"(c.t[j]), "+s"(c.t[j + 1]), "+s"(c.t[j + 2]), "+s"(c.t[j + 3]),
                      "+v"(c.v[j]), "+v"(c.v[j + 1]), "+v"(c.v[j + 2]), "+v"(c.v[j + 3]));
}

__device__ __forceinline__ void res_fma(const ResChunk& c, float& a0, float& a1) {
#pragma unroll
  for (int j = 0; j < kResChunk; j += 2) {
    a0 = __builtin_fmaf(c.t[j], c.v[j], a0);
    a1 = __builtin_fmaf(c.t[j + 1], c.v[j + 1], a1);
  }
}

template <typename In>
__device__ __forceinline__ void resample_body(const In* __restrict__ x,
                                              const ResSegs sg, int64_t total_out,
                                              float* __restrict__ y,
                                              const float* __restrict__ taps, int L, int M, int J,
                                              int Tp, int G, float* span, int64_t* bounds) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n_waves = blockDim.x >> 6;
  const int T = 2 * J + 1;
  const double inv_L = 1.0 / L;
  const int64_t total_in = sg.hi[sg.n - 1];   // the last segment ends the buffer
  const int64_t per_block = (int64_t)64 * G * L;
  const int items = G * L;

  for (int64_t g0 = (int64_t)blockIdx.x * per_block; g0 < total_out;
       g0 += (int64_t)gridDim.x * per_block) {
    // The block's windows run from its first output's first sample to its
    // last output's last (window starts never decrease along the outputs).
    const int64_t g_last = min(g0 + per_block, total_out) - 1;
    __syncthreads();                          // the previous block's span is consumed
    if (wave == 0) {
      const int64_t k_first = wave_k0(g0, sg, L, M, J, inv_L, lane);
      const int64_t k_last = wave_k0(g_last, sg, L, M, J, inv_L, lane);
      if (lane == 0) {
        bounds[0] = k_first;
        bounds[1] = k_last + Tp;
      }
    }
    __syncthreads();
    const int64_t s0 = bounds[0];
    const int span_len = (int)min(max(bounds[1] - s0, (int64_t)0), (int64_t)kResLdsFloats);
    for (int i = tid; i < span_len; i += blockDim.x) {
      const int64_t k = s0 + i;
      span[i] = (k >= 0 && k < total_in) ? res_sample(x, k) : 0.0f;
    }
    __syncthreads();

    ResClip cl{-1, 0, -1, 0, 0, 0};
    // items it = wave, wave + n_waves, ... as (period group gi, phase r)
    // with it = gi L + r, stepped without a division
    int gi = wave / L, r = wave - (wave / L) * L;
    const int step_q = n_waves / L, step_r = n_waves - (n_waves / L) * L;
    for (int it = wave; it < items; it += n_waves) {
      if (it != wave) {
        gi += step_q;
        r += step_r;
        if (r >= L) {
          r -= L;
          ++gi;
        }
      }
      const int64_t g = g0 + (int64_t)(gi * 64 + lane) * L + r;
      const bool active = g < total_out;
      ResSrc s{};
      bool ok = false;
      int64_t off = 0;
      if (active) {
        if (!(cl.o_lo <= g && g < cl.o_hi)) cl = res_clip(g, sg);
        s = res_pos(g, cl, L, M, J, inv_L);
        off = s.k0 - s0;
        ok = s.k0 >= s.lo && s.k0 + T <= s.hi && off >= 0 && off + Tp <= span_len;
      }
      // The lanes with a whole window, one phase at a time (one pass unless
      // the item's outputs lie in several clips): the first waiting lane's
      // phase, shared by the lanes that have it.
      uint64_t waiting = __ballot(ok);
      while (waiting) {
        const int lead = __builtin_ctzll(waiting);
        const int phi_w = __builtin_amdgcn_readlane(s.phi, lead);
        const bool mine = ok && s.phi == phi_w;
        waiting &= ~__ballot(mine);
        if (mine) {
          // The lanes here all have phase phi_w: the row address is uniform
          // (taken with readfirstlane, so that it stays scalar), read through
          // the constant address space, so the taps load with scalar loads
          // into scalar registers.
          const int pu = __builtin_amdgcn_readfirstlane(s.phi);
          const __attribute__((address_space(4))) float* trow =
              (const __attribute__((address_space(4))) float*)(taps + (int64_t)pu * Tp);
          const float* sp = span + off;
          float a0 = 0.0f, a1 = 0.0f;
          const int full = T / kResChunk;
          // Software pipeline over chunks of 16 taps, two buffers: the next
          // chunk's taps (scalar loads) and samples (LDS reads) are issued
          // before this chunk's multiply-adds and waited after them (scalar
          // loads return out of order, so one wait covers both kinds).
          ResChunk A, B;
          res_load(trow, sp, 0, A);
          res_wait(A);
          int ch = 0;
          for (; ch + 2 <= full; ch += 2) {
            res_load(trow, sp, ch + 1, B);
            asm volatile("" ::: "memory");
            res_fma(A, a0, a1);
            res_wait(B);
            res_load(trow, sp, min(ch + 2, full - 1), A);
            asm volatile("" ::: "memory");
            res_fma(B, a0, a1);
            res_wait(A);
          }
          if (ch < full) res_fma(A, a0, a1);
          // the last chunk: samples past the window's T taps are not read
          const int base = full * kResChunk;
#pragma unroll
          for (int j = 0; j < kResChunk; ++j)
            if (base + j < T) a0 = __builtin_fmaf(trow[base + j], sp[base + j], a0);
          y[g] = a0 + a1;
        }
      }
      if (active && !ok) y[g] = res_one(s, taps, Tp, T, span, s0, span_len, x);
    }
  }
}

#define LOGMEL_RESAMPLE_KERNEL(NAME, IN)                                                         \
  extern "C" __global__ void __launch_bounds__(1024)                                             \
  NAME(const IN* __restrict__ x, const int64_t* __restrict__ seg_lo,                            \
       const int64_t* __restrict__ seg_hi, const int64_t* __restrict__ nfirst,                  \
       const int64_t* __restrict__ out_off, int64_t n_segs, int64_t total_out,                  \
       float* __restrict__ y, const float* __restrict__ taps, int L, int M, int J, int Tp,       \
       int G) {                                                                                  \
    __shared__ float span[kResLdsFloats];                                                        \
    __shared__ int64_t bounds[2];                                                                \
    const ResSegs sg{seg_lo, seg_hi, nfirst, out_off, n_segs};                                   \
    resample_body<IN>(x, sg, total_out, y, taps, L, M, J, Tp, G, span, bounds);                 \
  }

LOGMEL_RESAMPLE_KERNEL(logmel_resample_kernel, float)
LOGMEL_RESAMPLE_KERNEL(logmel_resample_i16_kernel, int16_t)

}  // namespace logmel

hipError_t logmel_launch_resample(const void* x, int in_i16, const int64_t* seg_lo,
                                  const int64_t* seg_hi, const int64_t* nfirst,
                                  const int64_t* out_off, int64_t n_segs, int64_t total_out,
                                  float* y, const float* taps, int L, int M, int J, int Tp, int G,
                                  int grid, hipStream_t stream) {
  if (total_out <= 0 || n_segs <= 0) return hipSuccess;
  const int64_t per_block = (int64_t)64 * G * L;
  const int64_t blocks = (total_out + per_block - 1) / per_block;
  const int g = (int)(blocks < grid ? blocks : grid);
  if (in_i16)
    hipLaunchKernelGGL(logmel::logmel_resample_i16_kernel, dim3(g), dim3(1024), 0, stream,
                       static_cast<const int16_t*>(x), seg_lo, seg_hi, nfirst, out_off, n_segs,
                       total_out, y, taps, L, M, J, Tp, G);
  else
    hipLaunchKernelGGL(logmel::logmel_resample_kernel, dim3(g), dim3(1024), 0, stream,
                       static_cast<const float*>(x), seg_lo, seg_hi, nfirst, out_off, n_segs,
                       total_out, y, taps, L, M, J, Tp, G);
  return hipGetLastError();
}
