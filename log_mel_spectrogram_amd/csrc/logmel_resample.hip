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
// compute unit. Each lane forms NB consecutive outputs (NB = 4 for every
// common rate but the integer ratios with M odd, 48 kHz among them, where it
// is 3), reading each sample of their windows' union from LDS once and
// multiplying it into the NB sums. Lane l of item (gi, b) takes outputs
// g0 + (64 gi + l) Q + NB b + a, a < NB, where Q = L when NB divides L (a
// lane's outputs are NB of one period's L) and Q = NB when L divides NB
// (integer ratios: a lane's outputs are NB / L whole periods); either way
// all lanes of an item inside one clip have the same first phase, hence the
// same NB tap rows and the same window offsets. The outputs of the packed
// batch are cut into blocks of 64 G lanes; a workgroup stages the input
// samples a block's windows cover in LDS (coalesced, sixteen loads in flight
// per thread; int16 PCM converted to s / 32768 on the way), then its 16
// wavefronts take the block's items in turn. The taps of an item come from
// the shared path's table, NB rows per first phase, each shifted right by
// its window's offset and zero elsewhere, read with scalar loads into scalar
// registers; lanes' windows start Q M / L samples apart, so when that is odd
// the 64 lanes' LDS reads of one sample fall on 64 different banks.
// Per NB multiply-adds: one LDS read.
// Clips are packed back to back, so a block's windows cover one contiguous
// range of the batch even when the block spans clips. A lane whose NB
// outputs are not all in one clip, or whose windows' union crosses its
// clip's edge or lies beyond the staged span (blocks of many tiny clips),
// forms each output alone, masked to its clip, with its own row of taps;
// lanes of one item in different clips (different first phases) take one
// pass of the shared loop per phase.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "logmel_resample_launch.h"

namespace logmel {


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

// One output alone, with its own row of taps: the plain sum, in tap order,
// of the window's samples inside [lo, hi) times their taps; from the staged
// span when it holds the window, else from memory. The shared path below
// adds the same products in the same order (plus products with zero taps,
// which leave every nonzero sum unchanged), so an output gets the same
// value on either path.
template <typename In>
__device__ __forceinline__ float res_one(const ResSrc& s, const float* __restrict__ taps, int Tp,
                                         int T, const float* span, int64_t s0, int span_len,
                                         const In* __restrict__ x) {
  const float* tp = taps + (int64_t)s.phi * Tp;
  const int jlo = (int)max((int64_t)0, s.lo - s.k0);
  const int jhi = (int)min((int64_t)T, s.hi - s.k0);
  const int64_t off = s.k0 - s0;
  const bool staged = off + jlo >= 0 && off + jhi <= span_len;
  float a = 0.0f;
  for (int j = jlo; j < jhi; ++j) {
    const float v = staged ? span[off + j] : res_sample(x, s.k0 + j);
    a = __builtin_fmaf(tp[j], v, a);
  }
  return a;
}

// A chunk of CH samples (vector registers) and, for each of the NB outputs,
// CH taps (scalar registers).
// 16 bytes at a 4-byte aligned address (global memory allows this).
struct __attribute__((packed, aligned(4))) f4u {
  float x, y, z, w;
};

template <int NB, int CH>
struct ResChunk {
  float t[NB][CH];
  float v[CH];
};

// The chunk's NB x CH taps are consecutive in the table (sample-major), one
// or two scalar loads.
template <int NB, int CH>
__device__ __forceinline__ void res_load(const __attribute__((address_space(4))) float* trow,
                                         const float* sp, int ch, ResChunk<NB, CH>& c) {
#pragma unroll
  for (int j = 0; j < CH; ++j) c.v[j] = sp[ch * CH + j];
#pragma unroll
  for (int j = 0; j < CH; ++j)
#pragma unroll
    for (int a = 0; a < NB; ++a) c.t[a][j] = trow[(ch * CH + j) * NB + a];
}

// Ties every value of a chunk to this point, so that its loads are all
// issued before and waited here, in one wait.
template <int NB, int CH>
__device__ __forceinline__ void res_wait(ResChunk<NB, CH>& c) {
#pragma unroll
  for (int j = 0; j < CH; ++j) asm volatile("" : "+v"(c.v[j]));
#pragma unroll
  for (int a = 0; a < NB; ++a)
#pragma unroll
    for (int j = 0; j < CH; ++j) asm volatile("" : "+s"(c.t[a][j]));
}

template <int NB, int CH>
__device__ __forceinline__ void res_fma(const ResChunk<NB, CH>& c, float (&acc)[NB]) {
#pragma unroll
  for (int j = 0; j < CH; ++j)
#pragma unroll
    for (int a = 0; a < NB; ++a) acc[a] = __builtin_fmaf(c.t[a][j], c.v[j], acc[a]);
}

// Output g's clip and source (its segment looked up again only when g leaves
// the cached one).
__device__ __forceinline__ ResSrc res_at(int64_t g, ResClip& cl, const ResSegs& sg, int L, int M,
                                         int J, double inv_L) {
  if (!(cl.o_lo <= g && g < cl.o_hi)) cl = res_clip(g, sg);
  return res_pos(g, cl, L, M, J, inv_L);
}

// NB consecutive outputs per lane. Lane l of item (gi, b) forms outputs
// g0 + (64 gi + l) Q + NB b + a, a < NB (Q = L when NB divides L, else NB,
// which L divides), so all lanes of an item in one clip have the same first
// phase phi, and their outputs' windows start at offsets
// d_a = floor((phi + a M) / L) from the first's: the union of the NB windows
// is U = 2J + 1 + d_{NB-1} samples. taps_blk holds, for every first phase,
// TpX groups of NB taps: group s, tap a is output a's tap for the union's
// sample s (output a's row shifted right by d_a, zeros elsewhere), so each
// staged sample is read once and multiplied into the NB sums.
template <int NB, int CH, typename In>
__device__ __forceinline__ void resample_body(const In* __restrict__ x,
                                              const ResSegs sg, int64_t total_out,
                                              float* __restrict__ y,
                                              const float* __restrict__ taps,
                                              const float* __restrict__ taps_blk, int L, int M,
                                              int J, int Tp, int TpX, int Ur, int Q, int G,
                                              float* span, int64_t* bounds) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n_waves = blockDim.x >> 6;
  const int T = 2 * J + 1;
  const double inv_L = 1.0 / L;
  const int64_t total_in = sg.hi[sg.n - 1];   // the last segment ends the buffer
  const int64_t per_block = (int64_t)64 * G * Q;
  const int nb_per = Q / NB;                  // output blocks per lane stride
  const int items = G * nb_per;

  for (int64_t g0 = (int64_t)blockIdx.x * per_block; g0 < total_out;
       g0 += (int64_t)gridDim.x * per_block) {
    // The block's windows run from its first output's first sample to its
    // last output's (window starts never decrease along the outputs).
    const int64_t g_last = min(g0 + per_block, total_out) - 1;
    __syncthreads();                          // the previous block's span is consumed
    if (wave == 0) {
      const int64_t k_first = wave_k0(g0, sg, L, M, J, inv_L, lane);
      const int64_t k_last = wave_k0(g_last, sg, L, M, J, inv_L, lane);
      if (lane == 0) {
        bounds[0] = k_first;
        bounds[1] = k_last + TpX;
      }
    }
    __syncthreads();
    const int64_t s0 = bounds[0];
    const int span_len = (int)min(max(bounds[1] - s0, (int64_t)0), (int64_t)kResLdsFloats);
    // coalesced, sixteen loads in flight per thread before the first store
    for (int i0 = 0; i0 < span_len; i0 += 16 * 1024) {
      float v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int i = i0 + u * 1024 + tid;
        const int64_t k = s0 + i;
        v[u] = (i < span_len && k >= 0 && k < total_in) ? res_sample(x, k) : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int i = i0 + u * 1024 + tid;
        if (i < span_len) span[i] = v[u];
      }
    }
    __syncthreads();

    ResClip cl{-1, 0, -1, 0, 0, 0};
    // items it = wave, wave + n_waves, ... as (lane group gi, output block b)
    // with it = gi nb_per + b, stepped without a division
    int gi = wave / nb_per, b = wave - (wave / nb_per) * nb_per;
    const int step_q = n_waves / nb_per, step_r = n_waves - (n_waves / nb_per) * nb_per;
    for (int it = wave; it < items; it += n_waves) {
      if (it != wave) {
        gi += step_q;
        b += step_r;
        if (b >= nb_per) {
          b -= nb_per;
          ++gi;
        }
      }
      const int64_t g = g0 + (int64_t)(gi * 64 + lane) * Q + NB * b;
      const bool active = g < total_out;
      ResSrc s{};
      bool ok = false;
      int64_t off = 0;
      if (active) {
        s = res_at(g, cl, sg, L, M, J, inv_L);
        off = s.k0 - s0;
        ok = g + NB <= cl.o_hi && s.k0 >= s.lo && s.k0 + Ur <= s.hi && off >= 0 &&
             off + Ur <= span_len;
      }
      // The lanes whose NB windows are whole, one first phase at a time (one
      // pass unless the item's outputs lie in several clips): the first
      // waiting lane's phase, shared by the lanes that have it.
      uint64_t waiting = __ballot(ok);
      while (waiting) {
        const int lead = __builtin_ctzll(waiting);
        const int phi_w = __builtin_amdgcn_readlane(s.phi, lead);
        const bool mine = ok && s.phi == phi_w;
        waiting &= ~__ballot(mine);
        if (mine) {
          // The row block's address is uniform (taken with readfirstlane, so
          // that it stays scalar) and read through the constant address
          // space: the taps load with scalar loads into scalar registers.
          const int pu = __builtin_amdgcn_readfirstlane(s.phi);
          const __attribute__((address_space(4))) float* trow =
              (const __attribute__((address_space(4))) float*)(taps_blk +
                                                                (int64_t)pu * NB * TpX);
          const float* sp = span + off;
          float acc[NB];
#pragma unroll
          for (int a = 0; a < NB; ++a) acc[a] = 0.0f;
          const int full = Ur / CH;
          // Two chunks per step: both chunks' taps (scalar loads) and samples
          // (LDS reads) are issued, then waited for once; the wavefronts on
          // the other SIMDs' slots cover the wait.
          ResChunk<NB, CH> A, B, C, D;
          int ch = 0;
          for (; ch + 4 <= full; ch += 4) {
            res_load(trow, sp, ch, A);
            res_load(trow, sp, ch + 1, B);
            res_load(trow, sp, ch + 2, C);
            res_load(trow, sp, ch + 3, D);
            res_wait(A);
            res_wait(B);
            res_wait(C);
            res_wait(D);
            res_fma(A, acc);
            res_fma(B, acc);
            res_fma(C, acc);
            res_fma(D, acc);
          }
          for (; ch + 2 <= full; ch += 2) {
            res_load(trow, sp, ch, A);
            res_load(trow, sp, ch + 1, B);
            res_wait(A);
            res_wait(B);
            res_fma(A, acc);
            res_fma(B, acc);
          }
          if (ch < full) {
            res_load(trow, sp, ch, A);
            res_wait(A);
            res_fma(A, acc);
          }
          if (NB == 4) {
            *reinterpret_cast<f4u*>(y + g) = f4u{acc[0], acc[1], acc[2], acc[3]};
          } else {
#pragma unroll
            for (int a = 0; a < NB; ++a) y[g + a] = acc[a];
          }
        }
      }
      if (active && !ok) {
        // each output alone (its own segment, phase and window)
        for (int a = 0; a < NB; ++a) {
          const int64_t ga = g + a;
          if (ga < total_out) {
            const ResSrc sa = res_at(ga, cl, sg, L, M, J, inv_L);
            y[ga] = res_one(sa, taps, Tp, T, span, s0, span_len, x);
          }
        }
      }
    }
  }
}

#define LOGMEL_RESAMPLE_KERNEL(NAME, IN, NB, CH)                                                 \
  extern "C" __global__ void __launch_bounds__(1024)                                             \
  NAME(const IN* __restrict__ x, const int64_t* __restrict__ seg_lo,                            \
       const int64_t* __restrict__ seg_hi, const int64_t* __restrict__ nfirst,                  \
       const int64_t* __restrict__ out_off, int64_t n_segs, int64_t total_out,                  \
       float* __restrict__ y, const float* __restrict__ taps,                                   \
       const float* __restrict__ taps_blk, int L, int M, int J, int Tp, int TpX, int Ur, int Q,  \
       int G) {                                                                                  \
    __shared__ float span[kResLdsFloats];                                                        \
    __shared__ int64_t bounds[2];                                                                \
    const ResSegs sg{seg_lo, seg_hi, nfirst, out_off, n_segs};                                   \
    resample_body<NB, CH, IN>(x, sg, total_out, y, taps, taps_blk, L, M, J, Tp, TpX, Ur, Q, G,   \
                              span, bounds);                                                     \
  }

LOGMEL_RESAMPLE_KERNEL(logmel_resample_kernel, float, 4, 4)
LOGMEL_RESAMPLE_KERNEL(logmel_resample_i16_kernel, int16_t, 4, 4)
LOGMEL_RESAMPLE_KERNEL(logmel_resample3_kernel, float, 3, 4)
LOGMEL_RESAMPLE_KERNEL(logmel_resample3_i16_kernel, int16_t, 3, 4)
LOGMEL_RESAMPLE_KERNEL(logmel_resample2_kernel, float, 2, 8)
LOGMEL_RESAMPLE_KERNEL(logmel_resample2_i16_kernel, int16_t, 2, 8)
LOGMEL_RESAMPLE_KERNEL(logmel_resample1_kernel, float, 1, 16)
LOGMEL_RESAMPLE_KERNEL(logmel_resample1_i16_kernel, int16_t, 1, 16)

}  // namespace logmel

hipError_t logmel_launch_resample(const void* x, int in_i16, const int64_t* seg_lo,
                                  const int64_t* seg_hi, const int64_t* nfirst,
                                  const int64_t* out_off, int64_t n_segs, int64_t total_out,
                                  float* y, const float* taps, const float* taps_blk, int L, int M,
                                  int J, int Tp, int TpX, int NB, int Q, int G, int grid,
                                  hipStream_t stream) {
  if (total_out <= 0 || n_segs <= 0) return hipSuccess;
  const int64_t per_block = (int64_t)64 * G * Q;
  // every lane of the shared path reads Ur samples: the largest union of NB
  // windows rounded up to its chunk (taps beyond a phase's own union are zero)
  const int CH = NB == 3 ? 4 : 16 / NB;
  const int64_t d_max = (L - 1 + (int64_t)(NB - 1) * M) / L;
  const int Ur = (int)((2 * J + 1 + d_max + CH - 1) / CH * CH);
  const int64_t blocks = (total_out + per_block - 1) / per_block;
  const int g = (int)(blocks < grid ? blocks : grid);
#define LOGMEL_RES_LAUNCH(K, IN)                                                                \
  hipLaunchKernelGGL(logmel::K, dim3(g), dim3(1024), 0, stream, static_cast<const IN*>(x), seg_lo, \
                     seg_hi, nfirst, out_off, n_segs, total_out, y, taps, taps_blk, L, M, J, Tp,  \
                     TpX, Ur, Q, G)
  if (NB == 4) {
    if (in_i16) LOGMEL_RES_LAUNCH(logmel_resample_i16_kernel, int16_t);
    else LOGMEL_RES_LAUNCH(logmel_resample_kernel, float);
  } else if (NB == 3) {
    if (in_i16) LOGMEL_RES_LAUNCH(logmel_resample3_i16_kernel, int16_t);
    else LOGMEL_RES_LAUNCH(logmel_resample3_kernel, float);
  } else if (NB == 2) {
    if (in_i16) LOGMEL_RES_LAUNCH(logmel_resample2_i16_kernel, int16_t);
    else LOGMEL_RES_LAUNCH(logmel_resample2_kernel, float);
  } else {
    if (in_i16) LOGMEL_RES_LAUNCH(logmel_resample1_i16_kernel, int16_t);
    else LOGMEL_RES_LAUNCH(logmel_resample1_kernel, float);
  }
#undef LOGMEL_RES_LAUNCH
  return hipGetLastError();
}
