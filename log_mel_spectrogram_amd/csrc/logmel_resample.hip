// Resampling to 16 kHz on gfx950 (MI355X): band-limited interpolation with a
// Kaiser-windowed sinc. Output sample n of a clip sits at input position
// p = n R / 16000 = q + phi / L (R / 16000 = M / L in lowest terms, q integer,
// 0 <= phi < L), and is the dot product of the clip's samples
// x[q - J .. q + J] (zero outside the clip) with the phi-th row of taps,
// taps[phi][j] = h(phi / L + J - j). The host builds the taps (fp64 math,
// rounded once to fp32); see logmel_api.cpp.
//
// logmel_resample_kernel: the outputs as a matrix product on the matrix
// cores (v_mfma_f32_16x16x4f32). A clip's outputs are cut into super-periods
// of S = lcm(L, 16) outputs, which start S_in = S M / L input samples apart;
// output r of super-period sp has window start sp S_in + floor(r M / L) - J
// and phase r M mod L. Column group g holds outputs r = 16 g .. 16 g + 15;
// with base_g = floor(16 g M / L) and d = floor(r M / L) - base_g, output
// (sp, r) = sum_k W_g[k][r - 16 g] x[sp S_in + base_g - J + k], k < K, where
// W_g[k][c] is output c's tap row shifted right by its d (zeros elsewhere).
// So 16 super-periods (rows) x one column group (16 columns) is a
// 16 x K by K x 16 product: A = the staged samples, B = W_g from a table in
// the MFMA's lane layout (lane l holds B[4 s + l / 16][l % 16] for step s).
//
// Work: tiles of NT x 16 super-periods of one clip (aligned to the clip's own
// output grid, so an output always sits at the same place of the same tile
// whichever call forms it). The packed outputs are cut into windows of one
// tile's size TB (down to TB / 8 for calls of few windows); workgroup b
// forms the tiles whose first output in the call's range falls in window b
// (a clip's first tile at its first output, the others at their start), so
// every tile is formed once and clips of any length need no lookup table.
// A tile's input (zero outside the clip's
// available samples) is staged in LDS, super-period after super-period P
// floats apart (P = S_in, or S_in + 2 zero floats when 32 divides S_in, so
// that the 16 rows of an operand do not all start in one bank; the taps are
// zero at the pad floats), 8 samples per thread in flight, or 32
// for spans of 8192 floats or more (the *_wide_* instances: fewer round trips
// where the span is long, fewer registers where it is short); the 4
// wavefronts (8 in the *_8w_* instances, for tiles of 8 items or more) take
// its NT x C
// items (row block, column group) in turn, each K / 4 MFMAs with A read from
// LDS and B from the table, in chunks of 8 steps whose loads are issued one
// chunk ahead. Outputs outside the call's range are formed and dropped.
// A sample is multiplied by zero taps for the outputs of its column group
// whose window does not hold it: for finite input that leaves each output's
// sum unchanged (so a stream's outputs equal the offline ones, up to the sign
// of an exact zero), while a non-finite sample also reaches those outputs.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "logmel_resample_launch.h"

namespace logmel {

static constexpr int kRsmChunk = 8;       // MFMA steps per chunk (K / 4 is padded to a multiple)

typedef float rsm_f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float res_sample(const float* p, int64_t k) { return p[k]; }
__device__ __forceinline__ float res_sample(const int16_t* p, int64_t k) {
  return (float)p[k] * (1.0f / 32768.0f);
}

// Last index c in [0, n) with a[c] <= v (a non-decreasing, a[0] <= v), by a
// 64-ary search: one load per lane and one ballot per level.
__device__ __forceinline__ int64_t wave_last_le(const int64_t* __restrict__ a, int64_t n,
                                                int64_t v, int lane) {
  int64_t c0 = 0, len = n;
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

// One chunk of 8 MFMA steps: B (the taps, shared by the tile's row blocks)
// and, per row block, A (the samples).
template <int NT>
struct RsmChunk {
  float b[kRsmChunk];
  float a[NT][kRsmChunk];
};

template <int NT>
__device__ __forceinline__ void rsm_load(const float* __restrict__ xs, int a0, int row_stride,
                                         const float* __restrict__ bcol, int ch,
                                         RsmChunk<NT>& c) {
#pragma unroll
  for (int s = 0; s < kRsmChunk; ++s) c.b[s] = bcol[(ch * kRsmChunk + s) * 64];
#pragma unroll
  for (int rb = 0; rb < NT; ++rb)
#pragma unroll
    for (int s = 0; s < kRsmChunk; ++s)
      c.a[rb][s] = xs[a0 + rb * row_stride + 4 * (ch * kRsmChunk + s)];
}

template <int NT>
__device__ __forceinline__ void rsm_wait(RsmChunk<NT>& c) {
#pragma unroll
  for (int s = 0; s < kRsmChunk; ++s) asm volatile("" : "+v"(c.b[s]));
#pragma unroll
  for (int rb = 0; rb < NT; ++rb)
#pragma unroll
    for (int s = 0; s < kRsmChunk; ++s) asm volatile("" : "+v"(c.a[rb][s]));
}

template <int NT>
__device__ __forceinline__ void rsm_mma(const RsmChunk<NT>& c, rsm_f4 (&acc)[NT]) {
#pragma unroll
  for (int s = 0; s < kRsmChunk; ++s)
#pragma unroll
    for (int rb = 0; rb < NT; ++rb)
      acc[rb] = __builtin_amdgcn_mfma_f32_16x16x4f32(c.a[rb][s], c.b[s], acc[rb], 0, 0, 0);
}

template <int RB, int STG, int NTH, typename In>
__device__ __forceinline__ void rsm_body(const In* __restrict__ x, const int64_t* __restrict__ seg_lo,
                                         const int64_t* __restrict__ seg_hi,
                                         const int64_t* __restrict__ nfirst,
                                         const int64_t* __restrict__ out_off, int64_t n_segs,
                                         int64_t total_out, float* __restrict__ y,
                                         int64_t ystep, int64_t ybase,
                                         const float* __restrict__ btab,
                                         const int* __restrict__ abase, const RsmGeometry geo,
                                         int64_t win, float* xs) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t TB = geo.TB;
  const int64_t w0 = (int64_t)blockIdx.x * win, w1 = w0 + win;
  if (w0 >= total_out) return;
  const int chunks = geo.KS / kRsmChunk;
  const int row = lane & 15, kk = lane >> 4;

  // every wavefront finds the segment holding output w0 (the same answer)
  for (int64_t c = wave_last_le(out_off, n_segs, w0, lane); c < n_segs; ++c) {
    const int64_t o_lo = out_off[c], o_hi = out_off[c + 1];
    if (o_lo >= w1) break;
    if (o_hi <= w0 || o_hi <= o_lo) continue;
    const int64_t nf = nfirst ? nfirst[c] : 0;
    const int64_t cnt = o_hi - o_lo;
    // where the segment's outputs go: packed from y[o_lo] on, or (ystep > 0)
    // from y[c ystep + ybase] on, row c of a strided layout
    const int64_t ob = ystep > 0 ? c * ystep + ybase : o_lo;
    const int64_t j_first = nf / TB, j_last = (nf + cnt - 1) / TB;
    const int64_t lo = seg_lo[c], avail_hi = seg_hi[c];
    const int64_t avail_lo = max(lo, c > 0 ? seg_hi[c - 1] : (int64_t)0);
    // tiles of this segment whose first output here lies in [w0, w1)
    int64_t jt = (o_lo >= w0) ? j_first : max(j_first + 1, (w0 - o_lo + nf + TB - 1) / TB);
    for (; jt <= j_last; ++jt) {
      const int64_t at = jt == j_first ? o_lo : o_lo + jt * TB - nf;
      if (at >= w1) break;
      if (at < w0) continue;
      const int64_t sp0 = jt * geo.NT * 16;
      const int64_t k0 = lo + sp0 * geo.S_in - geo.J;   // buffer index of staged value 0
      __syncthreads();                                   // the previous tile's items are done
      if (STG == 8 && geo.P != geo.S_in) {
        // (narrow instances only: padded geometries stage narrow)
        // LDS float i = q P + o holds the tile's sample q S_in + o (o < S_in),
        // zero for o >= S_in and outside the available samples, which are
        // the floats [ia, ib); thread tid takes i = tid + NTH u, its (q, o)
        // stepping by (NTH / P, NTH % P)
        const int pad = geo.P - geo.S_in;
        const int64_t r_lo = max(avail_lo - k0, (int64_t)0);
        const int64_t r_hi = max(avail_hi - k0, r_lo);
        const int ia = (int)min(r_lo / geo.S_in * geo.P + r_lo % geo.S_in, (int64_t)geo.span);
        const int ib = (int)min(r_hi / geo.S_in * geo.P + r_hi % geo.S_in, (int64_t)geo.span);
        const int dq = NTH / geo.P, dq_o = NTH % geo.P;
        int q = tid / geo.P, o = tid % geo.P;   // this thread's first LDS float
        for (int i0 = 0; i0 < geo.span; i0 += 8 * NTH) {
          float v[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int i = i0 + u * NTH + tid;
            v[u] = (o < geo.S_in && i >= ia && i < ib) ? res_sample(x, k0 + (i - q * pad)) : 0.0f;
            q += dq;
            o += dq_o;
            if (o >= geo.P) {
              o -= geo.P;
              ++q;
            }
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int i = i0 + u * NTH + tid;
            if (i < geo.span) xs[i] = v[u];
          }
        }
      } else if constexpr (STG == 8) {
        for (int i0 = 0; i0 < geo.span; i0 += 8 * NTH) {
          float v[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int i = i0 + u * NTH + tid;
            const int64_t k = k0 + i;
            v[u] = (i < geo.span && k >= avail_lo && k < avail_hi) ? res_sample(x, k) : 0.0f;
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int i = i0 + u * NTH + tid;
            if (i < geo.span) xs[i] = v[u];
          }
        }
      } else {
        // STG samples per thread in flight: loads clamped into the available
        // staged indexes [ia, ib), the rest written as zero
        const int ia = (int)min(max(avail_lo - k0, (int64_t)0), (int64_t)geo.span);
        const int ib = (int)min(max(avail_hi - k0, (int64_t)ia), (int64_t)geo.span);
        for (int i0 = 0; i0 < geo.span; i0 += STG * NTH) {
          float v[STG];
#pragma unroll
          for (int u = 0; u < STG; ++u) {
            const int i = i0 + u * NTH + tid;
            v[u] = (ia < ib && i0 + u * NTH < geo.span)
                       ? res_sample(x, k0 + min(max(i, ia), ib - 1))
                       : 0.0f;
          }
#pragma unroll
          for (int u = 0; u < STG; ++u) {
            const int i = i0 + u * NTH + tid;
            if (i < geo.span) xs[i] = (i >= ia && i < ib) ? v[u] : 0.0f;
          }
        }
      }
      __syncthreads();
      // items (column group, RB row blocks), the RB blocks with one read of the taps
      const int groups = geo.NT / RB;
      for (int it = wave; it < geo.C * groups; it += NTH / 64) {
        const int gm = it / groups, rg = it - gm * groups;
        // an item with no output in the call's range (partial tiles at a
        // segment's edges: stream pushes, clip ends) is skipped
        const int64_t sp_lo = sp0 + (int64_t)rg * RB * 16;
        if ((sp_lo + RB * 16) * geo.S <= nf || sp_lo * geo.S >= nf + cnt) continue;
        const int a0 = (rg * RB * 16 + row) * geo.P + abase[gm] + kk;
        const int row_stride = 16 * geo.P;
        const float* bcol = btab + (int64_t)gm * geo.KS * 64 + lane;
        rsm_f4 acc[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) acc[rb] = rsm_f4{0.f, 0.f, 0.f, 0.f};
        RsmChunk<RB> A, B;
        rsm_load(xs, a0, row_stride, bcol, 0, A);
        rsm_wait(A);
        int ch = 0;
        for (; ch + 2 <= chunks; ch += 2) {
          rsm_load(xs, a0, row_stride, bcol, ch + 1, B);
          asm volatile("" ::: "memory");
          rsm_mma(A, acc);
          rsm_wait(B);
          rsm_load(xs, a0, row_stride, bcol, min(ch + 2, chunks - 1), A);
          asm volatile("" ::: "memory");
          rsm_mma(B, acc);
          rsm_wait(A);
        }
        if (ch < chunks) rsm_mma(A, acc);
        // lane l holds rows 4 (l / 16) + r of column l % 16
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int64_t sp = sp0 + (rg * RB + rb) * 16 + 4 * kk + r;
            const int64_t nn = sp * geo.S + 16 * gm + row;
            // offsets that overstate the output (a precondition the device
            // does not check) write nothing outside it
            const int64_t o = o_lo + (nn - nf);
            if (nn >= nf && nn < nf + cnt && o >= 0 && o < total_out) y[ob + (nn - nf)] = acc[rb][r];
          }
      }
    }
  }
}

#define LOGMEL_RESAMPLE_KERNEL(NAME, IN, RB, STG, NTH)                                           \
  extern "C" __global__ void __launch_bounds__(NTH)                                              \
  NAME(const IN* __restrict__ x, const int64_t* __restrict__ seg_lo,                            \
       const int64_t* __restrict__ seg_hi, const int64_t* __restrict__ nfirst,                  \
       const int64_t* __restrict__ out_off, int64_t n_segs, int64_t total_out,                  \
       float* __restrict__ y, int64_t ystep, int64_t ybase, const float* __restrict__ btab,     \
       const int* __restrict__ abase, RsmGeometry geo, int64_t win) {                            \
    extern __shared__ float xs[];                                                                \
    rsm_body<RB, STG, NTH, IN>(x, seg_lo, seg_hi, nfirst, out_off, n_segs, total_out, y, ystep, ybase, \
                               btab, abase, geo, win, xs);                                       \
  }

LOGMEL_RESAMPLE_KERNEL(logmel_resample_kernel, float, 1, 8, 256)
LOGMEL_RESAMPLE_KERNEL(logmel_resample_8w_kernel, float, 1, 8, 512)
LOGMEL_RESAMPLE_KERNEL(logmel_resample_i16_kernel, int16_t, 1, 8, 256)
LOGMEL_RESAMPLE_KERNEL(logmel_resample_i16_8w_kernel, int16_t, 1, 8, 512)
LOGMEL_RESAMPLE_KERNEL(logmel_resample2_kernel, float, 2, 8, 256)
LOGMEL_RESAMPLE_KERNEL(logmel_resample2_8w_kernel, float, 2, 8, 512)
LOGMEL_RESAMPLE_KERNEL(logmel_resample2_i16_kernel, int16_t, 2, 8, 256)
LOGMEL_RESAMPLE_KERNEL(logmel_resample2_i16_8w_kernel, int16_t, 2, 8, 512)
LOGMEL_RESAMPLE_KERNEL(logmel_resample_wide_kernel, float, 1, 32, 256)
LOGMEL_RESAMPLE_KERNEL(logmel_resample_wide_8w_kernel, float, 1, 32, 512)
LOGMEL_RESAMPLE_KERNEL(logmel_resample_wide_i16_kernel, int16_t, 1, 32, 256)
LOGMEL_RESAMPLE_KERNEL(logmel_resample_wide_i16_8w_kernel, int16_t, 1, 32, 512)
LOGMEL_RESAMPLE_KERNEL(logmel_resample2_wide_kernel, float, 2, 32, 256)
LOGMEL_RESAMPLE_KERNEL(logmel_resample2_wide_8w_kernel, float, 2, 32, 512)
LOGMEL_RESAMPLE_KERNEL(logmel_resample2_wide_i16_kernel, int16_t, 2, 32, 256)
LOGMEL_RESAMPLE_KERNEL(logmel_resample2_wide_i16_8w_kernel, int16_t, 2, 32, 512)

}  // namespace logmel

hipError_t logmel_launch_resample(const void* x, int in_i16, const int64_t* seg_lo,
                                  const int64_t* seg_hi, const int64_t* nfirst,
                                  const int64_t* out_off, int64_t n_segs, int64_t total_out,
                                  float* y, int64_t ystep, int64_t ybase, const float* btab,
                                  const int* abase, const RsmGeometry& geo, hipStream_t stream) {
  if (total_out <= 0 || n_segs <= 0) return hipSuccess;
  // windows of one tile's size; a call of few windows (a stream's push,
  // whose segment edges cut many partial tiles) halves them, down to TB / 8,
  // so that its tiles run in parallel workgroups
  int64_t win = geo.TB;
  for (int h = 0; h < 3 && win % 2 == 0 && (total_out + win - 1) / win < 2048; ++h) win /= 2;
  const int64_t blocks = (total_out + win - 1) / win;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const size_t lds = (size_t)geo.span * sizeof(float);
#define LOGMEL_RSM(K, IN)                                                                        \
  hipLaunchKernelGGL(logmel::K, dim3((unsigned)blocks), dim3(threads), lds, stream,         \
                     static_cast<const IN*>(x), seg_lo, seg_hi, nfirst, out_off, n_segs,         \
                     total_out, y, ystep, ybase, btab, abase, geo, win)
  // large spans: 32 staged samples per thread in flight, else 8 (fewer
  // registers, more workgroups per compute unit); 8 wavefronts per
  // workgroup when a tile has 8 items or more, else 4
  const bool wide = geo.P == geo.S_in && geo.span >= 32 * 256;
  const bool w8 = (int64_t)geo.C * (geo.NT / geo.RB) >= 8;
  const int threads = w8 ? 512 : 256;
#define LOGMEL_RSM_PICK(K, K8, IN) \
  if (w8) LOGMEL_RSM(K8, IN);       \
  else LOGMEL_RSM(K, IN)
  if (geo.RB == 2) {
    if (wide) {
      if (in_i16) { LOGMEL_RSM_PICK(logmel_resample2_wide_i16_kernel, logmel_resample2_wide_i16_8w_kernel, int16_t); }
      else { LOGMEL_RSM_PICK(logmel_resample2_wide_kernel, logmel_resample2_wide_8w_kernel, float); }
    } else {
      if (in_i16) { LOGMEL_RSM_PICK(logmel_resample2_i16_kernel, logmel_resample2_i16_8w_kernel, int16_t); }
      else { LOGMEL_RSM_PICK(logmel_resample2_kernel, logmel_resample2_8w_kernel, float); }
    }
  } else {
    if (wide) {
      if (in_i16) { LOGMEL_RSM_PICK(logmel_resample_wide_i16_kernel, logmel_resample_wide_i16_8w_kernel, int16_t); }
      else { LOGMEL_RSM_PICK(logmel_resample_wide_kernel, logmel_resample_wide_8w_kernel, float); }
    } else {
      if (in_i16) { LOGMEL_RSM_PICK(logmel_resample_i16_kernel, logmel_resample_i16_8w_kernel, int16_t); }
      else { LOGMEL_RSM_PICK(logmel_resample_kernel, logmel_resample_8w_kernel, float); }
    }
  }
#undef LOGMEL_RSM_PICK
#undef LOGMEL_RSM
  return hipGetLastError();
}
