// The log-mel transform kernel on four lanes per frame (gfx950, MI355X):
// logmel_quad_kernel and its int16-input / fp16-output instances.
//
// A workgroup of two wavefronts takes tiles of 32 consecutive frames of the
// flattened frame space (the steps of the page "从零理解 ASR：音频基础、
// Qwen3-ASR 架构，以及离线 vs 流式推理原理", §2.3: framing 400/160,
// symmetric Hamming window, 400-point real FFT, power, 128 mel filters, log).
// Frame f of a tile sits on lanes 2f and 2f + 1 of both wavefronts. Its
// windowed samples y[n] = w[n] x[n] are split four ways by n mod 4, each
// lane taking 100 of them (decimation in time):
//   wavefront 0, role 0: s[m] = y[4m]          (class 0)
//   wavefront 0, role 1: s[m] = y[399 - 4m]    (class 3, reversed)
//   wavefront 1, role 0: s[m] = y[4m + 1]      (class 1)
//   wavefront 1, role 1: s[m] = y[398 - 4m]    (class 2, reversed)
// The window is symmetric (w[399 - n] = w[n]), so both lanes of a pair use
// the window values w[4m + c] of their wavefront c, and every constant of a
// wavefront's code is uniform. Each lane computes the 100-point real DFT S
// of its samples in fp64 as a prime-factor 4 x 25 transform
//   m = (25 n1 + 4 n2) mod 100,  k = (25 k1 + 76 k2) mod 100,
// (four real 25-point DFTs, then 4-point DFTs over n1), for the bins
// kappa = 0..50 (the rest are conjugates). With X_r the natural-order
// spectrum of class r, the frame's spectrum is
//   X[kappa + 100 j] = sum_r W400^{r kappa} (-i)^{r j} X_r[kappa],
// and the reversed classes give X_3 = W100^-kappa conj(S), X_2 likewise.
// Rotating each lane's S by W800^{(2c + 1) kappa} (the same for both lanes
// of a wavefront) turns the four terms into U_0, conj(U_3), U_1, conj(U_2)
// up to a phase common to all four, so that with
//   G = (s own.re + p.re, own.im - s p.im),  F = (own.re + s p.im, own.im + s p.re)
// (own this lane's U, p its partner's, s = +1 for role 0 and -1 for role 1)
// the four outputs j = 0..3 at a bin kappa are, up to unit factors,
//   G + s G',  F - conj(F'')
// where G' is the other wavefront's role-s lane's G and F'' its other
// lane's F. The power |X|^2 needs no phase, so each lane forms two of the
// four powers of a bin: wavefront 0 those of kappa = 0..25, wavefront 1 of
// kappa = 25..50 (kappa 25 by both, with identical values). The other
// wavefront's U reach a lane through LDS, its partner's by DPP.
//
// The powers (fp32, each rounded once from fp64) go through LDS; wavefront
// 0 forms the mel bands 0..87 and wavefront 1 the bands 88..127, both lanes
// of a frame the same sums, each logging and storing half of them.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "logmel_frame.h"
#include "logmel_launch.h"
#include "logmel_tile.h"

namespace logmel {
namespace quad {

static constexpr int kThreads = 128;
static constexpr int kSpanQ = (kTile - 1) * 160 + 400;   // 5360 samples
// Tiles across clips are staged as a virtual span of pieces (below): at most
// kPassPieces pieces per pass, hop slots 0..kMaxSlots - 1.
static constexpr int kPassPieces = 7;
static constexpr int kMaxSlots = kTile + 2 * (kPassPieces - 1) + 2;   // 46
static constexpr int kPieceCols = 10 * (kMaxSlots - 1) + 5;          // 455 columns
// The span in LDS: 16 rows, row r holding samples n = 16 col + r of the span
// (so frame f's samples of one residue mod 16 are 25 consecutive columns
// from 10 f). Rows are stored in the order the lanes read them:
//   slots 0..3  rows 0, 4, 8, 12    (class 0, row n1 at slot n1)
//   slots 4..7  rows 15, 11, 7, 3   (class 3), columns reversed
//   slots 8..11 rows 1, 5, 9, 13    (class 1)
//   slots 12..15 rows 14, 10, 6, 2  (class 2), columns reversed
// A reversed row holds column col at position kCmax - col.
static constexpr int kRS = 464;    // row stride (floats): 16 mod 64 spreads 16-byte writes
static constexpr int kCmax = 463;  // 3 mod 4: reversed 16-byte groups stay aligned
static_assert(kPieceCols <= kRS && kRS % 64 == 16 && kCmax % 4 == 3, "span layout");
// The powers in LDS, per frame: four regions of bins, kappa at position
// kappa (kappa <= 25, written by wavefront 0) or kappa + 3 (kappa >= 26,
// written by wavefront 1): region 0 bin kappa, 1 bin 200 - kappa, 2 bin
// 100 + kappa, 3 bin 100 - kappa.
static constexpr int kPReg = 56;
static constexpr int kPFS = 4 * kPReg + 4;   // 228 floats per frame
// LDS shared by the span, the exchange and the powers (one at a time)
static constexpr int kRegionFloats = 16 * kRS;   // 7424 floats
static_assert(kTile * kPFS <= kRegionFloats, "the powers fit the region");
static constexpr int kXchSlots = 13;              // bins per exchange round
static_assert(kXchSlots * 2 * 64 * 4 <= kRegionFloats, "exchange fits the region");

__host__ __device__ constexpr int slot_row(int slot) {
  return slot < 4 ? 4 * slot : slot < 8 ? 15 - 4 * (slot - 4)
       : slot < 12 ? 4 * (slot - 8) + 1 : 14 - 4 * (slot - 12);
}
__host__ __device__ constexpr int row_slot(int r) {
  return (r & 3) == 0 ? r / 4 : (r & 3) == 3 ? 4 + (15 - r) / 4
       : (r & 3) == 1 ? 8 + (r - 1) / 4 : 12 + (14 - r) / 4;
}
__host__ __device__ constexpr bool slot_reversed(int slot) { return (slot & 4) != 0; }

// Position of bin kappa's power within its region, and of bin b in a frame.
__host__ __device__ constexpr int kapos(int k) { return k <= 25 ? k : k + 3; }
__host__ __device__ constexpr int ppos(int b) {
  return b <= 50 ? kapos(b) : b < 100 ? 3 * kPReg + kapos(100 - b)
       : b <= 150 ? 2 * kPReg + kapos(b - 100) : kPReg + kapos(200 - b);
}

// Bin kappa of the 4 x 25 transform's output (k1, k2), and whether the value
// there is the conjugate of S[kappa].
__host__ __device__ constexpr int pfa_k4(int k1, int k2) { return (25 * k1 + 76 * k2) % 100; }

// ---------------------------------------------------------------------------
// Span staging. Chunk q (four columns) and quarter t (rows 4t..4t+3) are one
// thread's task: its four 16-byte groups u = 0..3 hold column 4q + u of
// those rows (sample e of group u is row 4t + e), and each row's four
// columns go to LDS as one 16-byte store.
//
// A tile inside one clip is its 5360 samples from s0 (84 chunks; loads past
// the span's end repeat its last group). A tile across clips (or the
// batch's last tile) is staged as a virtual span of pieces: the frames of a
// piece (consecutive frames of one clip) keep their 160-sample hops, and a
// piece starts three hops after the previous piece's last frame, so frame f
// of piece p sits at hop slot f + 2p. Hop slot j holds samples [g, g + lim)
// of the batch (lim 160, or 80 for a piece's last slot; zeros past lim).
// A pass stages at most kPassPieces pieces (hop slots counted from the
// pass's first frame); a tile of more pieces takes several passes over its
// frames, each storing the rows of its own pieces.
// ---------------------------------------------------------------------------
static constexpr int kFastTasks = 4 * ((kSpanQ + 63) / 64);        // 336
static constexpr int kFastRounds = (kFastTasks + kThreads - 1) / kThreads;   // 3
static constexpr int kPieceTasks = 4 * ((kPieceCols + 3) / 4);      // 456
static constexpr int kPieceRounds = (kPieceTasks + kThreads - 1) / kThreads;   // 4

__device__ __forceinline__ float4 ld4(const float* p) {
  const f4u t = *reinterpret_cast<const f4u*>(p);
  return make_float4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ float4 ld4(const int16_t* p) {
  return make_float4(sample_value(p), sample_value(p + 1), sample_value(p + 2),
                     sample_value(p + 3));
}

typedef float f4v __attribute__((ext_vector_type(4)));

struct SpanQ {
  f4v g[kFastRounds][4];
};

template <typename In>
__device__ __forceinline__ void load_span_q(const In* __restrict__ base, int64_t s0, int tid,
                                            SpanQ& sp) {
  const In* src = base + s0;
#pragma unroll
  for (int r = 0; r < kFastRounds; ++r) {
    const int task = min(tid + kThreads * r, kFastTasks - 1);
    const int q = task >> 2, t = task & 3;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int off = min(64 * q + 4 * t + 16 * u, kSpanQ - 4);
      const float4 v = ld4(src + off);
      sp.g[r][u] = f4v{v.x, v.y, v.z, v.w};
    }
  }
}

__device__ __forceinline__ float comp(const float4& v, int e) {
  return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
}

__device__ __forceinline__ void write_task(const float4 (&g)[4], int q, int t, float* lds) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int row = 4 * t + e;
    const int slot = row_slot(row);
    const float a = comp(g[0], e), b = comp(g[1], e), c = comp(g[2], e), d = comp(g[3], e);
    if (slot_reversed(slot))
      *reinterpret_cast<float4*>(lds + slot * kRS + kCmax - 4 * q - 3) = make_float4(d, c, b, a);
    else
      *reinterpret_cast<float4*>(lds + slot * kRS + 4 * q) = make_float4(a, b, c, d);
  }
}

__device__ __forceinline__ void span_to_lds_q(const SpanQ& sp, int tid, float* lds) {
#pragma unroll
  for (int r = 0; r < kFastRounds; ++r) {
    const int task = tid + kThreads * r;
    if (task < kFastTasks) {
      const float4 g[4] = {
          make_float4(sp.g[r][0].x, sp.g[r][0].y, sp.g[r][0].z, sp.g[r][0].w),
          make_float4(sp.g[r][1].x, sp.g[r][1].y, sp.g[r][1].z, sp.g[r][1].w),
          make_float4(sp.g[r][2].x, sp.g[r][2].y, sp.g[r][2].z, sp.g[r][2].w),
          make_float4(sp.g[r][3].x, sp.g[r][3].y, sp.g[r][3].z, sp.g[r][3].w)};
      write_task(g, task >> 2, task & 3, lds);
    }
  }
}

// Per-tile bookkeeping in LDS: the output row of each frame for this tile
// and the next (INT64_MIN: not written; a negative value ~row: the frame is
// not computable and its row is NaN), and for tiles across clips each
// frame's first sample, piece (-1: not computable), hop slot in the current
// pass, and the pass's hop slot records.
struct __attribute__((aligned(16))) QuadMeta {
  int64_t row[2][kTile];
  int64_t s[kTile];
  int piece[kTile];
  int sig[kTile];
  PieceSlot slot[kMaxSlots];
};

template <typename In>
__device__ __forceinline__ void pieces_to_lds_q(const In* __restrict__ samples,
                                                const PieceSlot* slots, int tid, float* lds) {
#pragma unroll
  for (int r = 0; r < kPieceRounds; ++r) {
    const int task = tid + kThreads * r;
    if (task < kPieceTasks) {
      const int q = task >> 2, t = task & 3;
      float4 g[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int col = 4 * q + u;
        const int j = col / 10;
        const int off = 16 * (col - 10 * j) + 4 * t;
        const PieceSlot rec = slots[min(j, kMaxSlots - 1)];
        g[u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (off + 4 <= rec.lim) g[u] = ld4(samples + rec.g + off);
      }
      write_task(g, q, t, lds);
    }
  }
}

// ---------------------------------------------------------------------------
// The transform of one lane: four real 25-point DFTs (the window folded into
// their first butterflies), 4-point DFTs over n1, rotation by the
// wavefront's W800^{(2c + 1) kappa}. lds_base: this lane's class row 0 at
// its frame's first column (reversed rows: the first position of the
// frame's reversed run).
// ---------------------------------------------------------------------------
// One row n1: the real 25-point DFT (5 x 5, as dft25_real) of the windowed
// samples row[(6 n1 + n2) mod 25] * win[25 n1 + n2], n2 = 0..24, each group
// of five samples read from LDS right before its 5-point DFT.
template <int n1>
__device__ __forceinline__ void dft25_row(const float* row, const double* __restrict__ win,
                                          cd (&Z)[13]) {
  double r0[5];
  cd r1[5], r2[5];
#pragma unroll
  for (int na = 0; na < 5; ++na) {
    double x[5], w[5];
#pragma unroll
    for (int nb = 0; nb < 5; ++nb) {
      const int n2 = na + 5 * nb;
      x[nb] = (double)row[(6 * n1 + n2) % 25];
      w[nb] = win[25 * n1 + n2];
    }
    dft5_real_w(w[0], x[0], w[1], x[1], w[2], x[2], w[3], x[3], w[4], x[4], r0[na], r1[na],
                r2[na]);
    fence(r0[na]);
    fence(r1[na]);
    fence(r2[na]);
  }
#pragma unroll
  for (int na = 1; na < 5; ++na) {
    r1[na] = c_twiddle(r1[na], kDCos25[na], kDSin25[na]);
    r2[na] = c_twiddle(r2[na], kDCos25[2 * na], kDSin25[2 * na]);
  }
  double z0;
  cd z5, z10;
  dft5_real(r0[0], r0[1], r0[2], r0[3], r0[4], z0, z5, z10);
  dft5(r1[0], r1[1], r1[2], r1[3], r1[4]);
  dft5(r2[0], r2[1], r2[2], r2[3], r2[4]);
  Z[0] = {z0, 0.0};
  Z[5] = z5;
  Z[10] = z10;
  Z[1] = r1[0]; Z[6] = r1[1]; Z[11] = r1[2];
  Z[2] = r2[0]; Z[7] = r2[1]; Z[12] = r2[2];
  Z[3] = {r2[4].re, -r2[4].im};
  Z[4] = {r1[4].re, -r1[4].im};
  Z[8] = {r2[3].re, -r2[3].im};
  Z[9] = {r1[3].re, -r1[3].im};
}

template <int n1>
__device__ __forceinline__ void stage1_row(const float* lds_base, const double* __restrict__ win,
                                           cd (&A)[4][13]) {
  cd Z[13];
  dft25_row<n1>(lds_base + n1 * kRS, win, Z);
#pragma unroll
  for (int k = 0; k <= 12; ++k) {
    A[n1][k] = Z[k];
    fence(A[n1][k].re);
    if (k > 0) fence(A[n1][k].im);
  }
}

__device__ __forceinline__ void lane_transform(const float* lds_base, const double* __restrict__ win,
                                               const double* __restrict__ rot, cd (&U)[51]) {
  cd A[4][13];
  stage1_row<0>(lds_base, win, A);
  stage1_row<1>(lds_base, win, A);
  stage1_row<2>(lds_base, win, A);
  stage1_row<3>(lds_base, win, A);
#pragma unroll
  for (int k2 = 0; k2 <= 12; ++k2) {
    cd q0 = A[0][k2], q1 = A[1][k2], q2 = A[2][k2], q3 = A[3][k2];
    dft4(q0, q1, q2, q3);
    const cd B[4] = {q0, q1, q2, q3};
#pragma unroll
    for (int k1 = 0; k1 < 4; ++k1) {
      if (k2 == 0 && k1 == 3) continue;     // the conjugate of k1 = 1
      const int k = pfa_k4(k1, k2);
      const int kap = k <= 50 ? k : 100 - k;
      const cd sv = k <= 50 ? B[k1] : cd{B[k1].re, -B[k1].im};
      U[kap] = kap == 0 ? sv : c_twiddle(sv, rot[2 * kap], rot[2 * kap + 1]);
      fence(U[kap]);
    }
  }
}

// ---------------------------------------------------------------------------
// The exchange and the powers of one bin: own = this lane's U, the partner's
// by DPP, o1 and o2 the other wavefront's U of this lane and of its partner.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void bin_powers(cd own, cd o1, cd o2, double s, float& pa, float& pb) {
  const cd p = {pair_swap(own.re), pair_swap(own.im)};
  const cd Gm = {s * own.re + p.re, own.im - s * p.im};
  const cd Fm = {own.re + s * p.im, own.im + s * p.re};
  const cd Go = {s * o1.re + o2.re, o1.im - s * o2.im};
  const cd Fo = {o2.re - s * o1.im, o2.im - s * o1.re};
  const double ar = Gm.re + s * Go.re, ai = Gm.im + s * Go.im;
  const double br = Fm.re - Fo.re, bi = Fm.im + Fo.im;
  pa = (float)(ar * ar + ai * ai);
  pb = (float)(br * br + bi * bi);
}

// Exchange buffer: [slot][wavefront][lane] complex fp64.
__device__ __forceinline__ cd* xch_at(float* lds, int slot, int wave, int lane) {
  return reinterpret_cast<cd*>(lds) + (slot * 2 + wave) * 64 + lane;
}

// Wavefront c produces the other wavefront's bins kappa1 + 13 h + t and
// consumes its own bins kappa0 + 13 h + t, t = 0..12, in rounds h = 0, 1
// through LDS (the barriers between the halves are the caller's).
template <int kappa1>
__device__ __forceinline__ void xch_put(const cd (&U)[51], float* lds, int c, int lane, int h) {
#pragma unroll
  for (int t = 0; t < kXchSlots; ++t) *xch_at(lds, t, c, lane) = U[kappa1 + 13 * h + t];
}

template <int kappa0>
__device__ __forceinline__ void xch_take(const cd (&U)[51], const float* lds, int c, int lane,
                                         int h, double s, float (&pa)[26], float (&pb)[26]) {
#pragma unroll
  for (int t = 0; t < kXchSlots; ++t) {
    const cd o1 = *xch_at(const_cast<float*>(lds), t, 1 - c, lane);
    const cd o2 = *xch_at(const_cast<float*>(lds), t, 1 - c, lane ^ 1);
    bin_powers(U[kappa0 + 13 * h + t], o1, o2, s, pa[13 * h + t], pb[13 * h + t]);
  }
}

// ---------------------------------------------------------------------------
// Mel bands from the powers of a frame held in LDS (positions ppos), the
// band-sparse fp32 weights as compile-time literals. An empty filter's sum
// of zero-weight terms is 0 times a power: NaN where the frame's powers are.
// ---------------------------------------------------------------------------
template <int m>
__device__ __forceinline__ float mel_band_q(const float (&pl)[kPFS]) {
  constexpr int n = kMelCount[m], k0 = kMelStart[m];
  if constexpr (n == 0) {
    return 0.0f * pl[ppos(1)];
  } else {
    float e = kMelW[m][0] * pl[ppos(k0)];
#pragma unroll
    for (int j = 1; j < n; ++j) e = __builtin_fmaf(kMelW[m][j], pl[ppos(k0 + j)], e);
    return e;
  }
}

template <int M0, int... I>
__device__ __forceinline__ void mel_range(const float (&pl)[kPFS], float* E,
                                          std::integer_sequence<int, I...>) {
  ((E[I] = mel_band_q<M0 + I>(pl)), ...);
}

// Loads positions [a, b) of a frame's powers (16-byte groups).
template <int a, int b>
__device__ __forceinline__ void load_powers(const float* frame, float (&pl)[kPFS]) {
#pragma unroll
  for (int i = a / 4; i < (b + 3) / 4; ++i) {
    const float4 v = *reinterpret_cast<const float4*>(frame + 4 * i);
    pl[4 * i] = v.x;
    pl[4 * i + 1] = v.y;
    pl[4 * i + 2] = v.z;
    pl[4 * i + 3] = v.w;
  }
}

__device__ __forceinline__ float log_floor(float e) {
  e = (e < kLogFloor) ? kLogFloor : e;   // a NaN energy stays NaN
  return __builtin_amdgcn_logf(e) * kLn2;
}

// Stores a frame's N consecutive outputs (o[0..N)) at dst; NaN if !ok.
template <int N>
__device__ __forceinline__ void store_row(float* __restrict__ dst, const float* o, bool ok) {
  static_assert(N % 4 == 0, "16-byte stores");
  float4* d = reinterpret_cast<float4*>(dst);
  const float qnan = __builtin_nanf("");
#pragma unroll
  for (int i = 0; i < N / 4; ++i)
    d[i] = ok ? make_float4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3])
              : make_float4(qnan, qnan, qnan, qnan);
}

template <int N>
__device__ __forceinline__ void store_row(_Float16* __restrict__ dst, const float* o, bool ok) {
  static_assert(N % 4 == 0, "8-byte stores");
  uint2* d = reinterpret_cast<uint2*>(dst);
  const uint32_t qnan2 = 0x7e007e00u;
#pragma unroll
  for (int i = 0; i < N / 4; ++i)
    d[i] = ok ? make_uint2(pack_half2(o[4 * i], o[4 * i + 1]), pack_half2(o[4 * i + 2], o[4 * i + 3]))
              : make_uint2(qnan2, qnan2);
}

// Bands [M0, M0 + 2H) of frame f: both lanes form them all, role r keeps
// the logs of [M0 + r H, M0 + (r + 1) H) in o[0..H).
template <int M0, int H, int pa0, int pb0, int pa1, int pb1, int pa2, int pb2>
__device__ __forceinline__ void bands_log(const float* frame, int role, float* o) {
  float pl[kPFS];
  load_powers<pa0, pb0>(frame, pl);
  load_powers<pa1, pb1>(frame, pl);
  if constexpr (pb2 > pa2) load_powers<pa2, pb2>(frame, pl);
  float E[2 * H];
  mel_range<M0>(pl, E, std::make_integer_sequence<int, 2 * H>{});
#pragma unroll
  for (int i = 0; i < H; ++i) o[i] = log_floor(role ? E[H + i] : E[i]);
}

// This lane's share of frame f's row (wavefront 0: bands 44 r .. 44 r + 43;
// wavefront 1: bands 88 + 20 r .. 88 + 20 r + 19), or nothing for a frame
// with no row; NaN for a frame that is not computable.
template <typename Out>
__device__ __forceinline__ void store_share(Out* __restrict__ out, int64_t rw, int c, int r,
                                            const float* o) {
  if (rw == INT64_MIN) return;
  const bool ok = rw >= 0;
  Out* dst = out + (ok ? rw : ~rw) * 128;
  if (c == 0) store_row<44>(dst + 44 * r, o, ok);
  else store_row<20>(dst + 88 + 20 * r, o, ok);
}

// Locates tile `tile` (both wavefronts, identically), records its frames'
// output rows in rowbuf and, for a tile inside one clip, loads its span into
// sp. Returns whether it did (the tile is inside one clip).
template <typename In>
__device__ __forceinline__ bool locate_next(int64_t tile, int c, int lane,
                                            const In* __restrict__ samples,
                                            const int64_t* __restrict__ seg_start,
                                            const int64_t* __restrict__ seg_end,
                                            const int64_t* __restrict__ frame_off, RowMap rows,
                                            int64_t n_clips, int64_t total_frames,
                                            int64_t out_rows, int64_t* rowbuf, SpanQ& sp,
                                            ClipCache& cc) {
  int ln = lane;
  asm volatile("" : "+v"(ln));
  const TileSrc cur = locate_tile(tile, ln, seg_start, seg_end, frame_off, rows, n_clips,
                                  total_frames, cc);
  if (c == 0 && !(ln & 1))
    rowbuf[ln >> 1] = (cur.in_range && cur.row >= 0 && cur.row < out_rows)
                          ? (cur.valid ? cur.row : ~cur.row) : INT64_MIN;
  if (cur.fast) {
    int t = 64 * c + ln;
    asm volatile("" : "+v"(t));
    load_span_q(samples, cur.s0, t, sp);
  }
  return cur.fast;
}

// A tile across clips: each frame's first sample and piece into m (written
// by wavefront 0); returns the number of passes (wave-uniform).
__device__ __forceinline__ int pieces_setup(int64_t tile, int c, int lane,
                                            const int64_t* __restrict__ seg_start,
                                            const int64_t* __restrict__ seg_end,
                                            const int64_t* __restrict__ frame_off, RowMap rows,
                                            int64_t n_clips, int64_t total_frames, QuadMeta& m,
                                            ClipCache& cc) {
  int ln = lane;
  asm volatile("" : "+v"(ln));
  const TileSrc cur = locate_tile(tile, ln, seg_start, seg_end, frame_off, rows, n_clips,
                                  total_frames, cc);
  int sigma, breaks;
  piece_slot(cur, ln, sigma, breaks);
  if (c == 0 && !(ln & 1)) {
    m.s[ln >> 1] = cur.s;
    m.piece[ln >> 1] = cur.valid ? (sigma - (ln >> 1)) / 2 : -1;
  }
  return breaks / kPassPieces + 1;
}

// The hop slots of pass `pass` (wavefront 0; the caller's barriers order
// them): every frame's slot in the pass (0 for frames outside it), then the
// slot records of the pass's frames.
__device__ __forceinline__ void pieces_pass(int pass, int lane, QuadMeta& m) {
  int ln = lane;
  asm volatile("" : "+v"(ln));
  const int f = ln >> 1;
  const int pc = m.piece[f];
  const bool in = pc >= kPassPieces * pass && pc < kPassPieces * (pass + 1);
  const uint64_t bm = __ballot(in);
  const int f0 = bm ? (int)(__builtin_ctzll(bm) >> 1) : 0;
  const int sig = in ? f + 2 * (pc - kPassPieces * pass) - f0 : 0;
  if (!(ln & 1)) m.sig[f] = sig;
  if (ln < kMaxSlots) m.slot[ln] = PieceSlot{0, 0, 0};
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  if (in && !(ln & 1)) {
    const int64_t s = m.s[f];
    m.slot[sig] = PieceSlot{s, 160, 0};
    const bool last = f == kTile - 1 || m.piece[f + 1] != pc;
    if (last) {
      m.slot[sig + 1] = PieceSlot{s + 160, 160, 0};
      m.slot[sig + 2] = PieceSlot{s + 320, 80, 0};
    }
  }
}

template <typename In, typename Out>
__device__ __forceinline__ void quad_body(const In* __restrict__ samples,
                                          const int64_t* __restrict__ seg_start,
                                          const int64_t* __restrict__ seg_end,
                                          const int64_t* __restrict__ frame_off, int64_t n_clips,
                                          int64_t total_frames, Out* __restrict__ out,
                                          const int64_t* __restrict__ row_base, int64_t row_unit,
                                          int64_t out_rows, const double* __restrict__ tables,
                                          float* lds, QuadMeta& m) {
  const RowMap rows{row_base, row_unit};
  const int tid = threadIdx.x;
  const int c = __builtin_amdgcn_readfirstlane(tid >> 6);   // wavefront: class pair
  const int lane = tid & 63;
  __builtin_assume(lane < 64);
  const double* win = tables + kTabQWin + 100 * c;
  const double* rot = tables + kTabQRot + 102 * c;
  const int64_t n_tiles = (total_frames + kTile - 1) / kTile;
  const int64_t per = n_tiles / gridDim.x, extra = n_tiles % gridDim.x;
  int64_t tile = blockIdx.x * per + min((int64_t)blockIdx.x, extra);
  const int64_t tile_end = tile + per + ((int64_t)blockIdx.x < extra ? 1 : 0);
  ClipCache cc{0, 0, 0, 0, 0};
  SpanQ sp;
  float ob[44];           // this lane's outputs of the last tile
  bool pending = false;   // ob holds a tile's outputs not yet stored
  // pf: the current tile is inside one clip and its span is in sp
  bool pf = tile < tile_end &&
            locate_next(tile, c, lane, samples, seg_start, seg_end, frame_off, rows, n_clips,
                        total_frames, out_rows, m.row[tile & 1], sp, cc);
  for (; tile < tile_end; ++tile) {
    const int buf = (int)(tile & 1);
    const bool fast = pf;
    const int npass = fast ? 1
        : pieces_setup(tile, c, lane, seg_start, seg_end, frame_off, rows, n_clips,
                       total_frames, m, cc);
    for (int pass = 0; pass < npass; ++pass) {
      if (fast) {
        // the span as loaded (16-byte groups in consecutive registers): the
        // regrouping for the LDS stores happens here, after its loads landed,
        // not where they were issued
#pragma unroll
        for (int r = 0; r < kFastRounds; ++r)
#pragma unroll
          for (int u = 0; u < 4; ++u) asm volatile("" : "+v"(sp.g[r][u]));
        int t = tid;
        asm volatile("" : "+v"(t));
        span_to_lds_q(sp, t, lds);
      } else {
        if (c == 0) pieces_pass(pass, lane, m);
        lds_barrier();
        int t = tid;
        asm volatile("" : "+v"(t));
        pieces_to_lds_q(samples, m.slot, t, lds);
      }
      if (pending) {
        // the previous tile's rows: issued after this tile's span loads
        // have landed, so that the wait for the next span does not include
        // them, and written while this tile is transformed
        int ln = lane;
        asm volatile("" : "+v"(ln));
        store_share(out, m.row[buf ^ 1][ln >> 1], c, ln & 1, ob);
        pending = false;
      }
      // ob holds no value until this tile's bands (no registers across the
      // transform)
#pragma unroll
      for (int i = 0; i < 44; ++i) ob[i] = __builtin_nondeterministic_value(ob[i]);
      // sp is consumed: until the next prefetch it holds no value (so that it
      // takes no registers across the transform)
#pragma unroll
      for (int r = 0; r < kFastRounds; ++r)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          sp.g[r][u] = __builtin_nondeterministic_value(sp.g[r][u]);
        }
      lds_barrier();
      cd U[51];
      {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int f = ln >> 1, r = ln & 1;
        const int sg = fast ? f : m.sig[f];
        const float* base = lds + (8 * c + 4 * r) * kRS + (r ? kCmax - 24 - 10 * sg : 10 * sg);
        lane_transform(base, win, rot, U);
      }
      lds_barrier();   // every lane has read the span: the region takes the exchange
      float pa[26], pb[26];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        if (c == 0) xch_put<25>(U, lds, 0, ln, h);
        else xch_put<0>(U, lds, 1, ln, h);
        lds_barrier();
        int lt = lane;
        asm volatile("" : "+v"(lt));
        const double sg = (lt & 1) ? -1.0 : 1.0;
        if (c == 0) xch_take<0>(U, lds, 0, lt, h, sg, pa, pb);
        else xch_take<25>(U, lds, 1, lt, h, sg, pa, pb);
        lds_barrier();
      }
      if (pass == npass - 1) {
        // the next tile: its rows, and its span's loads in flight while this
        // tile's powers and bands run
        pf = tile + 1 < tile_end &&
             locate_next(tile + 1, c, lane, samples, seg_start, seg_end, frame_off, rows,
                         n_clips, total_frames, out_rows, m.row[buf ^ 1], sp, cc);
      }
      // powers into LDS: bin kappa of (role, wavefront) in regions role and
      // 2 + (wavefront xor role), at kapos
      {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int f = ln >> 1, r = ln & 1;
        float* fr = lds + f * kPFS + 28 * c;
        float* ra = fr + kPReg * r;
        float* rb = fr + kPReg * (2 + (c ^ r));
#pragma unroll
        for (int i = 0; i < 24; i += 4) {
          *reinterpret_cast<float4*>(ra + i) = make_float4(pa[i], pa[i + 1], pa[i + 2], pa[i + 3]);
          *reinterpret_cast<float4*>(rb + i) = make_float4(pb[i], pb[i + 1], pb[i + 2], pb[i + 3]);
        }
        *reinterpret_cast<float2*>(ra + 24) = make_float2(pa[24], pa[25]);
        *reinterpret_cast<float2*>(rb + 24) = make_float2(pb[24], pb[25]);
      }
      lds_barrier();
      {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int f = ln >> 1, r = ln & 1;
        const float* frame = lds + f * kPFS;
        if (c == 0)   // bands 0..87: bins up to 84 (regions 0 and 3)
          bands_log<0, 44, 0, 56, 3 * kPReg + 16, 3 * kPReg + 56, 0, 0>(frame, r, ob);
        else          // bands 88..127: bins 81..200 (regions 3, 2, 1)
          bands_log<88, 20, 3 * kPReg, 3 * kPReg + 20, 2 * kPReg, 2 * kPReg + 56, kPReg,
                    kPReg + 56>(frame, r, ob);
        if (fast) {
          pending = true;   // stored after the next tile's span is staged
        } else {
          // in a tile of several passes, a computable frame's row is stored
          // by its own piece's pass
          const int64_t rw = m.row[buf][f];
          if (npass == 1 || rw < 0 || m.piece[f] / kPassPieces == pass)
            store_share(out, rw, c, r, ob);
        }
      }
      lds_barrier();   // the powers are read: the region takes the next span
    }
  }
  if (pending) store_share(out, m.row[(tile - 1) & 1][lane >> 1], c, lane & 1, ob);
}

#define LOGMEL_QUAD_KERNEL(NAME, IN, OUT)                                                       \
  extern "C" __global__ void __attribute__((amdgpu_flat_work_group_size(128, 128),              \
                                            amdgpu_waves_per_eu(2, 2)))                          \
  NAME(const IN* __restrict__ samples, const int64_t* __restrict__ seg_start,                   \
       const int64_t* __restrict__ seg_end, const int64_t* __restrict__ frame_off,              \
       int64_t n_clips, int64_t total_frames, OUT* __restrict__ out,                             \
       const int64_t* __restrict__ row_base, int64_t row_unit, int64_t out_rows,                \
       const double* __restrict__ tables) {                                                     \
    __shared__ float4 region[kRegionFloats / 4];                                                \
    __shared__ QuadMeta meta;                                                                   \
    quad_body<IN, OUT>(samples, seg_start, seg_end, frame_off, n_clips, total_frames, out,      \
                       row_base, row_unit, out_rows, tables,                                    \
                       reinterpret_cast<float*>(region), meta);                                 \
  }

LOGMEL_QUAD_KERNEL(logmel_quad_kernel, float, float)
LOGMEL_QUAD_KERNEL(logmel_quad_kernel_f16, float, _Float16)
LOGMEL_QUAD_KERNEL(logmel_quad_kernel_i16, int16_t, float)
LOGMEL_QUAD_KERNEL(logmel_quad_kernel_i16_f16, int16_t, _Float16)

}  // namespace quad
}  // namespace logmel

hipError_t logmel_launch_quad(const double* tables, const void* samples, int in_i16,
                              const int64_t* seg_start, const int64_t* seg_end,
                              const int64_t* frame_off, int64_t n_clips, int64_t total_frames,
                              void* out, int out_f16, const int64_t* row_base, int64_t row_unit,
                              int64_t out_rows, int resident_groups, hipStream_t stream) {
  using namespace logmel::quad;
  if (total_frames <= 0) return hipSuccess;
  const int64_t tiles = (total_frames + logmel::kTile - 1) / logmel::kTile;
  const int64_t grid = tiles < resident_groups ? tiles : resident_groups;
  const dim3 g((unsigned)grid), b(kThreads);
  if (!in_i16 && !out_f16)
    hipLaunchKernelGGL(logmel_quad_kernel, g, b, 0, stream, static_cast<const float*>(samples),
                       seg_start, seg_end, frame_off, n_clips, total_frames,
                       static_cast<float*>(out), row_base, row_unit, out_rows, tables);
  else if (!in_i16)
    hipLaunchKernelGGL(logmel_quad_kernel_f16, g, b, 0, stream,
                       static_cast<const float*>(samples), seg_start, seg_end, frame_off, n_clips,
                       total_frames, static_cast<_Float16*>(out), row_base, row_unit, out_rows,
                       tables);
  else if (!out_f16)
    hipLaunchKernelGGL(logmel_quad_kernel_i16, g, b, 0, stream,
                       static_cast<const int16_t*>(samples), seg_start, seg_end, frame_off,
                       n_clips, total_frames, static_cast<float*>(out), row_base, row_unit,
                       out_rows, tables);
  else
    hipLaunchKernelGGL(logmel_quad_kernel_i16_f16, g, b, 0, stream,
                       static_cast<const int16_t*>(samples), seg_start, seg_end, frame_off,
                       n_clips, total_frames, static_cast<_Float16*>(out), row_base, row_unit,
                       out_rows, tables);
  return hipGetLastError();
}

hipError_t logmel_launch_tiles(const double* tables, const void* samples, int in_i16,
                               const int64_t* seg_start, const int64_t* seg_end,
                               const int64_t* frame_off, int64_t n_clips, int64_t total_frames,
                               void* out, int out_f16, const int64_t* row_base, int64_t row_unit,
                               int64_t out_rows, int resident_waves, hipStream_t stream) {
  const char* k = std::getenv("LOGMEL_KERNEL");
  if (!(k && k[0] == 'q'))
    return logmel_launch_tiles_v1(tables, samples, in_i16, seg_start, seg_end, frame_off, n_clips,
                                  total_frames, out, out_f16, row_base, row_unit, out_rows,
                                  resident_waves, stream);
  return logmel_launch_quad(tables, samples, in_i16, seg_start, seg_end, frame_off, n_clips,
                            total_frames, out, out_f16, row_base, row_unit, out_rows,
                            resident_waves, stream);
}
