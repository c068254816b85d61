// Per-frame log-mel routine for gfx950: one 400-sample frame per lane.
//
// The steps follow the five-step recipe of the page "从零理解 ASR：音频基础、
// Qwen3-ASR 架构，以及离线 vs 流式推理原理" (§2.3): symmetric Hamming window,
// 400-point real FFT to 201 bins, power |X|^2, 128 triangular mel filters
// (mel = 2595 log10(1 + f/700), 0..8000 Hz), ln(max(E, 1e-10)).
//
// Layout of the work: every lane owns one whole frame and keeps it in
// registers. The 400-point transform is a prime-factor (Good-Thomas) 16 x 25
// decomposition, so there are no twiddles between the two stages:
//   n = (25 n1 + 16 n2) mod 400,  k = (225 k1 + 176 k2) mod 400,
//   X[k] = sum_n1 W16^(n1 k1) sum_n2 W25^(n2 k2) y[n].
// Stage 1 runs 16 real 25-point DFTs (two at a time as one complex DFT,
// 5 x 5 Cooley-Tukey), stage 2 runs 13 16-point DFTs (4 x 4 Cooley-Tukey)
// for k2 = 0..12, which by Hermitian symmetry covers every bin 0..200 once.
// All twiddles, window values and filter weights are compile-time literals,
// the same for every lane, so no lane-varying constant is ever loaded.
#pragma once

#include <hip/hip_runtime.h>

#include "logmel_tables.h"

namespace logmel {

struct cf {
  float re, im;
};

__device__ __forceinline__ cf c_add(cf a, cf b) { return {a.re + b.re, a.im + b.im}; }
__device__ __forceinline__ cf c_sub(cf a, cf b) { return {a.re - b.re, a.im - b.im}; }
// a * conj-free twiddle exp(-2 pi i j / n) = (c, -s)
__device__ __forceinline__ cf c_twiddle(cf a, float c, float s) {
  return {a.re * c + a.im * s, a.im * c - a.re * s};
}

// Forward 5-point DFT, Winograd-style grouping of conjugate pairs.
__device__ __forceinline__ void dft5(cf& x0, cf& x1, cf& x2, cf& x3, cf& x4) {
  const cf t1 = c_add(x1, x4), t2 = c_add(x2, x3);
  const cf t3 = c_sub(x1, x4), t4 = c_sub(x2, x3);
  const cf y0 = {x0.re + t1.re + t2.re, x0.im + t1.im + t2.im};
  const cf a1 = {x0.re + kC51 * t1.re + kC52 * t2.re, x0.im + kC51 * t1.im + kC52 * t2.im};
  const cf a2 = {x0.re + kC52 * t1.re + kC51 * t2.re, x0.im + kC52 * t1.im + kC51 * t2.im};
  const cf b1 = {kS51 * t3.re + kS52 * t4.re, kS51 * t3.im + kS52 * t4.im};
  const cf b2 = {kS52 * t3.re - kS51 * t4.re, kS52 * t3.im - kS51 * t4.im};
  x0 = y0;
  x1 = {a1.re + b1.im, a1.im - b1.re};  // a1 - i b1
  x4 = {a1.re - b1.im, a1.im + b1.re};  // a1 + i b1
  x2 = {a2.re + b2.im, a2.im - b2.re};  // a2 - i b2
  x3 = {a2.re - b2.im, a2.im + b2.re};  // a2 + i b2
}

// Forward 4-point DFT.
__device__ __forceinline__ void dft4(cf& x0, cf& x1, cf& x2, cf& x3) {
  const cf s02 = c_add(x0, x2), d02 = c_sub(x0, x2);
  const cf s13 = c_add(x1, x3), d13 = c_sub(x1, x3);
  x0 = c_add(s02, s13);
  x2 = c_sub(s02, s13);
  x1 = {d02.re + d13.im, d02.im - d13.re};  // d02 - i d13
  x3 = {d02.re - d13.im, d02.im + d13.re};  // d02 + i d13
}

// In-place forward 25-point DFT, 5 x 5: n = na + 5 nb, k = 5 ka + kb.
// Input z[n] in natural order; output Z[k] in natural order.
__device__ __forceinline__ void dft25(cf (&z)[25]) {
  cf t[5][5];
#pragma unroll
  for (int na = 0; na < 5; ++na) {
    cf a = z[na], b = z[na + 5], c = z[na + 10], d = z[na + 15], e = z[na + 20];
    dft5(a, b, c, d, e);
    t[na][0] = a; t[na][1] = b; t[na][2] = c; t[na][3] = d; t[na][4] = e;
  }
#pragma unroll
  for (int na = 1; na < 5; ++na)
#pragma unroll
    for (int kb = 1; kb < 5; ++kb)
      t[na][kb] = c_twiddle(t[na][kb], kCos25[na * kb], kSin25[na * kb]);
#pragma unroll
  for (int kb = 0; kb < 5; ++kb) {
    cf a = t[0][kb], b = t[1][kb], c = t[2][kb], d = t[3][kb], e = t[4][kb];
    dft5(a, b, c, d, e);
    z[kb] = a; z[5 + kb] = b; z[10 + kb] = c; z[15 + kb] = d; z[20 + kb] = e;
  }
}

// In-place forward 16-point DFT, 4 x 4: n = na + 4 nb, k = 4 ka + kb.
__device__ __forceinline__ void dft16(cf (&v)[16]) {
  cf t[4][4];
#pragma unroll
  for (int na = 0; na < 4; ++na) {
    cf a = v[na], b = v[na + 4], c = v[na + 8], d = v[na + 12];
    dft4(a, b, c, d);
    t[na][0] = a; t[na][1] = b; t[na][2] = c; t[na][3] = d;
  }
#pragma unroll
  for (int na = 1; na < 4; ++na)
#pragma unroll
    for (int kb = 1; kb < 4; ++kb)
      t[na][kb] = c_twiddle(t[na][kb], kCos16[na * kb], kSin16[na * kb]);
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    cf a = t[0][kb], b = t[1][kb], c = t[2][kb], d = t[3][kb];
    dft4(a, b, c, d);
    v[kb] = a; v[4 + kb] = b; v[8 + kb] = c; v[12 + kb] = d;
  }
}

// Compiler ordering fence for a value: an empty volatile asm that "rewrites"
// v in a VGPR. Volatile asm statements keep their program order, so fencing a
// phase's inputs after the previous phase's outputs stops the scheduler from
// interleaving independent phases (which would raise register pressure far
// beyond the ~430 values one frame needs). It emits no instruction.
__device__ __forceinline__ void fence(float& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void fence(cf& v) { fence(v.re); fence(v.im); }

__host__ __device__ constexpr int pfa_in(int n1, int n2) { return (25 * n1 + 16 * n2) % 400; }
__host__ __device__ constexpr int pfa_out(int k1, int k2) { return (225 * k1 + 176 * k2) % 400; }
__host__ __device__ constexpr int bin_of(int k1, int k2) {
  return pfa_out(k1, k2) <= 200 ? pfa_out(k1, k2) : 400 - pfa_out(k1, k2);
}

// One frame: x[400] raw samples -> out[128] log-mel.
// Bins that are not multiples of 25 come out of the transform at twice their
// amplitude (the factor 1/2 of the two-real-sequences split is not applied);
// their filter weights carry the compensating 1/4.
__device__ __forceinline__ void logmel_frame(const float (&x)[400], float (&out)[128]) {
  // Stage 1: 16 real 25-point DFTs over n2, two per complex DFT.
  // A[n1][k2] for k2 = 0..12 (k2 = 0 is real: its .im is an exact 0).
  cf A[16][13];
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    cf z[25];
#pragma unroll
    for (int n2 = 0; n2 < 25; ++n2) {
      const int ia = pfa_in(2 * p, n2), ib = pfa_in(2 * p + 1, n2);
      float xa = x[ia], xb = x[ib];
      fence(xa);
      fence(xb);
      z[n2] = {kWin[ia] * xa, kWin[ib] * xb};
    }
    dft25(z);
    A[2 * p][0] = {z[0].re, 0.0f};
    A[2 * p + 1][0] = {z[0].im, 0.0f};
#pragma unroll
    for (int k = 1; k <= 12; ++k) {
      const cf zk = z[k], zc = z[25 - k];
      // 2 * DFT of the real part:  zk + conj(zc)
      A[2 * p][k] = {zk.re + zc.re, zk.im - zc.im};
      // 2 * DFT of the imaginary part: -i (zk - conj(zc))
      A[2 * p + 1][k] = {zk.im + zc.im, zc.re - zk.re};
    }
#pragma unroll
    for (int k = 0; k <= 12; ++k) {
      fence(A[2 * p][k].re);
      fence(A[2 * p + 1][k].re);
      if (k > 0) {
        fence(A[2 * p][k].im);
        fence(A[2 * p + 1][k].im);
      }
    }
  }

  // Stage 2: for each k2, a 16-point DFT over n1, then power.
  float P[201];
#pragma unroll
  for (int k2 = 0; k2 <= 12; ++k2) {
    cf v[16];
#pragma unroll
    for (int n1 = 0; n1 < 16; ++n1) {
      v[n1] = A[n1][k2];
      fence(v[n1].re);
      if (k2 > 0) fence(v[n1].im);
    }
    dft16(v);
#pragma unroll
    for (int k1 = 0; k1 < 16; ++k1) {
      if (k2 == 0 && k1 > 8) continue;  // conjugates of k1 = 1..7
      P[bin_of(k1, k2)] = v[k1].re * v[k1].re + v[k1].im * v[k1].im;
      fence(P[bin_of(k1, k2)]);
    }
  }

  // Band-sparse mel projection and log with the 1e-10 floor. The floor test
  // is written so that a NaN energy stays NaN.
#pragma unroll
  for (int m = 0; m < 128; ++m) {
    if (kMelCount[m] == 0) {
      out[m] = kLnFloor;
      continue;
    }
    float e = kMelW[m][0] * P[kMelStart[m]];
#pragma unroll
    for (int j = 1; j < kMelMaxBins; ++j)
      if (j < kMelCount[m]) e += kMelW[m][j] * P[kMelStart[m] + j];
    e = (e < kLogFloor) ? kLogFloor : e;
    out[m] = __builtin_amdgcn_logf(e) * kLn2;
  }
}

}  // namespace logmel
