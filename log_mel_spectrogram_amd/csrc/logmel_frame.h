// Per-frame log-mel routine for gfx950: one 400-sample frame per lane pair.
//
// The steps follow the five-step recipe of the page "从零理解 ASR：音频基础、
// Qwen3-ASR 架构，以及离线 vs 流式推理原理" (§2.3): symmetric Hamming window,
// 400-point real FFT to 201 bins, power |X|^2, 128 triangular mel filters
// (mel = 2595 log10(1 + f/700), 0..8000 Hz), ln(max(E, 1e-10)).
//
// Precision. The result must hold to 1e-3 in the log wherever a band's
// energy is at least 1e-7, also in loud frames whose quietest bands sit
// 90 dB or more below their loudest. An fp32 transform leaves a rounding
// floor about 1e-7 of the frame's amplitude in every bin, which is above
// such bands, so the window and the whole transform run in fp64 (full rate
// on CDNA). Power, filterbank and log run in fp32: a bin's power is formed
// in fp64 and rounded once.
//
// Work split. fp64 doubles the registers a frame needs, so a frame takes two
// lanes of a wavefront, f and f + 32 (a "pair"): role 0 (lanes 0..31)
// transforms the even samples in order, e[m] = x[2m], role 1 (lanes 32..63)
// the odd samples in reverse order, o[m] = x[399 - 2m] (decimation in time).
// The window is symmetric, w[399 - 2m] = w[2m], so both roles apply the same
// window values, and every constant of the routine is the same for all
// lanes. Each role runs the same code:
//   * a 200-point real DFT as a prime-factor (Good-Thomas) 8 x 25 transform,
//       m = (25 n1 + 8 n2) mod 200,  k = (25 k1 + 176 k2) mod 200,
//     with 8 real-input 25-point DFTs (5 x 5, conjugate halves skipped)
//     and 13 8-point DFTs for k2 = 0..12, which cover k = 0..100;
//   * the radix-2 combine. With E and R the two roles' spectra, the odd
//     samples' spectrum is W200^-k conj(R[k]), and multiplying X[k] by
//     W800^k (a unit phase) gives, with u = W800^k E[k], v = W800^k R[k],
//       |X[k]|       = |u + conj(v)|,
//       |X[200 - k]| = |u - conj(v)|.
//     Every column k2 of the 8-point DFTs holds bins k <= 50 and k + 50 in
//     pairs (bins taken as k or 200 - k, whichever is <= 100). One
//     v_permlane32_swap per 32-bit word exchanges the upper lanes' first bin
//     with the lower lanes' second: afterwards lane f holds E and R of bin k
//     and lane f + 32 those of bin k + 50, so one swap word serves two bins.
//     Dividing u + conj(v) by W800^k, each lane forms with its own bin's
//     rotation (from LDS: the two halves combine different bins)
//       t = W400^-k conj(R[k]),  |X[k]| = |E[k] + t|,  |X[200 - k]| = |E[k] - t|.
//     So role 0 holds bins 1..50 and 150..199, role 1 bins 51..149. The
//     filterbank runs on these halves (see pair_logmel); each role logs and
//     stores 64 bands, in alternate runs of the row (band_role).
#pragma once

#include <hip/hip_runtime.h>
#include <utility>

#include "logmel_tables.h"

namespace logmel {

struct cd {
  double re, im;
};

__device__ __forceinline__ cd c_add(cd a, cd b) { return {a.re + b.re, a.im + b.im}; }
__device__ __forceinline__ cd c_sub(cd a, cd b) { return {a.re - b.re, a.im - b.im}; }
// a * exp(-2 pi i j / n) = a * (c - i s)
__device__ __forceinline__ cd c_twiddle(cd a, double c, double s) {
  return {a.re * c + a.im * s, a.im * c - a.re * s};
}

// Compiler ordering fence: an empty volatile asm that "rewrites" v in VGPRs.
// Volatile asm statements keep their program order, so fencing a phase's
// inputs after the previous phase's outputs keeps independent phases from
// being interleaved, which would raise register pressure. No instruction.
__device__ __forceinline__ void fence(float& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void fence(double& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void fence(cd& v) { fence(v.re); fence(v.im); }

// Forward 5-point DFT, conjugate pairs grouped.
__device__ __forceinline__ void dft5(cd& x0, cd& x1, cd& x2, cd& x3, cd& x4) {
  const cd t1 = c_add(x1, x4), t2 = c_add(x2, x3);
  const cd t3 = c_sub(x1, x4), t4 = c_sub(x2, x3);
  const cd y0 = {x0.re + t1.re + t2.re, x0.im + t1.im + t2.im};
  const cd a1 = {x0.re + kDC51 * t1.re + kDC52 * t2.re, x0.im + kDC51 * t1.im + kDC52 * t2.im};
  const cd a2 = {x0.re + kDC52 * t1.re + kDC51 * t2.re, x0.im + kDC52 * t1.im + kDC51 * t2.im};
  const cd b1 = {kDS51 * t3.re + kDS52 * t4.re, kDS51 * t3.im + kDS52 * t4.im};
  const cd b2 = {kDS52 * t3.re - kDS51 * t4.re, kDS52 * t3.im - kDS51 * t4.im};
  x0 = y0;
  x1 = {a1.re + b1.im, a1.im - b1.re};  // a1 - i b1
  x4 = {a1.re - b1.im, a1.im + b1.re};  // a1 + i b1
  x2 = {a2.re + b2.im, a2.im - b2.re};  // a2 - i b2
  x3 = {a2.re - b2.im, a2.im + b2.re};  // a2 + i b2
}

// Forward 4-point DFT.
__device__ __forceinline__ void dft4(cd& x0, cd& x1, cd& x2, cd& x3) {
  const cd s02 = c_add(x0, x2), d02 = c_sub(x0, x2);
  const cd s13 = c_add(x1, x3), d13 = c_sub(x1, x3);
  x0 = c_add(s02, s13);
  x2 = c_sub(s02, s13);
  x1 = {d02.re + d13.im, d02.im - d13.re};  // d02 - i d13
  x3 = {d02.re - d13.im, d02.im + d13.re};  // d02 + i d13
}

// In-place forward 8-point DFT: even/odd 4-point DFTs and one radix-2 step.
__device__ __forceinline__ void dft8(cd (&v)[8]) {
  cd e0 = v[0], e1 = v[2], e2 = v[4], e3 = v[6];
  cd o0 = v[1], o1 = v[3], o2 = v[5], o3 = v[7];
  dft4(e0, e1, e2, e3);
  dft4(o0, o1, o2, o3);
  // W8^1 = (1 - i)/sqrt2, W8^2 = -i, W8^3 = -(1 + i)/sqrt2
  const cd t1 = {(o1.re + o1.im) * kDRootHalf, (o1.im - o1.re) * kDRootHalf};
  const cd t2 = {o2.im, -o2.re};
  const cd t3 = {(o3.im - o3.re) * kDRootHalf, -(o3.re + o3.im) * kDRootHalf};
  v[0] = c_add(e0, o0); v[4] = c_sub(e0, o0);
  v[1] = c_add(e1, t1); v[5] = c_sub(e1, t1);
  v[2] = c_add(e2, t2); v[6] = c_sub(e2, t2);
  v[3] = c_add(e3, t3); v[7] = c_sub(e3, t3);
}

// Forward 5-point DFT of real input: y0 real, y1 and y2 (y3 = conj y2 and
// y4 = conj y1 are not formed).
__device__ __forceinline__ void dft5_real(double x0, double x1, double x2, double x3, double x4,
                                          double& y0, cd& y1, cd& y2) {
  const double t1 = x1 + x4, t2 = x2 + x3, t3 = x1 - x4, t4 = x2 - x3;
  y0 = x0 + t1 + t2;
  const double a1 = x0 + kDC51 * t1 + kDC52 * t2, a2 = x0 + kDC52 * t1 + kDC51 * t2;
  const double b1 = kDS51 * t3 + kDS52 * t4, b2 = kDS52 * t3 - kDS51 * t4;
  y1 = {a1, -b1};
  y2 = {a2, -b2};
}

// dft5_real of the windowed input w[i] * v[i], the window products folded
// into the first sums and differences (x1 +- x4 = fma(w1, v1, +-w4 v4)).
__device__ __forceinline__ void dft5_real_w(double w0, double v0, double w1, double v1, double w2,
                                            double v2, double w3, double v3, double w4, double v4,
                                            double& y0, cd& y1, cd& y2) {
  const double x0 = w0 * v0, p4 = w4 * v4, p3 = w3 * v3;
  const double t1 = __builtin_fma(w1, v1, p4), t3 = __builtin_fma(w1, v1, -p4);
  const double t2 = __builtin_fma(w2, v2, p3), t4 = __builtin_fma(w2, v2, -p3);
  y0 = x0 + t1 + t2;
  const double a1 = x0 + kDC51 * t1 + kDC52 * t2, a2 = x0 + kDC52 * t1 + kDC51 * t2;
  const double b1 = kDS51 * t3 + kDS52 * t4, b2 = kDS52 * t3 - kDS51 * t4;
  y1 = {a1, -b1};
  y2 = {a2, -b2};
}

// Forward 25-point DFT of the real windowed input w[n] * v[n] (5 x 5,
// n = na + 5 nb, k = 5 ka + kb), giving Z[0..12] (Z[0] real; the rest by
// Hermitian symmetry). Only kb = 0, 1, 2 of the first stage are formed:
// kb = 3, 4 are conjugates.
__device__ __forceinline__ void dft25_real(const double (&w)[25], const double (&v)[25],
                                           cd (&Z)[13]) {
  double r0[5];
  cd r1[5], r2[5];
#pragma unroll
  for (int na = 0; na < 5; ++na)
    dft5_real_w(w[na], v[na], w[na + 5], v[na + 5], w[na + 10], v[na + 10], w[na + 15],
                v[na + 15], w[na + 20], v[na + 20], r0[na], r1[na], r2[na]);
#pragma unroll
  for (int na = 1; na < 5; ++na) {
    r1[na] = c_twiddle(r1[na], kDCos25[na], kDSin25[na]);
    r2[na] = c_twiddle(r2[na], kDCos25[2 * na], kDSin25[2 * na]);
  }
  // kb = 0: real input again.
  double z0;
  cd z5, z10;
  dft5_real(r0[0], r0[1], r0[2], r0[3], r0[4], z0, z5, z10);
  // kb = 1 and kb = 2: complex.
  dft5(r1[0], r1[1], r1[2], r1[3], r1[4]);   // Z[1], Z[6], Z[11], Z[16], Z[21]
  dft5(r2[0], r2[1], r2[2], r2[3], r2[4]);   // Z[2], Z[7], Z[12], Z[17], Z[22]
  Z[0] = {z0, 0.0};
  Z[5] = z5;
  Z[10] = z10;
  Z[1] = r1[0]; Z[6] = r1[1]; Z[11] = r1[2];
  Z[2] = r2[0]; Z[7] = r2[1]; Z[12] = r2[2];
  Z[3] = {r2[4].re, -r2[4].im};    // conj Z[22]
  Z[4] = {r1[4].re, -r1[4].im};    // conj Z[21]
  Z[8] = {r2[3].re, -r2[3].im};    // conj Z[17]
  Z[9] = {r1[3].re, -r1[3].im};    // conj Z[16]
}

__host__ __device__ constexpr int pfa_m(int n1, int n2) { return (25 * n1 + 8 * n2) % 200; }
__host__ __device__ constexpr int pfa_k(int k1, int k2) { return (25 * k1 + 176 * k2) % 200; }

// Exchange of the wavefront's halves: lanes 32..63 of a trade places with
// lanes 0..31 of b (v_permlane32_swap on each 32-bit word). Afterwards a
// holds the lower lanes' a in lanes 0..31 and their b in lanes 32..63, and b
// holds the upper lanes' a in lanes 0..31 and their b in lanes 32..63.
__device__ __forceinline__ void half_swap(double& a, double& b) {
  const uint64_t ua = __builtin_bit_cast(uint64_t, a), ub = __builtin_bit_cast(uint64_t, b);
  const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)ua, (uint32_t)ub, false, false);
  const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(ua >> 32), (uint32_t)(ub >> 32), false, false);
  a = __builtin_bit_cast(double, ((uint64_t)hi[0] << 32) | lo[0]);
  b = __builtin_bit_cast(double, ((uint64_t)hi[1] << 32) | lo[1]);
}

// The value of the pair's lane of role `src` (0: lane f, 1: lane f + 32) in
// both lanes of the pair.
__device__ __forceinline__ float pair_from(float v, int src) {
  const uint32_t b = __builtin_bit_cast(uint32_t, v);
  const auto r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  return __builtin_bit_cast(float, src == 0 ? r[0] : r[1]);
}

// Bins of column k2: kap(k1, k2) is bin k = pfa_k(k1, k2) taken as k or
// 200 - k (whichever is <= 100), 0 where the column has no such bin
// (k1 > 4 of column 0 repeats k1 = 3..1 conjugated; bin 0 carries no weight).
__host__ __device__ constexpr int pfa_kap(int k1, int k2) {
  return (k2 == 0 && k1 > 4) ? 0
       : (pfa_k(k1, k2) <= 100 ? pfa_k(k1, k2) : 200 - pfa_k(k1, k2));
}
// The k1 of column k2 whose bin is kap(k1a, k2) + 50 (-1: none).
__host__ __device__ constexpr int pfa_partner(int k1a, int k2) {
  int r = -1;
  for (int k1 = 0; k1 < 8; ++k1)
    if (pfa_kap(k1a, k2) != 0 && pfa_kap(k1, k2) == pfa_kap(k1a, k2) + 50) r = k1;
  return r;
}
// Whether (k1a, k2) is the first bin of a pair, and the pair's slot: pairs
// numbered in order of k2, then k1 (the order of the plan's rotation table).
__host__ __device__ constexpr bool pfa_pair_first(int k1a, int k2) {
  return pfa_kap(k1a, k2) >= 1 && pfa_kap(k1a, k2) <= 50 && pfa_partner(k1a, k2) >= 0;
}
__host__ __device__ constexpr int pfa_slot(int k1a, int k2) {
  int n = 0;
  for (int c = 0; c < 13; ++c)
    for (int k1 = 0; k1 < 8; ++k1) {
      if (c == k2 && k1 == k1a) return n;
      if (pfa_pair_first(k1, c)) ++n;
    }
  return n;
}
static_assert(pfa_slot(0, 13) == 50, "50 bin pairs");
// This half's rotations of column k2's pairs (LDS), by the k1 of the
// pair's first bin.
__device__ __forceinline__ void column_rotations(const double* rot, int k2, double (&c)[8],
                                                 double (&s)[8]) {
#pragma unroll
  for (int k1 = 0; k1 < 8; ++k1) {
    if (!pfa_pair_first(k1, k2)) continue;
    c[k1] = rot[2 * pfa_slot(k1, k2)];
    s[k1] = rot[2 * pfa_slot(k1, k2) + 1];
  }
}

// Power spectrum of one frame on a lane pair.
//   v[200]   this lane's samples, m = 0..199 (fp32): x[2m] for role 0,
//            x[399 - 2m] for role 1
//   win      w[2m], m = (25 n1 + 8 n2) mod 200, in [n1][n2] order (uniform)
//   rot      this half's cos, sin of 2 pi kap / 400 in pair order (LDS: role 0
//            bins a, role 1 bins a + 50; see pfa_slot)
//   Pp, Pm   this lane's half of the power spectrum, a = 1..50:
//            role 0: Pp[a] = |X[a]|^2,      Pm[a] = |X[200 - a]|^2
//            role 1: Pp[a] = |X[a + 50]|^2, Pm[a] = |X[150 - a]|^2
__device__ __forceinline__ void pair_power(const float (&v)[200], const double* __restrict__ win,
                                           const double* rot, float (&Pp)[51],
                                           float (&Pm)[51]) {
  // Stage 1: 8 real 25-point DFTs over n2, two rows n1 per scheduling region
  // (two independent transforms give the scheduler work to overlap).
  // A[n1][k2], k2 = 0..12 (k2 = 0 is real: its .im is an exact 0).
  cd A[8][13];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    float xr[2][25];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int n2 = 0; n2 < 25; ++n2) xr[h][n2] = v[pfa_m(2 * p + h, n2)];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int n2 = 0; n2 < 25; ++n2) fence(xr[h][n2]);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int n1 = 2 * p + h;
      double wv[25], y[25];
#pragma unroll
      for (int n2 = 0; n2 < 25; ++n2) {
        wv[n2] = win[25 * n1 + n2];
        y[n2] = (double)xr[h][n2];
      }
      cd Z[13];
      dft25_real(wv, y, Z);
#pragma unroll
      for (int k = 0; k <= 12; ++k) A[n1][k] = Z[k];
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int k = 0; k <= 12; ++k) {
        fence(A[2 * p + h][k].re);
        if (k > 0) fence(A[2 * p + h][k].im);
      }
  }

  // Stage 2 and the combine: for each k2, an 8-point DFT over n1 gives this
  // role's spectrum at k = pfa_k(k1, k2) (k > 100 through conjugation); for
  // each pair of bins a, a + 50 of the column, exchange halves, rotate this
  // half's R and form the two powers of this half's bin.
#pragma unroll
  for (int k2 = 0; k2 <= 12; ++k2) {
    // The column's rotations (LDS); the compiler places the reads.
    double rc[8], rs[8];
    column_rotations(rot, k2, rc, rs);
    cd q[8];
#pragma unroll
    for (int n1 = 0; n1 < 8; ++n1) {
      q[n1] = A[n1][k2];
      fence(q[n1].re);
      if (k2 > 0) fence(q[n1].im);
    }
    dft8(q);
#pragma unroll
    for (int ka = 0; ka < 8; ++ka) {
      if (!pfa_pair_first(ka, k2)) continue;
      const int a = pfa_kap(ka, k2), kb = pfa_partner(ka, k2);
      // this role's spectrum at bins a and a + 50
      cd e = pfa_k(ka, k2) <= 100 ? q[ka] : cd{q[ka].re, -q[ka].im};
      cd r = pfa_k(kb, k2) <= 100 ? q[kb] : cd{q[kb].re, -q[kb].im};
      // e := role 0's spectrum E, r := role 1's R, at bin a in the lower
      // lanes and at bin a + 50 in the upper ones
      half_swap(e.re, r.re);
      half_swap(e.im, r.im);
      // t = W400^-kap conj(R) = (c + i s)(R.re - i R.im), this half's kap
      const double c = rc[ka], s = rs[ka];
      const double tre = c * r.re + s * r.im, tim = s * r.re - c * r.im;
      const double pre = e.re + tre, pim = e.im + tim;   // X[kap]
      const double mre = e.re - tre, mim = e.im - tim;   // conj X[200 - kap]
      Pp[a] = (float)(pre * pre + pim * pim);
      Pm[a] = (float)(mre * mre + mim * mim);
    }
    // one scheduling region per column
#pragma unroll
    for (int ka = 0; ka < 8; ++ka) {
      if (!pfa_pair_first(ka, k2)) continue;
      fence(Pp[pfa_kap(ka, k2)]);
      fence(Pm[pfa_kap(ka, k2)]);
    }
  }

}

// Band-sparse mel projection and log. Role 0 holds the powers of bins 1..50
// and 150..199, role 1 those of bins 51..149 (see pair_power), and both run
// the same code: every band is summed over this lane's registers, which
// gives the right sum in the half that holds the band's bins (a band whose
// bins lie in both halves is the sum of two partial sums). Each role logs 64
// bands (band_role); the sums a role logs but the other half holds move
// across the pair with v_permlane32_swap. The log has the 1e-10 floor, taken
// so that a NaN energy stays NaN.

// Half of the pair that holds bin b (1..199): 0 for bins 1..50 and
// 150..199, 1 for bins 51..149.
__host__ __device__ constexpr int bin_half(int b) { return (b >= 51 && b <= 149) ? 1 : 0; }

// Where band m's bins lie: 0 all in role 0's half, 1 all in role 1's, 2 in
// both, -1 no bins.
__host__ __device__ constexpr int mel_side(int m) {
  int in0 = 0, in1 = 0;
  for (int j = 0; j < kMelCount[m]; ++j) {
    if (bin_half(kMelStart[m] + j)) in1 = 1; else in0 = 1;
  }
  return (in0 && in1) ? 2 : (in1 ? 1 : (in0 ? 0 : -1));
}
// First tap of band m whose bin lies in half h (-1: none).
__host__ __device__ constexpr int mel_first_tap(int m, int h) {
  int r = -1;
  for (int j = kMelCount[m] - 1; j >= 0; --j)
    if (bin_half(kMelStart[m] + j) == h) r = j;
  return r;
}
__host__ __device__ constexpr bool mel_layout_ok() {
  for (int m = 0; m < 128; ++m) {
    if (kMelCount[m] > 0 && (kMelStart[m] < 1 || kMelStart[m] + kMelCount[m] - 1 > 199))
      return false;                     // bins 0 and 200 have no register
  }
  return true;
}
static_assert(mel_layout_ok(), "mel bands do not fit the lane-pair layout");

// Power of bin b (1..199) in this lane's registers (right in half bin_half(b)).
__device__ __forceinline__ float bin_power(const float (&Pp)[51], const float (&Pm)[51], int b) {
  return b <= 50 ? Pp[b] : (b <= 100 ? Pp[b - 50] : (b <= 149 ? Pm[150 - b] : Pm[200 - b]));
}

// Sum of band m's terms whose bins lie in half h, over this lane's registers
// (right in half h; one instance per band and half, so that every index
// and weight is a constant).
template <int m, int h>
__device__ __forceinline__ float mel_part(const float (&Pp)[51], const float (&Pm)[51]) {
  constexpr int n = kMelCount[m], k0 = kMelStart[m], f = mel_first_tap(m, h);
  static_assert(f >= 0, "band has no bins in this half");
  float acc = 0.0f;
#pragma unroll
  for (int j = 0; j < n; ++j) {
    if (bin_half(k0 + j) != h) continue;
    const float t = kMelW[m][j] * bin_power(Pp, Pm, k0 + j);
    acc = (j == f) ? t : acc + t;
  }
  return acc;
}

// Which role of a pair logs band m: the roles take alternate runs of U
// bands of the row, role 0 the first. With a run of one 16-byte piece (U = 4
// for fp32 output, 8 for fp16) the two lanes of a pair store adjacent pieces
// of their frame's row, 32 contiguous bytes per store instruction and frame,
// which the memory pipeline takes faster than pieces 256 bytes apart.
template <int U>
__host__ __device__ constexpr int band_role(int m) { return (m / U) & 1; }
// The j-th band (j = 0..63) that role r logs.
template <int U>
__host__ __device__ constexpr int band_of(int r, int j) { return (j / U) * 2 * U + r * U + j % U; }
// Whether band m's logging role needs the other half's partial sum.
template <int U>
__host__ __device__ constexpr bool band_xfer(int m) {
  return mel_side(m) == 2 || (mel_side(m) >= 0 && mel_side(m) != band_role<U>(m));
}
// Slot of band m among the partial sums moved towards its logging role (in
// band order), and the number moved towards role r.
template <int U>
__host__ __device__ constexpr int xfer_slot(int m) {
  int n = 0;
  for (int k = 0; k < m; ++k)
    if (band_xfer<U>(k) && band_role<U>(k) == band_role<U>(m)) ++n;
  return n;
}
template <int U>
__host__ __device__ constexpr int xfer_count(int r) {
  int n = 0;
  for (int k = 0; k < 128; ++k)
    if (band_xfer<U>(k) && band_role<U>(k) == r) ++n;
  return n;
}

// The k-th band (in band order) whose partial sum moves towards role r.
template <int U>
__host__ __device__ constexpr int xfer_band(int r, int k) {
  int n = 0;
  for (int m = 0; m < 128; ++m)
    if (band_xfer<U>(m) && band_role<U>(m) == r && n++ == k) return m;
  return -1;
}

// The k-th moved sum of each direction, formed with the whole wavefront
// active (half 0's partial sum for the k-th band role 1 logs, half 1's for
// the k-th band role 0 logs) and exchanged with one v_permlane32_swap; a
// select by half then leaves role 0's received sum in lanes 0..31 and role
// 1's in lanes 32..63 of one register.
template <int U, int k, int NM>
__device__ __forceinline__ void xfer_one(const float (&Pp)[51], const float (&Pm)[51], bool upper,
                                         float (&M)[NM]) {
  constexpr int N0 = xfer_count<U>(1), N1 = xfer_count<U>(0);
  if constexpr (k < N0 && k < N1) {
    const float x0 = mel_part<xfer_band<U>(1, k), 0>(Pp, Pm);
    const float x1 = mel_part<xfer_band<U>(0, k), 1>(Pp, Pm);
    const auto w = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x1),
                                                     __builtin_bit_cast(uint32_t, x0), false,
                                                     false);
    // w[0]: x0 of lanes 0..31 in lanes 32..63; w[1]: x1 of lanes 32..63 in lanes 0..31
    M[k] = __builtin_bit_cast(float, upper ? w[0] : w[1]);
  } else if constexpr (k < N0) {
    M[k] = pair_from(mel_part<xfer_band<U>(1, k), 0>(Pp, Pm), 0);
  } else if constexpr (k < N1) {
    M[k] = pair_from(mel_part<xfer_band<U>(0, k), 1>(Pp, Pm), 1);
  }
}
template <int U, int NM, int... K>
__device__ __forceinline__ void xfer_all(const float (&Pp)[51], const float (&Pm)[51], bool upper,
                                         float (&M)[NM], std::integer_sequence<int, K...>) {
  (xfer_one<U, K, NM>(Pp, Pm, upper, M), ...);
}

// Energy of the j-th band role r logs; R holds the partial sums received
// from the other half (right in role r's lanes).
template <int U, int r, int j, int NR>
__device__ __forceinline__ float band_energy(const float (&Pp)[51], const float (&Pm)[51],
                                             const float (&R)[NR > 0 ? NR : 1]) {
  constexpr int m = band_of<U>(r, j);
  constexpr int side = mel_side(m);
  constexpr int slot = band_xfer<U>(m) ? xfer_slot<U>(m) : 0;
  if constexpr (side < 0) {
    // An empty filter's sum of zero-weight terms: 0, or NaN where the
    // frame's powers are NaN (a NaN sample reaches every bin).
    return 0.0f * Pp[1];
  } else if constexpr (side == r) {
    return mel_part<m, r>(Pp, Pm);
  } else if constexpr (side == 1 - r) {
    return R[slot];
  } else {
    // Half 0's partial sum plus half 1's, one rounding, whichever role adds
    // them: with contraction off the add is not folded into the last
    // multiply-add of either sum, so the fp32 and fp16 kernels (whose roles
    // log different bands) give a band the same energy.
    const float own = mel_part<m, r>(Pp, Pm), other = R[slot];
    {
#pragma clang fp contract(off)
      return own + other;
    }
  }
}
template <int U, int r, int NR, int... J>
__device__ __forceinline__ void role_bands(const float (&Pp)[51], const float (&Pm)[51],
                                           const float (&R)[NR > 0 ? NR : 1], float (&E)[64],
                                           std::integer_sequence<int, J...>) {
  ((E[J] = band_energy<U, r, J, NR>(Pp, Pm, R)), ...);
}

// The log-mel values of the 64 bands this lane logs, out[j] for band
// band_of<U>(role, j).
template <int U>
__device__ __forceinline__ void pair_logmel(const float (&Pp)[51], const float (&Pm)[51], int role,
                                            float (&out)[64]) {
  constexpr int N0 = xfer_count<U>(1), N1 = xfer_count<U>(0);   // towards role 1, role 0
  constexpr int NM = (N0 > N1 ? N0 : N1) > 0 ? (N0 > N1 ? N0 : N1) : 1;
  float M[NM];
  xfer_all<U, NM>(Pp, Pm, role != 0, M, std::make_integer_sequence<int, NM>{});
  // Each role sums only the bands it logs (the other half of the wavefront
  // is masked off meanwhile), so no select between the two sets is needed.
  float E[64];
  if (role == 0) {
    role_bands<U, 0, NM>(Pp, Pm, M, E, std::make_integer_sequence<int, 64>{});
  } else {
    role_bands<U, 1, NM>(Pp, Pm, M, E, std::make_integer_sequence<int, 64>{});
  }
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    // A band's energy is a sum of products of non-negative weights and
    // powers: +0 or more, or NaN. Such floats order like their bit patterns
    // read as unsigned integers, and every NaN lies above +Inf, so the
    // integer maximum with the floor is max(e, 1e-10) that keeps NaN.
    const uint32_t b = __builtin_bit_cast(uint32_t, E[i]), f = __builtin_bit_cast(uint32_t, kLogFloor);
    out[i] = __builtin_amdgcn_logf(__builtin_bit_cast(float, __builtin_elementwise_max(b, f))) * kLn2;
  }
}

}  // namespace logmel
