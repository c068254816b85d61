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
// adjacent lanes (a "pair"): role 0 transforms the even samples in order,
// e[m] = x[2m], role 1 the odd samples in reverse order, o[m] = x[399 - 2m]
// (decimation in time). The window is symmetric, w[399 - 2m] = w[2m], so
// both roles apply the same window values, and every constant of the
// routine is the same for all lanes. Each role runs the same code:
//   * a 200-point real DFT as a prime-factor (Good-Thomas) 8 x 25 transform,
//       m = (25 n1 + 8 n2) mod 200,  k = (25 k1 + 176 k2) mod 200,
//     with 8 real-input 25-point DFTs (5 x 5, conjugate halves skipped)
//     and 13 8-point DFTs for k2 = 0..12, which cover k = 0..100;
//   * the radix-2 combine. With E and R the two roles' spectra, the odd
//     samples' spectrum is W200^-k conj(R[k]), and multiplying X[k] by
//     W800^k (a unit phase) gives, with u = W800^k E[k], v = W800^k R[k],
//       |X[k]|       = |u + conj(v)|,
//       |X[200 - k]| = |u - conj(v)|.
//     Each role forms its own rotation (the same W800^k for both), swaps it
//     with its partner (DPP) and forms one of the two powers, so each lane
//     holds one half of the spectrum; the filterbank runs on the halves (see
//     pair_logmel) and each lane logs and stores one half of the 128 bands.
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

// Swap a double with the pair partner (lanes 2f <-> 2f+1): DPP quad_perm [1,0,3,2].
__device__ __forceinline__ double pair_swap(double v) {
  const long long b = __builtin_bit_cast(long long, v);
  // quad_perm reads a lane of the same quad for every lane, so no lane keeps
  // an old value (bound_ctrl is irrelevant and set).
  const int lo = __builtin_amdgcn_mov_dpp((int)b, 0xB1, 0xf, 0xf, true);
  const int hi = __builtin_amdgcn_mov_dpp((int)(b >> 32), 0xB1, 0xf, 0xf, true);
  return __builtin_bit_cast(double, ((long long)hi << 32) | (unsigned int)lo);
}

// The value of the pair's lane `src` (0 = even, 1 = odd) in both lanes.
__device__ __forceinline__ float pair_from(float v, int src) {
  const int b = __builtin_bit_cast(int, v);
  return __builtin_bit_cast(float, src == 0 ? __builtin_amdgcn_mov_dpp(b, 0xA0, 0xf, 0xf, true)
                                            : __builtin_amdgcn_mov_dpp(b, 0xF5, 0xf, 0xf, true));
}

// Power spectrum of one frame on a lane pair.
//   v[200]   this lane's samples, m = 0..199 (fp32): x[2m] for role 0,
//            x[399 - 2m] for role 1
//   win      w[2m], m = (25 n1 + 8 n2) mod 200, in [n1][n2] order (uniform)
//   rot      cos, sin of 2 pi kap / 800 for the bins in [k2][k1] order (uniform)
//   sgn      +1.0 for role 0, -1.0 for role 1
//   own[101] this lane's half of the power spectrum: own[kap] = |X[kap]|^2
//            for role 0 and |X[200 - kap]|^2 for role 1, kap = 1..100
__device__ __forceinline__ void pair_power(const float (&v)[200], const double* __restrict__ win,
                                           const double* __restrict__ rot, double sgn,
                                           float (&P)[101]) {
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
  // role's spectrum R at k = pfa_k(k1, k2) (k > 100 through conjugation);
  // rotate, swap with the partner, and form this role's power of bin k or
  // bin 200 - k.
  P[0] = 0.0f;   // no filter reaches bins 0 and 200
#pragma unroll
  for (int k2 = 0; k2 <= 12; ++k2) {
    cd q[8];
#pragma unroll
    for (int n1 = 0; n1 < 8; ++n1) {
      q[n1] = A[n1][k2];
      fence(q[n1].re);
      if (k2 > 0) fence(q[n1].im);
    }
    // This column's rotations, loaded ahead of the 8-point DFT so that the
    // scalar loads overlap it.
    double rc[8], rs[8];
#pragma unroll
    for (int k1 = 0; k1 < 8; ++k1) {
      rc[k1] = rot[16 * k2 + 2 * k1];
      rs[k1] = rot[16 * k2 + 2 * k1 + 1];
    }
    dft8(q);
#pragma unroll
    for (int k1 = 0; k1 < 8; ++k1) {
      if (k2 == 0 && k1 > 4) continue;          // conjugates of k1 = 1..3
      const int k = pfa_k(k1, k2);
      const int kap = k <= 100 ? k : 200 - k;
      if (kap == 0) continue;                   // bins 0 and 200 carry no weight
      const cd r = k <= 100 ? q[k1] : cd{q[k1].re, -q[k1].im};
      // r * W800^kap, the same rotation in both roles
      const cd u = c_twiddle(r, rc[k1], rs[k1]);
      const cd w = {pair_swap(u.re), pair_swap(u.im)};
      // role 0: |u + conj(w)|^2 = bin kap; role 1: |u - conj(w)|^2 = bin 200 - kap
      const double are = w.re * sgn + u.re, aim = u.im - w.im * sgn;
      P[kap] = (float)(are * are + aim * aim);
    }
    // one scheduling region per column
#pragma unroll
    for (int k1 = 0; k1 < 8; ++k1) {
      if (k2 == 0 && k1 > 4) continue;
      const int k = pfa_k(k1, k2);
      const int kap = k <= 100 ? k : 200 - k;
      if (kap == 0) continue;
      fence(P[kap]);
    }
  }

}

// Band-sparse mel projection and log. Each lane holds only its own half of
// the spectrum (own[kap]: bin kap in role 0, bin 200 - kap in role 1), and
// both run the same code: a band whose bins all lie below 100 is summed over
// own[bin] (right in role 0), a band whose bins all lie above 100 over
// own[200 - bin] (right in role 1), and the bands around bin 100 as the two
// partial sums. Role 0 logs bands 0..63, all below bin 100; role 1 logs bands
// 64..127 and takes the energies that only role 0 holds from its partner
// (DPP). The log has the 1e-10 floor; the floor test keeps a NaN energy NaN.
__host__ __device__ constexpr int mel_side(int m) {   // 0: bins < 100, 1: bins > 100, 2: both
  return kMelCount[m] == 0 ? 0
       : (kMelStart[m] + kMelCount[m] - 1 < 100 ? 0 : (kMelStart[m] > 100 ? 1 : 2));
}

// Energy of band m from this lane's half spectrum (bins in order, one
// instance per band so that every index and weight is a constant).
template <int m>
__device__ __forceinline__ float mel_band(const float (&own)[101]) {
  constexpr int n = kMelCount[m], k0 = kMelStart[m], side = mel_side(m);
  if constexpr (n == 0) {
    // An empty filter's sum of zero-weight terms: 0, or NaN where the
    // frame's powers are NaN (a NaN sample reaches every bin).
    return 0.0f * own[1];
  } else {
    float lo = 0.0f, hi = 0.0f;
#pragma unroll
    for (int j = 0; j < n; ++j) {
      const int bin = k0 + j;
      if (bin <= 100) {
        lo = (bin == k0) ? kMelW[m][j] * own[bin] : lo + kMelW[m][j] * own[bin];
      } else {
        hi = (bin == k0 || bin == 101) ? kMelW[m][j] * own[200 - bin]
                                       : hi + kMelW[m][j] * own[200 - bin];
      }
    }
    if constexpr (side == 0) {
      return m < 64 ? lo : pair_from(lo, 0);
    } else if constexpr (side == 1) {
      return hi;
    } else {
      return pair_from(lo, 0) + hi;
    }
  }
}

template <int... M>
__device__ __forceinline__ void mel_bands(const float (&own)[101], float (&E)[128],
                                          std::integer_sequence<int, M...>) {
  ((E[M] = mel_band<M>(own)), ...);
}

__device__ __forceinline__ void pair_logmel(const float (&own)[101], int role, float (&out)[64]) {
  float E[128];
  mel_bands(own, E, std::make_integer_sequence<int, 128>{});
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    float e = role ? E[64 + i] : E[i];
    e = (e < kLogFloor) ? kLogFloor : e;
    out[i] = __builtin_amdgcn_logf(e) * kLn2;
  }
}

}  // namespace logmel
