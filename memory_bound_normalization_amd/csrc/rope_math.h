// Rotary-angle arithmetic of the fused QK-norm + RoPE kernel, shared by the
// kernel (device) and a host build of the same functions that the CPU tests
// check against high-precision values.
//
// Rotary embedding with rotate-half pairing ("[pretuned] Optimize
// fused_qk_norm_rope on B200", Summary): pair i < R/2 of a head turns by the
// angle pos * theta^(-2i/R). The inverse frequencies theta^(-2i/R) do not
// depend on the token: the host evaluates the six powers theta^(-2^(k+1)/R),
// k < 6, once per launch, and lane i of the kernel multiplies the powers whose
// bit k is set in i.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>

namespace mbn {

// theta^(-2^(k+1)/R) for k < 6 (fp64); pair i < R/2 <= 64 has the inverse
// frequency prod_{bit k of i set} p[k].
struct InvFreqPowers {
  double p[6];
};

// Host: the six powers in x87 extended precision (64-bit significands: the
// exponent -2^(k+1)/R, inexact in fp64 for R not a power of two, then errs by
// ~5e-20 rather than ~1e-16 relative, which pow would scale by ln theta),
// rounded to fp64. Against exact values each power is within about half an
// ulp; formed in fp64 the worst product over theta in {2, 1e4, 5e5, 1e6} and
// R = 16 ... 128 was 9.6e-16 relative, this way 3.3e-16.
inline InvFreqPowers rope_inv_freq_powers(float theta, int rotary_dim) {
  InvFreqPowers ip{};
  for (int k = 0; k < 6; ++k)
    ip.p[k] = (double)std::pow((long double)theta, -(long double)(2 << k) / (long double)rotary_dim);
  return ip;
}

// theta^(-2i/R) for pair i from the powers: at most six fp64 products, taken
// in the order of the bits of i (the kernel's order), so a relative error of
// at most about seven ulps.
__host__ __device__ inline double rope_inv_freq(const InvFreqPowers& ip, int i) {
  double f = 1.0;
#pragma unroll
  for (int k = 0; k < 6; ++k)
    if ((i >> k) & 1) f *= ip.p[k];
  return f;
}

// sin and cos of an fp64 angle for |phi| < 2^40 (else the library's sincos).
// Cody-Waite reduction: k = rint(phi * 2/pi), r = phi - k * pi/2 with pi/2
// split into three doubles P1 + P2 + P3 and one FMA per part. phi - k * P1 is
// a multiple of 2^-53 below 2 in magnitude, hence exact; the other two parts
// add about one ulp of r. On |r| <= pi/4 (+ a rounding of k), Taylor series
// to r^15 (sine) and r^16 (cosine), truncation below 5e-17, plus a few ulps of
// Horner rounding. The quadrant k mod 4 then permutes and negates the pair.
// About 30 fp64 operations against the library routine's general path; the
// angle work sits on the critical path of short launches.
__host__ __device__ inline void sincos_reduced(double phi, double* s_out, double* c_out) {
  if (!(__builtin_fabs(phi) < 0x1p40)) {
    sincos(phi, s_out, c_out);
    return;
  }
  constexpr double kTwoOverPi = 0.6366197723675814;  // fl(2/pi)
  constexpr double kP1 = 1.5707963267948966;         // fl(pi/2)
  constexpr double kP2 = 6.123233995736766e-17;      // fl(pi/2 - P1)
  constexpr double kP3 = -1.4973849048591698e-33;    // fl(pi/2 - P1 - P2)
  const double k = __builtin_rint(phi * kTwoOverPi);
  double r = __builtin_fma(-k, kP1, phi);
  r = __builtin_fma(-k, kP2, r);
  r = __builtin_fma(-k, kP3, r);
  const double r2 = r * r;
  // sin r = r + r^3 * ps, ps = -1/3! + r^2/5! - r^4/7! + ... - r^12/15!
  double ps = -1.0 / 1307674368000.0;
  ps = __builtin_fma(ps, r2, 1.0 / 6227020800.0);
  ps = __builtin_fma(ps, r2, -1.0 / 39916800.0);
  ps = __builtin_fma(ps, r2, 1.0 / 362880.0);
  ps = __builtin_fma(ps, r2, -1.0 / 5040.0);
  ps = __builtin_fma(ps, r2, 1.0 / 120.0);
  ps = __builtin_fma(ps, r2, -1.0 / 6.0);
  const double sn = __builtin_fma(ps * r2, r, r);
  // cos r = 1 - r^2 * pc, pc = 1/2! - r^2/4! + r^4/6! - ... - r^14/16!
  double pc = -1.0 / 20922789888000.0;
  pc = __builtin_fma(pc, r2, 1.0 / 87178291200.0);
  pc = __builtin_fma(pc, r2, -1.0 / 479001600.0);
  pc = __builtin_fma(pc, r2, 1.0 / 3628800.0);
  pc = __builtin_fma(pc, r2, -1.0 / 40320.0);
  pc = __builtin_fma(pc, r2, 1.0 / 720.0);
  pc = __builtin_fma(pc, r2, -1.0 / 24.0);
  pc = __builtin_fma(pc, r2, 0.5);
  const double cs = __builtin_fma(-pc, r2, 1.0);
  // phi = k pi/2 + r: quadrant q = k mod 4 (two's complement for k < 0)
  const int q = (int)((long long)k & 3);
  const double s = (q & 1) ? cs : sn;
  const double c = (q & 1) ? sn : cs;
  *s_out = (q & 2) ? -s : s;
  *c_out = ((q + 1) & 2) ? -c : c;
}

}  // namespace mbn
