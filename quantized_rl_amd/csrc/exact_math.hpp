// Exactly rounded fp32 helpers used by the quantisation kernels.
//
// Host and device code: the host build exists so that the CPU test-suite can
// check these functions exhaustively against x86's IEEE fp32 division and
// square root (tests/test_exact_math.py).
#pragma once

#include <stdint.h>
#include <string.h>

#if defined(__HIPCC__)
#include <hip/hip_runtime.h>
#define JETFP8_HD __host__ __device__ __forceinline__
#else
#define JETFP8_HD inline
#endif

namespace jetfp8 {

JETFP8_HD uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
JETFP8_HD float f32_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
JETFP8_HD uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = f32_bits(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// 1 / d in fp64 to within one ulp (relative error below 2^-52) for an fp64 d
// that is an fp32 value (normal or subnormal), from a seed r0 with relative
// error below 2^-20: two Newton-Raphson steps with fused multiply-adds.  Each
// step squares the seed's relative error (2^-20 -> 2^-40 -> 2^-80) and adds
// the rounding of its own fma (2^-53).  The device seed is v_rcp_f64; the host
// check drives it with seeds perturbed by +-2^-20.
JETFP8_HD double recip_nr(double d, double r0) {
  double e = __builtin_fma(-d, r0, 1.0);
  const double r1 = __builtin_fma(r0, e, r0);
  e = __builtin_fma(-d, r1, 1.0);
  return __builtin_fma(r1, e, r1);
}

// fl32(1 / c) for a non-negative fp32 c, from an fp64 value r within 2^-52
// (relative) of 1 / c when c is positive and finite: c * m != 1 for every
// fp32 rounding midpoint m (m has an odd 25-bit significand), and C * Mi - 2^j
// for the integer significands is a nonzero integer, so 1 / c lies at least
// 2^-49 (relative) from every midpoint and r rounds to the same fp32 value.
// c = +inf gives +0 and c = 0 gives +inf, as the IEEE division does (r is
// not used there: the Newton steps give NaN for those two).
JETFP8_HD float recip_f32_from(float c, double r) {
  const float inf = __builtin_inff();
  return c == inf ? 0.0f : (c == 0.0f ? inf : (float)r);
}

// fl32(x / S) computed as fl32(fl64(x * inv_s)), with inv_s within one ulp of
// 1 / S (fl64(1 / S), or recip_nr's result).
//
// Why this equals the correctly rounded fp32 quotient: inv_s adds a relative
// error of at most 2^-52 and the fp64 product at most 2^-53, so
// z = fl64(x * inv_s) is within 2^-51.4 (relative) of x / S.  For fp32 x and S, x / S is never an fp32
// rounding midpoint (a midpoint has an odd 25-bit significand, so S times it
// needs more than 24 significant bits), and its relative distance to the
// nearest midpoint is at least 2^-49 (x - S * midpoint is a nonzero multiple of
// the last place of that product).  So z rounds to the same fp32 value as
// x / S.  Quotients below 2^-126 may round differently in the fp32 subnormal
// range, where the E4M3 cast gives a zero code either way.
JETFP8_HD float div_by_scale(float x, double inv_s) { return (float)((double)x * inv_s); }

// S = fl32(amax / 448) for a non-negative finite amax, computed as
// fl32(fl64(amax * fl64(1 / 448))).  fl64(1/448) and the fp64 product each add
// at most 2^-53 of relative error, so the fp64 value is within 2^-52 of
// amax / 448, which is never an fp32 rounding midpoint in the normal range (a
// midpoint times 448 = 7 * 2^6 needs at least 27 significant bits) and lies
// relatively at least about 2^-27 away from one; the one fp32 rounding then
// gives the correctly rounded quotient.  The host check compares it with the
// IEEE fp32 division on every positive finite fp32 value, subnormal results
// included (no mismatch).  Three operations instead of a full division.
JETFP8_HD float amax_over_448(float amax) { return (float)((double)amax * (1.0 / 448.0)); }

// Correctly rounded fp32 square root of a non-negative finite d.
//
// The hardware square root is only accurate to about one ulp, so the result is
// settled exactly: c is within one ulp of sqrt(d); sqrt(d) lies above the
// midpoint m between c and its upper neighbour iff d > m * m, and below the
// lower midpoint iff d < m' * m'.  Each midpoint has at most 25 significant
// bits, so its square is exact in fp64, and d is exact in fp64: both tests are
// exact.  (sqrt(d) is never exactly a midpoint: its square would need more
// than 24 significant bits.)
JETFP8_HD float sqrt_rn(float d) {
  const float c = (float)__builtin_sqrt((double)d);
  if (!(d > 0.0f) || !(c < 3.0e38f)) return c;
  const float up = f32_from_bits(f32_bits(c) + 1u);
  const float dn = f32_from_bits(f32_bits(c) - 1u);
  const double mu = 0.5 * ((double)c + (double)up);
  const double md = 0.5 * ((double)c + (double)dn);
  const double dd = (double)d;
  if (dd > mu * mu) return up;
  if (dd < md * md) return dn;
  return c;
}

}  // namespace jetfp8
