// Integer-arithmetic definitions of the two conversions the library takes from
// the hardware (test infrastructure): fp32 -> OCP E4M3FN code (nearest, ties to
// even, saturating at +-448, sign of zero kept) and fp32 -> bf16 (nearest, ties
// to even).  Host and device: the CPU tests tie the host build to the oracle's
// table encoder and to torch's bf16 conversion; the GPU probe compares the
// device build with the hardware conversions on every fp32 bit pattern.
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#include <hip/hip_runtime.h>
#define CASTREF_HD __host__ __device__ __forceinline__
#else
#define CASTREF_HD inline
#endif

namespace castref {

// E4M3FN: value (1 + m/8) 2^(e-7) for e = 1..15, (m/8) 2^-6 for e = 0.  For a
// magnitude with binade exponent E, the spacing of E4M3 values is 2^(max(E,-6)-3),
// and the code of n spacings is (max(E,-6) + 6) * 8 + n (n = 8..16 in the normal
// binades, where n = 16 carries into the next exponent; n = 0..8 below 2^-6).
CASTREF_HD uint32_t e4m3_code(uint32_t u) {
  const uint32_t sign = (u >> 31) << 7;
  const uint32_t a = u & 0x7fffffffu;
  if (a >= 0x43e00000u) return sign | 0x7eu;  // |x| >= 448 (and +-inf): saturate
  if (a == 0) return sign;
  const int bexp = (int)(a >> 23);
  const uint32_t frac = a & 0x7fffffu;
  // |x| = mant * 2^(E - 23) with a 24-bit mant for normals, E = -126 for subnormals
  const int E = bexp ? bexp - 127 : -126;
  const uint32_t mant = bexp ? (frac | 0x800000u) : frac;
  const int Ec = E > -6 ? E : -6;
  const int s = Ec - E + 20;  // mant / 2^s = |x| / 2^(Ec - 3)
  uint32_t n;
  if (s >= 32) {
    n = 0;  // mant < 2^24, so |x| is below 2^-8 spacings: rounds to zero
  } else {
    const uint32_t q = mant >> s, rem = mant & ((1u << s) - 1u), half = 1u << (s - 1);
    n = q + ((rem > half || (rem == half && (q & 1u))) ? 1u : 0u);
  }
  return sign | (uint32_t)((Ec + 6) * 8 + (int)n);
}

// fp32 -> bf16 bits, nearest even, for non-NaN inputs.
CASTREF_HD uint32_t bf16_bits(uint32_t u) {
  const uint32_t lsb = (u >> 16) & 1u;
  return (u + 0x7fffu + lsb) >> 16;
}

}  // namespace castref
