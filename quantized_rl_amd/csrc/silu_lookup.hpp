// SiLU of a bf16 gate from its 16 bits, by lookup, for gfx950.
//
//   silu(g) = fl32(g / fl32(1 + E)),  E = the fp32 value nearest to e^-g
//
// (SiLU and its exponential are readings: the pages print no formula.)  For the
// 8192 bf16 values with 2^-25 <= |g| < 2^7 the value comes from a table that
// silu_table_gen.cpp generates at build time from the definition (the
// test-suite compares every entry with the oracle); the kernels copy it into
// LDS.  Outside that range silu has a closed form: |g| < 2^-25 gives E = 1 and
// silu = g / 2 (exact), g >= 2^7 gives E = 0 and silu = g, g <= -2^7 gives
// E = +inf and silu = -0.  Table index: sign << 12 | (biased exponent - 102) << 7
// | mantissa.
#pragma once
#include <cstdint>

namespace jetfp8 {

constexpr uint32_t kSiluExpLo = 102, kSiluExpHi = 134;  // biased exponents of 2^-25 and 2^7
constexpr int kSiluBinades = (int)(kSiluExpHi - kSiluExpLo);
constexpr int kSiluTable = 2 * kSiluBinades * 128;  // 8192 entries (32 KB)

__device__ __forceinline__ float silu_of_bits(uint32_t b, const float* tab) {
  const float g = __uint_as_float(b << 16);
  const uint32_t e = (b >> 7) & 0xFFu;
  const bool in = e - kSiluExpLo < (uint32_t)kSiluBinades;
  const uint32_t idx = in ? (((b >> 15) & 1u) << 12) + ((e - kSiluExpLo) << 7) + (b & 0x7Fu) : 0u;
  const float t = tab[idx];
  const float outside = e < kSiluExpLo ? g * 0.5f : ((b & 0x8000u) ? -0.0f : g);
  return in ? t : outside;
}

}  // namespace jetfp8
