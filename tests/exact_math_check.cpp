// Host check of the exactly rounded helpers in quantized_rl_amd/csrc/exact_math.hpp
// against x86 IEEE-754 fp32 division and square root (SSE, round to nearest even).
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <random>
#include <cstring>

#include "../quantized_rl_amd/csrc/exact_math.hpp"

using namespace jetfp8;

int main(int argc, char** argv) {
  const uint32_t stride = argc > 1 ? (uint32_t)atoi(argv[1]) : 3;
  uint64_t bad_sqrt = 0, n_sqrt = 0;
  // every stride-th positive finite fp32, including all subnormals near zero
  for (uint64_t b = 1; b < 0x7f800000ull; b += (b < (1u << 20) ? 1 : stride)) {
    const float d = f32_from_bits((uint32_t)b);
    volatile float ref = std::sqrt(d);
    if (f32_bits(sqrt_rn(d)) != f32_bits(ref)) {
      if (bad_sqrt < 5) printf("sqrt mismatch d=%a got %a want %a\n", d, sqrt_rn(d), (float)ref);
      ++bad_sqrt;
    }
    ++n_sqrt;
  }
  // S = amax / 448: every stride-th positive finite fp32 (all of them with stride 1),
  // all subnormals and the smallest normals
  uint64_t bad_s = 0, n_s = 0;
  for (uint64_t b = 1; b < 0x7f800000ull; b += (b < (1u << 24) ? 1 : stride)) {
    const float a = f32_from_bits((uint32_t)b);
    volatile float ref = a / 448.0f;
    if (f32_bits(amax_over_448(a)) != f32_bits(ref)) {
      if (bad_s < 5) printf("amax/448 mismatch amax=%a got %a want %a\n", a, amax_over_448(a), (float)ref);
      ++bad_s;
    }
    ++n_s;
  }
  // quotient x / S: random pairs, plus pairs constructed next to fp32 midpoints
  std::mt19937_64 rng(1234);
  uint64_t bad_div = 0, n_div = 0;
  auto check = [&](float x, float s) {
    if (!(std::isfinite(x) && std::isfinite(s)) || s == 0.0f) return;
    volatile float ref = x / s;
    if (!std::isfinite(ref) || std::fabs(ref) < 0x1p-126f) return;  // subnormal quotients: zero code either way
    const float got = div_by_scale(x, 1.0 / (double)s);
    if (f32_bits(got) != f32_bits(ref)) {
      if (bad_div < 5) printf("div mismatch x=%a s=%a got %a want %a\n", x, s, got, (float)ref);
      ++bad_div;
    }
    ++n_div;
  };
  for (int i = 0; i < 20000000; ++i) {
    const float x = f32_from_bits((uint32_t)rng() & 0x7fffffffu) * ((rng() & 1) ? 1.f : -1.f);
    const float s = f32_from_bits(((uint32_t)rng() % 0x7f000000u) + 0x00800000u);
    check(x, s);
    // amax-style scales and in-range quotients
    const float a = std::ldexp((float)(rng() % 16777216u) / 16777216.0f + 0.5f, (int)(rng() % 200) - 100);
    const float sc = a / 448.0f;
    const float xi = a * ((float)(rng() % 1000000u) / 1000000.0f) * ((rng() & 1) ? 1.f : -1.f);
    check(xi, sc);
  }
  for (int i = 0; i < 5000000; ++i) {
    const float s = f32_from_bits(((uint32_t)rng() % 0x3f000000u) + 0x20000000u);
    const uint32_t mant = (uint32_t)(rng() & 0xffffffu) | 0x1000000u | 1u;  // odd 25-bit significand
    const double mid = std::ldexp((double)mant, -24 + (int)(rng() % 16) - 8);
    const float x0 = (float)(mid * (double)s);
    for (int k = -3; k <= 3; ++k) check(f32_from_bits(f32_bits(x0) + k), s);
  }
  // recip_nr from seeds perturbed by +-2^-14 (far worse than v_rcp_f64): within one
  // fp64 ulp of the correctly rounded 1/d, and fl32 of it equal to the fp32 division
  uint64_t bad_rcp = 0, n_rcp = 0, bad_r32 = 0, n_r32 = 0;
  for (uint64_t b = 1; b < 0x7f800000ull; b += (b < (1u << 20) ? 1 : 7 * stride)) {
    const float c = f32_from_bits((uint32_t)b);
    const double d = (double)c;
    volatile double ref64 = 1.0 / d;
    volatile float ref32 = 1.0f / c;
    for (int sgn = -1; sgn <= 1; sgn += 2) {
      const double r = recip_nr(d, ref64 * (1.0 + sgn * 0x1p-14));
      uint64_t rb, qb;
      double rr = ref64;
      memcpy(&rb, &r, 8);
      memcpy(&qb, &rr, 8);
      if ((rb > qb ? rb - qb : qb - rb) > 1) {
        if (bad_rcp < 5) printf("recip_nr mismatch d=%a got %a want %a\n", d, r, rr);
        ++bad_rcp;
      }
      ++n_rcp;
      if (std::isfinite(ref32) && std::fabs(ref32) >= 0x1p-126f) {
        if (f32_bits(recip_f32_from(c, r)) != f32_bits(ref32)) {
          if (bad_r32 < 5) printf("recip_f32 mismatch c=%a got %a want %a\n", c, recip_f32_from(c, r), (float)ref32);
          ++bad_r32;
        }
        ++n_r32;
      }
    }
  }
  // the two special operands, with the NaN the Newton steps give for them
  {
    const float inf = __builtin_inff();
    const double nan = __builtin_nan("");
    if (f32_bits(recip_f32_from(inf, recip_nr((double)inf, 0.0))) != f32_bits(1.0f / inf) ||
        f32_bits(recip_f32_from(0.0f, nan)) != f32_bits(1.0f / 0.0f)) {
      printf("recip_f32 special-case mismatch\n");
      ++bad_r32;
    }
    n_r32 += 2;
  }
  // the quotient with recip_nr's inverse (seeds perturbed as above)
  uint64_t bad_dnr = 0, n_dnr = 0;
  std::mt19937_64 rng2(99);
  for (int i = 0; i < 10000000; ++i) {
    const float a = std::ldexp((float)(rng2() % 16777216u) / 16777216.0f + 0.5f, (int)(rng2() % 250) - 140);
    const float sc = a / 448.0f;
    if (!(sc > 0.0f)) continue;
    const float xi = f32_from_bits(f32_bits(a) - (uint32_t)(rng2() % (1u << 26))) * ((rng2() & 1) ? 1.f : -1.f);
    volatile float ref = xi / sc;
    if (!std::isfinite(ref) || std::fabs(ref) < 0x1p-126f) continue;
    const double inv = recip_nr((double)sc, (1.0 / (double)sc) * (1.0 + ((rng2() & 1) ? 0x1p-14 : -0x1p-14)));
    if (f32_bits(div_by_scale(xi, inv)) != f32_bits(ref)) {
      if (bad_dnr < 5) printf("div (recip_nr) mismatch x=%a s=%a\n", xi, sc);
      ++bad_dnr;
    }
    ++n_dnr;
  }
  printf("recip_nr: %llu checked, %llu mismatches\n", (unsigned long long)n_rcp, (unsigned long long)bad_rcp);
  printf("recip_f32_from: %llu checked, %llu mismatches\n", (unsigned long long)n_r32, (unsigned long long)bad_r32);
  printf("div_by_scale (recip_nr inverse): %llu checked, %llu mismatches\n", (unsigned long long)n_dnr,
         (unsigned long long)bad_dnr);
  printf("sqrt_rn: %llu checked, %llu mismatches\n", (unsigned long long)n_sqrt, (unsigned long long)bad_sqrt);
  printf("amax_over_448: %llu checked, %llu mismatches\n", (unsigned long long)n_s, (unsigned long long)bad_s);
  printf("div_by_scale: %llu checked, %llu mismatches\n", (unsigned long long)n_div, (unsigned long long)bad_div);
  return (bad_sqrt || bad_div || bad_s || bad_rcp || bad_r32 || bad_dnr) ? 1 : 0;
}
