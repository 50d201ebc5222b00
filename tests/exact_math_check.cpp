// Host check of the exactly rounded helpers in quantized_rl_amd/csrc/exact_math.hpp
// against x86 IEEE-754 fp32 division and square root (SSE, round to nearest even).
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <random>

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
  printf("sqrt_rn: %llu checked, %llu mismatches\n", (unsigned long long)n_sqrt, (unsigned long long)bad_sqrt);
  printf("amax_over_448: %llu checked, %llu mismatches\n", (unsigned long long)n_s, (unsigned long long)bad_s);
  printf("div_by_scale: %llu checked, %llu mismatches\n", (unsigned long long)n_div, (unsigned long long)bad_div);
  return (bad_sqrt || bad_div || bad_s) ? 1 : 0;
}
