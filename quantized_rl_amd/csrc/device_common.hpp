// Device helpers shared by the gfx950 kernels of the FP8 linear layer.
//
// E4M3 here is the OCP E4M3FN format (largest finite value 448), the format
// fixed by the Jet-RL pages (paper.rainbus.top, section "FP8 量化 (E4M3 格式)").
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "exact_math.hpp"

namespace jetfp8 {

constexpr int kGroup = 128;        // quantisation group / block edge
constexpr float kE4M3Max = 448.0f;

// bf16 bits -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 values -> two E4M3 codes, packed into the low (hi_half = false) or
// high 16 bits of `old`.  Rounding is nearest-even; the explicit clamp to
// +-448 gives saturation (the hardware conversion alone turns values of 480 and
// above into NaN).  On gfx950 v_cvt_pk_fp8_f32 of a value in [-448, 448] equals
// the nearest-even E4M3 code, sign of zero and fp32 subnormals included: the
// GPU test tests/test_gpu_casts.py compares this function with an integer
// definition of the cast on every non-NaN fp32 bit pattern.
__device__ __forceinline__ int cvt_pk_e4m3(float a, float b, int old, bool hi_half) {
  a = __builtin_amdgcn_fmed3f(a, -kE4M3Max, kE4M3Max);
  b = __builtin_amdgcn_fmed3f(b, -kE4M3Max, kE4M3Max);
  return hi_half ? __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, true)
                 : __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, false);
}

// S = amax / 448 rounded as the IEEE fp32 division (amax_over_448, exact for
// every non-negative finite amax); S = 1 when that quotient is zero: an
// all-zero group, or a nonzero amax of at most 448 * 2^-150 whose quotient
// underflows (reachable only from fp32 inputs: requantised or normalised
// values).  With S = 1 every code of such a group is e4m3(x), a signed zero.
__device__ __forceinline__ float scale_from_amax(float amax) {
  const float s = amax_over_448(amax);
  return s == 0.0f ? 1.0f : s;
}

// 1 / S in fp64 within one ulp, for the quotient fl32(fl64(x * (1 / S))):
// v_rcp_f64 refined by recip_nr (a handful of full-rate fp64 operations
// instead of the IEEE division sequence).
__device__ __forceinline__ double inv_scale(float s) {
  const double d = (double)s;
  return recip_nr(d, __builtin_amdgcn_rcp(d));
}

// fl32(1 / c), correctly rounded, for a non-negative fp32 c (recip_f32_from).
__device__ __forceinline__ float recip_f32_rn(float c) { return recip_f32_from(c, inv_scale(c)); }

// Cross-lane moves inside a 16-lane DPP row (a quarter-wave), in registers:
//   kXor1  quad_perm [1,0,3,2]: lane l reads lane l ^ 1
//   kXor2  quad_perm [2,3,0,1]: lane l reads lane l ^ 2
//   kHalfMirror row_half_mirror: lane l reads lane 7 - l within its 8-lane half-row
//   kMirror     row_mirror:      lane l reads lane 15 - l within its row
// Once every lane of an aligned group of 4 (resp. 8) holds the same value, the
// two mirrors deliver the value of the neighbouring group, exactly as a xor 4
// (resp. xor 8) exchange would.
constexpr int kXor1 = 0xB1, kXor2 = 0x4E, kHalfMirror = 0x141, kMirror = 0x140;
template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, false));
}

// Max over the 16 lanes of a quarter-wave (lanes 16q .. 16q+15) of
// non-negative values (group amaxes).  The fp32 bit patterns are compared as
// unsigned integers, which orders non-negative floats as their values, so the
// DPP reads need none of the NaN-quieting moves an fp32 max puts around them.
template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t u) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, kCtrl, 0xF, 0xF, false);
}
__device__ __forceinline__ float quarter_wave_max(float v) {
  uint32_t u = __float_as_uint(v);
  u = max(u, dpp_u32<kXor1>(u));
  u = max(u, dpp_u32<kXor2>(u));
  u = max(u, dpp_u32<kHalfMirror>(u));
  u = max(u, dpp_u32<kMirror>(u));
  return __uint_as_float(u);
}

// Max over the 64 lanes of non-negative values.
__device__ __forceinline__ float wave_max(float v) {
  uint32_t u = __float_as_uint(quarter_wave_max(v));
  u = max(u, (uint32_t)__shfl_xor((int)u, 16, 64));
  u = max(u, (uint32_t)__shfl_xor((int)u, 32, 64));
  return __uint_as_float(u);
}

// Sum over the 64 lanes as the balanced binary tree over lane order: level k
// adds the partial sums of the aligned lane groups of size 2^k that differ in
// bit k (a xor butterfly), so every partial is a node of the canonical tree and
// all lanes end with the same value.  Levels 0..3 stay inside a 16-lane row.
__device__ __forceinline__ float wave_sum_tree(float v) {
  v = v + dpp<kXor1>(v);
  v = v + dpp<kXor2>(v);
  v = v + dpp<kHalfMirror>(v);
  v = v + dpp<kMirror>(v);
  v = v + __shfl_xor(v, 16, 64);
  v = v + __shfl_xor(v, 32, 64);
  return v;
}

// Quantise eight fp32 values of one group with inverse scale `inv_s`;
// returns their eight codes as two dwords (element order preserved).
__device__ __forceinline__ uint2 quant8(const float (&f)[8], double inv_s) {
  int lo = cvt_pk_e4m3(div_by_scale(f[0], inv_s), div_by_scale(f[1], inv_s), 0, false);
  lo = cvt_pk_e4m3(div_by_scale(f[2], inv_s), div_by_scale(f[3], inv_s), lo, true);
  int hi = cvt_pk_e4m3(div_by_scale(f[4], inv_s), div_by_scale(f[5], inv_s), 0, false);
  hi = cvt_pk_e4m3(div_by_scale(f[6], inv_s), div_by_scale(f[7], inv_s), hi, true);
  return make_uint2((uint32_t)lo, (uint32_t)hi);
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Streaming (non-temporal) 16-byte load: the quantisers read each input byte
// once.  Their outputs go out with plain 8- and 16-byte stores: the codes are
// the operands of the GEMM (or requantisation) that runs next, and left in the
// caches (L2, MALL) they made the 8B training step about 4 % faster than
// streaming stores did (FProp and DGrad 6-8 % faster, the quantisers 1-4 us
// slower each).
__device__ __forceinline__ uint4 ld_stream16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_global8(void* p, uint2 v) {
  *reinterpret_cast<u32x2_t*>(p) = u32x2_t{v.x, v.y};
}
__device__ __forceinline__ void st_global16(void* p, uint4 v) {
  *reinterpret_cast<u32x4_t*>(p) = u32x4_t{v.x, v.y, v.z, v.w};
}

// Eight bf16 values (one 16-byte load) -> fp32.
__device__ __forceinline__ void unpack_bf16x8(uint4 v, float (&f)[8]) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
  f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
  f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

__device__ __forceinline__ float absmax8(const float (&f)[8]) {
  float a = fabsf(f[0]);
#pragma unroll
  for (int i = 1; i < 8; ++i) a = fmaxf(a, fabsf(f[i]));
  return a;
}

}  // namespace jetfp8
