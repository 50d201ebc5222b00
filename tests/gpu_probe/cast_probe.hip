// GPU probe (test infrastructure): the library's E4M3 and bf16 conversions,
// as compiled into its kernels, against the integer definitions of cast_ref.hpp
// on every non-NaN fp32 bit pattern.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../quantized_rl_amd/csrc/device_common.hpp"
#include "cast_ref.hpp"

namespace {

constexpr uint32_t kThreads = 256;
constexpr uint32_t kBlocks = 8192;
constexpr uint64_t kPatterns = 1ull << 32;

__device__ __forceinline__ bool is_nan_bits(uint32_t u) { return (u & 0x7fffffffu) > 0x7f800000u; }

// Pairs of consecutive patterns (2p, 2p + 1) go through one packed conversion,
// as in the quantisers; mismatches are counted per thread and added once.
__global__ __launch_bounds__(kThreads) void probe_e4m3_kernel(unsigned long long* bad, uint32_t* first) {
  const uint64_t nthreads = (uint64_t)kThreads * kBlocks;
  unsigned long long nbad = 0;
  uint32_t f = 0xffffffffu;
  for (uint64_t p = (uint64_t)blockIdx.x * kThreads + threadIdx.x; p < kPatterns / 2; p += nthreads) {
    const uint32_t u0 = (uint32_t)(2 * p), u1 = u0 + 1;
    const int packed = jetfp8::cvt_pk_e4m3(__uint_as_float(u0), __uint_as_float(u1), 0, false);
    const uint32_t h0 = (uint32_t)packed & 0xffu, h1 = ((uint32_t)packed >> 8) & 0xffu;
    if (!is_nan_bits(u0) && h0 != castref::e4m3_code(u0)) { ++nbad; f = min(f, u0); }
    if (!is_nan_bits(u1) && h1 != castref::e4m3_code(u1)) { ++nbad; f = min(f, u1); }
  }
  if (nbad) {
    atomicAdd(bad, nbad);
    atomicMin(first, f);
  }
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// The GEMM epilogues' packed bf16 conversion (v_cvt_pk_bf16_f32 through the
// vector convert), lo in bits 0..15.
__global__ __launch_bounds__(kThreads) void probe_bf16_kernel(unsigned long long* bad, uint32_t* first) {
  const uint64_t nthreads = (uint64_t)kThreads * kBlocks;
  unsigned long long nbad = 0;
  uint32_t f = 0xffffffffu;
  for (uint64_t p = (uint64_t)blockIdx.x * kThreads + threadIdx.x; p < kPatterns / 2; p += nthreads) {
    const uint32_t u0 = (uint32_t)(2 * p), u1 = u0 + 1;
    const uint32_t packed = __builtin_bit_cast(
        uint32_t, __builtin_convertvector((f32x2_t){__uint_as_float(u0), __uint_as_float(u1)}, bf16x2_t));
    if (!is_nan_bits(u0) && (packed & 0xffffu) != castref::bf16_bits(u0)) { ++nbad; f = min(f, u0); }
    if (!is_nan_bits(u1) && (packed >> 16) != castref::bf16_bits(u1)) { ++nbad; f = min(f, u1); }
  }
  if (nbad) {
    atomicAdd(bad, nbad);
    atomicMin(first, f);
  }
}

}  // namespace

// bad: device u64 (zeroed by the caller); first: device u32 (0xffffffff by the caller).
extern "C" int probe_e4m3_all_fp32(unsigned long long* bad, uint32_t* first, void* stream) {
  hipLaunchKernelGGL(probe_e4m3_kernel, dim3(kBlocks), dim3(kThreads), 0, (hipStream_t)stream, bad, first);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

extern "C" int probe_bf16_all_fp32(unsigned long long* bad, uint32_t* first, void* stream) {
  hipLaunchKernelGGL(probe_bf16_kernel, dim3(kBlocks), dim3(kThreads), 0, (hipStream_t)stream, bad, first);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}
