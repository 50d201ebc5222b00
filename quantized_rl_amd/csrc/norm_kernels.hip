// RMSNorm backward for gfx950: the gradients of y = x * gamma * rstd
// (rstd = (mean_k x_k^2 + eps)^(-1/2) per row, saved by the forward) for an
// upstream gradient dy, all in fp32 from bf16 inputs:
//
//   c_m      = fl32(S_m / K),  S_m = sum_k fl32(fl32(gamma_k * dy_mk) * x_mk)
//   dx_mk    = fl32(r * fl32(fl32(gamma_k * dy_mk) - fl32(x_mk * fl32(fl32(r * r) * c_m))))
//   dgamma_k = sum_m fl32(fl32(dy_mk * x_mk) * r_m)
//
// dx is rounded to bf16 (nearest even); dgamma stays fp32.  The pages name a
// fused RMSNorm in the forward of the FP8 linear (Jet-RL pages,
// paper.rainbus.top summary, "方法步骤详情" step 5) and train through it;
// the formulas are calculus on the standard RMSNorm.
//
// Both are HBM-bound: x and dy are read once, dx written once.
//   rmsnorm_backward_rows_kernel: a workgroup of 4 waves owns 4 R consecutive
//     rows, R per wave, one row at a time; R = ceil(M / 1024) clamped to
//     1..8, so that small batches still spread over many workgroups.  Lane l
//     covers the 8 elements at 512 p + 8 l of pass p (all loads of a row
//     issued up front).  S is the lane's sequential sum followed by the wave
//     butterfly.  Each wave keeps its rows' dgamma terms in registers (summed
//     in row order); the four waves then add theirs in wave order through LDS
//     and the workgroup writes its partial row of dgamma to the workspace.
//   rmsnorm_dgamma_reduce_kernel: dgamma_k = the partials summed in a fixed
//     order (four quarters in sequence, then ((q0 + q1) + q2) + q3).
// Identical inputs give identical bits; no atomics.
#include "device_common.hpp"
#include "launch.hpp"

namespace jetfp8 {

constexpr int kBwdMaxPasses = 12;  // K <= 6144

static int64_t bwd_rows_per_wave(int64_t M) {
  const int64_t r = (M + 1023) / 1024;
  return r < 1 ? 1 : (r > 8 ? 8 : r);
}

int64_t rmsnorm_backward_parts(int64_t M) {
  const int64_t rows = 4 * bwd_rows_per_wave(M);
  return (M + rows - 1) / rows;
}

__device__ __forceinline__ uint4 pack_bf16x8(const float (&f)[8]) {
  return make_uint4(f32_to_bf16_rne(f[0]) | (f32_to_bf16_rne(f[1]) << 16),
                    f32_to_bf16_rne(f[2]) | (f32_to_bf16_rne(f[3]) << 16),
                    f32_to_bf16_rne(f[4]) | (f32_to_bf16_rne(f[5]) << 16),
                    f32_to_bf16_rne(f[6]) | (f32_to_bf16_rne(f[7]) << 16));
}

template <int kP>
__global__ __launch_bounds__(256) void rmsnorm_backward_rows_kernel(const uint16_t* __restrict__ x,
                                                                    const uint16_t* __restrict__ gamma,
                                                                    const float* __restrict__ rstd,
                                                                    const uint16_t* __restrict__ dy,
                                                                    int64_t M, int64_t K, int rows_per_wave,
                                                                    uint16_t* __restrict__ dx,
                                                                    float* __restrict__ part) {
  __shared__ float red[512 * kP];
  const int t = threadIdx.x, l = t & 63, w = t >> 6;
  const int64_t row0 = ((int64_t)blockIdx.x * 4 + w) * rows_per_wave;

  float u[kP][8];
#pragma unroll
  for (int p = 0; p < kP; ++p)
#pragma unroll
    for (int i = 0; i < 8; ++i) u[p][i] = 0.0f;

  for (int r = 0; r < rows_per_wave; ++r) {
    const int64_t row = row0 + r;
    if (row >= M) break;  // uniform over the wave; no barrier inside the loop
    const float rr = rstd[row];
    uint4 xv[kP], dv[kP];
#pragma unroll
    for (int p = 0; p < kP; ++p) {
      const int64_t e = 512 * p + 8 * l;
      const bool in = p < kP - 1 || e < K;
      xv[p] = in ? ld_stream16(x + row * K + e) : make_uint4(0, 0, 0, 0);
      dv[p] = in ? ld_stream16(dy + row * K + e) : make_uint4(0, 0, 0, 0);
    }
    float sl = 0.0f;
#pragma unroll
    for (int p = 0; p < kP; ++p) {
      const int64_t e = 512 * p + 8 * l;
      const bool in = p < kP - 1 || e < K;
      float fx[8], fd[8], fg[8];
      unpack_bf16x8(xv[p], fx);
      unpack_bf16x8(dv[p], fd);
      unpack_bf16x8(in ? *reinterpret_cast<const uint4*>(gamma + e) : make_uint4(0, 0, 0, 0), fg);
#pragma unroll
      for (int i = 0; i < 8; ++i) sl = sl + (fg[i] * fd[i]) * fx[i];
    }
    const float c = wave_sum_tree(sl) / (float)K;
    const float rc = (rr * rr) * c;
#pragma unroll
    for (int p = 0; p < kP; ++p) {
      const int64_t e = 512 * p + 8 * l;
      const bool in = p < kP - 1 || e < K;
      float fx[8], fd[8], fg[8], o[8];
      unpack_bf16x8(xv[p], fx);
      unpack_bf16x8(dv[p], fd);
      unpack_bf16x8(in ? *reinterpret_cast<const uint4*>(gamma + e) : make_uint4(0, 0, 0, 0), fg);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        o[i] = rr * ((fg[i] * fd[i]) - fx[i] * rc);
        u[p][i] = u[p][i] + (fd[i] * fx[i]) * rr;
      }
      if (in) *reinterpret_cast<uint4*>(dx + row * K + e) = pack_bf16x8(o);
    }
  }

  // the four waves' dgamma terms, added in wave order
  for (int ww = 0; ww < 4; ++ww) {
    if (w == ww) {
#pragma unroll
      for (int p = 0; p < kP; ++p) {
        const int64_t e = 512 * p + 8 * l;
        if (p < kP - 1 || e < K) {
#pragma unroll
          for (int i = 0; i < 8; ++i) red[e + i] = ww == 0 ? u[p][i] : red[e + i] + u[p][i];
        }
      }
    }
    __syncthreads();
  }
  for (int64_t k = t; k < K; k += 256) part[(int64_t)blockIdx.x * K + k] = red[k];
}

__global__ __launch_bounds__(256) void rmsnorm_dgamma_reduce_kernel(const float* __restrict__ part,
                                                                    int64_t nparts, int64_t K,
                                                                    float* __restrict__ dgamma) {
  __shared__ float q[4][64];
  const int t = threadIdx.x, c = t & 63, w = t >> 6;
  const int64_t k = (int64_t)blockIdx.x * 64 + c;
  const int64_t per = (nparts + 3) / 4;
  const int64_t b = w * per;
  const int64_t e = b + per < nparts ? b + per : nparts;
  float acc = 0.0f;
  if (k < K) {
#pragma unroll 8
    for (int64_t j = b; j < e; ++j) acc = acc + part[j * K + k];
  }
  q[w][c] = acc;
  __syncthreads();
  if (w == 0 && k < K) dgamma[k] = ((q[0][c] + q[1][c]) + q[2][c]) + q[3][c];
}

template <int kP>
static void launch_bwd_rows(const uint16_t* x, const uint16_t* gamma, const float* rstd, const uint16_t* dy,
                            int64_t M, int64_t K, uint16_t* dx, float* part, hipStream_t stream) {
  hipLaunchKernelGGL(rmsnorm_backward_rows_kernel<kP>, dim3((unsigned)rmsnorm_backward_parts(M)), dim3(256), 0,
                     stream, x, gamma, rstd, dy, M, K, (int)bwd_rows_per_wave(M), dx, part);
}

hipError_t launch_rmsnorm_backward(const uint16_t* x, const uint16_t* gamma, const float* rstd,
                                   const uint16_t* dy, int64_t M, int64_t K, uint16_t* dx,
                                   float* dgamma, float* workspace, hipStream_t stream) {
  if (K == 0) return hipSuccess;
  const int64_t nparts = rmsnorm_backward_parts(M);
  if (M > 0) {
    switch ((K + 511) / 512) {
      case 1: launch_bwd_rows<1>(x, gamma, rstd, dy, M, K, dx, workspace, stream); break;
      case 2: launch_bwd_rows<2>(x, gamma, rstd, dy, M, K, dx, workspace, stream); break;
      case 3: launch_bwd_rows<3>(x, gamma, rstd, dy, M, K, dx, workspace, stream); break;
      case 4: launch_bwd_rows<4>(x, gamma, rstd, dy, M, K, dx, workspace, stream); break;
      case 5: launch_bwd_rows<5>(x, gamma, rstd, dy, M, K, dx, workspace, stream); break;
      case 6: launch_bwd_rows<6>(x, gamma, rstd, dy, M, K, dx, workspace, stream); break;
      case 7: launch_bwd_rows<7>(x, gamma, rstd, dy, M, K, dx, workspace, stream); break;
      case 8: launch_bwd_rows<8>(x, gamma, rstd, dy, M, K, dx, workspace, stream); break;
      case 9: launch_bwd_rows<9>(x, gamma, rstd, dy, M, K, dx, workspace, stream); break;
      case 10: launch_bwd_rows<10>(x, gamma, rstd, dy, M, K, dx, workspace, stream); break;
      case 11: launch_bwd_rows<11>(x, gamma, rstd, dy, M, K, dx, workspace, stream); break;
      default: launch_bwd_rows<kBwdMaxPasses>(x, gamma, rstd, dy, M, K, dx, workspace, stream); break;
    }
  }
  hipLaunchKernelGGL(rmsnorm_dgamma_reduce_kernel, dim3((unsigned)((K + 63) / 64)), dim3(256), 0, stream,
                     workspace, nparts, K, dgamma);
  return hipGetLastError();
}

}  // namespace jetfp8
