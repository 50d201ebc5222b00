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
//   rmsnorm_backward_rows_kernel: a workgroup of W waves (4 up to K = 6144,
//     8 up to 12288, 16 up to 24576) owns R consecutive rows (R = 2 ceil(M /
//     512) clamped to 1..32) and walks them one at a time, all its waves on the
//     same row: wave w covers the 512-element passes w, w + W, ... (lane l: the
//     8 elements at 512 p + 8 l), so a lane holds at most three passes of the
//     row and the next row's loads are issued before the current row is
//     finished.  S is each wave's lane-sequential sum and butterfly, the W wave
//     sums added in wave order through LDS.  A wave
//     keeps its columns' dgamma terms in registers, summed in row order, and
//     writes them as its part of the workgroup's partial row of dgamma.
//   rmsnorm_dgamma_reduce_kernel: dgamma_k = the partials summed in a fixed
//     order (four quarters in sequence, then ((q0 + q1) + q2) + q3).
// Identical inputs give identical bits; no atomics.
#include "device_common.hpp"
#include "launch.hpp"

namespace jetfp8 {

// Rows per workgroup: 2 ceil(M / 512) clamped to 1..32 (measured best of
// 1..8, 1..16 and 1..32 at M = 256 .. 16384).
static int64_t bwd_rows_per_group(int64_t M) {
  const int64_t r = 2 * ((M + 511) / 512);
  return r < 1 ? 1 : (r > 32 ? 32 : r);
}

int64_t rmsnorm_backward_parts(int64_t M) {
  const int64_t rows = bwd_rows_per_group(M);
  return (M + rows - 1) / rows;
}

__device__ __forceinline__ uint4 pack_bf16x8(const float (&f)[8]) {
  return make_uint4(f32_to_bf16_rne(f[0]) | (f32_to_bf16_rne(f[1]) << 16),
                    f32_to_bf16_rne(f[2]) | (f32_to_bf16_rne(f[3]) << 16),
                    f32_to_bf16_rne(f[4]) | (f32_to_bf16_rne(f[5]) << 16),
                    f32_to_bf16_rne(f[6]) | (f32_to_bf16_rne(f[7]) << 16));
}

// kQ: passes per wave (ceil(ceil(K / 512) / kW)); kW: waves per workgroup.
template <int kQ, int kW>
__global__ __launch_bounds__(64 * kW) void rmsnorm_backward_rows_kernel(const uint16_t* __restrict__ x,
                                                                    const uint16_t* __restrict__ gamma,
                                                                    const float* __restrict__ rstd,
                                                                    const uint16_t* __restrict__ dy,
                                                                    int64_t M, int64_t K, int rows_per_group,
                                                                    uint16_t* __restrict__ dx,
                                                                    float* __restrict__ part) {
  __shared__ float wsum[2][kW];
  const int t = threadIdx.x, l = t & 63, w = t >> 6;
  const int64_t row0 = (int64_t)blockIdx.x * rows_per_group;
  const int64_t rows = (M - row0) < rows_per_group ? (M - row0) : rows_per_group;

  // this lane's element offsets and whether they exist
  int64_t e[kQ];
  bool in[kQ];
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    e[q] = 512 * (int64_t)(w + kW * q) + 8 * l;
    in[q] = e[q] < K;
  }
  float fg[kQ][8], u[kQ][8];
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    unpack_bf16x8(in[q] ? *reinterpret_cast<const uint4*>(gamma + e[q]) : make_uint4(0, 0, 0, 0), fg[q]);
#pragma unroll
    for (int i = 0; i < 8; ++i) u[q][i] = 0.0f;
  }
  auto load_row = [&](int64_t row, uint4 (&xv)[kQ], uint4 (&dv)[kQ]) {
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      xv[q] = in[q] ? ld_stream16(x + row * K + e[q]) : make_uint4(0, 0, 0, 0);
      dv[q] = in[q] ? ld_stream16(dy + row * K + e[q]) : make_uint4(0, 0, 0, 0);
    }
  };
  uint4 xv[kQ], dv[kQ];
  load_row(row0, xv, dv);
  for (int64_t r = 0; r < rows; ++r) {
    const int64_t row = row0 + r;
    const float rr = rstd[row];
    float fx[kQ][8], fd[kQ][8];
    float sl = 0.0f;
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      unpack_bf16x8(xv[q], fx[q]);
      unpack_bf16x8(dv[q], fd[q]);
#pragma unroll
      for (int i = 0; i < 8; ++i) sl = sl + (fg[q][i] * fd[q][i]) * fx[q][i];
    }
    // the next row's loads go out before this row's reduction and stores
    if (r + 1 < rows) load_row(row + 1, xv, dv);
    const float ws = wave_sum_tree(sl);
    if (l == 0) wsum[r & 1][w] = ws;
    __syncthreads();
    float ssum = wsum[r & 1][0];
#pragma unroll
    for (int v = 1; v < kW; ++v) ssum = ssum + wsum[r & 1][v];
    const float c = ssum / (float)K;
    const float rc = (rr * rr) * c;
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      float o[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        o[i] = rr * ((fg[q][i] * fd[q][i]) - fx[q][i] * rc);
        u[q][i] = u[q][i] + (fd[q][i] * fx[q][i]) * rr;
      }
      if (in[q]) *reinterpret_cast<uint4*>(dx + row * K + e[q]) = pack_bf16x8(o);
    }
  }
  // this wave's columns of the workgroup's partial row of dgamma
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    if (in[q]) {
      float* pp = part + (int64_t)blockIdx.x * K + e[q];
      *reinterpret_cast<float4*>(pp) = make_float4(u[q][0], u[q][1], u[q][2], u[q][3]);
      *reinterpret_cast<float4*>(pp + 4) = make_float4(u[q][4], u[q][5], u[q][6], u[q][7]);
    }
  }
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

template <int kQ, int kW>
static void launch_bwd_rows(const uint16_t* x, const uint16_t* gamma, const float* rstd, const uint16_t* dy,
                            int64_t M, int64_t K, uint16_t* dx, float* part, hipStream_t stream) {
  hipLaunchKernelGGL((rmsnorm_backward_rows_kernel<kQ, kW>), dim3((unsigned)rmsnorm_backward_parts(M)),
                     dim3(64 * kW), 0, stream, x, gamma, rstd, dy, M, K, (int)bwd_rows_per_group(M), dx, part);
}

template <int kW>
static void launch_bwd_rows_w(const uint16_t* x, const uint16_t* gamma, const float* rstd, const uint16_t* dy,
                              int64_t M, int64_t K, uint16_t* dx, float* part, hipStream_t stream) {
  const int64_t passes = (K + 511) / 512;
  switch ((passes + kW - 1) / kW) {
    case 1: launch_bwd_rows<1, kW>(x, gamma, rstd, dy, M, K, dx, part, stream); break;
    case 2: launch_bwd_rows<2, kW>(x, gamma, rstd, dy, M, K, dx, part, stream); break;
    default: launch_bwd_rows<3, kW>(x, gamma, rstd, dy, M, K, dx, part, stream); break;
  }
}

hipError_t launch_rmsnorm_backward(const uint16_t* x, const uint16_t* gamma, const float* rstd,
                                   const uint16_t* dy, int64_t M, int64_t K, uint16_t* dx,
                                   float* dgamma, float* workspace, hipStream_t stream) {
  if (K == 0) return hipSuccess;
  const int64_t nparts = rmsnorm_backward_parts(M);
  if (M > 0) {
    const int64_t passes = (K + 511) / 512;  // at most 48: the API takes K <= 24576
    if (passes <= 12)
      launch_bwd_rows_w<4>(x, gamma, rstd, dy, M, K, dx, workspace, stream);
    else if (passes <= 24)
      launch_bwd_rows_w<8>(x, gamma, rstd, dy, M, K, dx, workspace, stream);
    else
      launch_bwd_rows_w<16>(x, gamma, rstd, dy, M, K, dx, workspace, stream);
  }
  hipLaunchKernelGGL(rmsnorm_dgamma_reduce_kernel, dim3((unsigned)((K + 63) / 64)), dim3(256), 0, stream,
                     workspace, nparts, K, dgamma);
  return hipGetLastError();
}

}  // namespace jetfp8
