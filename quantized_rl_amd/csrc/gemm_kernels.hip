// Block-scaled FP8 GEMMs of the FP8 linear layer for gfx950.
//
//   FProp  Y  = X W^T   (1x128) x (128x128)
//   DGrad  dX = dY W    (1x128) x (128x128), weight blocks used transposed
//   WGrad  dW = dY^T X  (1x128) x (128x1), both operands from the 128x1 requantiser
//
// (Jet-RL pages, paper.rainbus.top summary, sections "GEMM 量化布局", "核心方法",
// "方法步骤详情" steps 2 and 4.)
//
// All three are one kernel template computing
//   C[i][j] = sum_kb  sa[kb][i] * sb(kb, j) * P_kb[i][j],
//   P_kb[i][j] = sum_{k in block kb} A[i][k] * Bop[k][j]       (exact FP8 products, fp32 sum)
// where A is [rows][Kc] with the contraction contiguous, and Bop is either
// B[cols][Kc] (contraction contiguous; FProp, WGrad) or B[Kc][cols] (DGrad: the
// weight as stored, transposed while reading LDS).  sb(kb, j) is a per-block
// scalar (FProp, DGrad) or a per-column value (WGrad).
//
// Each 128-deep block product P_kb of a 16x16 sub-tile is exactly one
// v_mfma_f32_16x16x128_f8f6f4 with a zero accumulator; the fp32 partial is
// multiplied by the product of the two scales and added to the running fp32
// accumulator in registers (one FMA per output element per K-block).
#include "device_common.hpp"
#include "launch.hpp"

namespace jetfp8 {

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v4f_t __attribute__((ext_vector_type(4)));
typedef int v2i_t __attribute__((ext_vector_type(2)));

enum GemmMode { kFprop = 0, kDgrad = 1, kWgrad = 2 };

constexpr int kBM = 128, kBN = 128, kBK = 128;
constexpr int kThreads = 256;
constexpr int kTileBytes = kBM * kBK;  // 16 KB per operand tile

// 16-byte chunk c of tile row r is stored at chunk position c ^ swz(r).
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int lds_off(int r, int c) { return r * 128 + ((c ^ swz(r)) << 4); }

__device__ __forceinline__ v2i_t lds_tr8(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (__attribute__((address_space(3))) v2i_t*)((__attribute__((address_space(3))) uint8_t*)(p)));
}

__device__ __forceinline__ v4f_t mfma_fp8(const v8i_t& a, const v8i_t& b) {
  const v4f_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
  // cbsz = blgp = 0: both operands OCP E4M3; zero scale operands select the
  // unscaled instruction.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

template <int kMode>
__global__ __launch_bounds__(kThreads, 2) void gemm_fp8_kernel(const uint8_t* __restrict__ A,
                                                               const float* __restrict__ sa,
                                                               const uint8_t* __restrict__ B,
                                                               const float* __restrict__ sb,
                                                               int64_t Mr, int64_t Nc, int64_t Kc,
                                                               uint16_t* __restrict__ C) {
  __shared__ __attribute__((aligned(16))) uint8_t As[2][kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t Bs[2][kTileBytes];
  __shared__ __attribute__((aligned(16))) float sas[2][kBM];
  __shared__ __attribute__((aligned(16))) float sbs[2][kBN];

  const int t = threadIdx.x, l = t & 63, w = t >> 6;
  const int wm = w >> 1, wn = w & 1;        // wave's 64x64 quadrant
  const int64_t row0 = (int64_t)blockIdx.y * kBM;
  const int64_t col0 = (int64_t)blockIdx.x * kBN;
  const int64_t nkb = Kc / kBK;

  // global -> register staging: four 16-byte chunks of A and of B per thread
  uint4 ra[4], rb[4];
  float rsa = 0.0f, rsb = 0.0f;

  auto load_tile = [&](int64_t kb) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int id = t + kThreads * p, r = id >> 3, c = id & 7;
      int64_t gr = row0 + r;
      gr = gr < Mr ? gr : Mr - 1;  // ragged last row tile: clamp, results are not stored
      ra[p] = *reinterpret_cast<const uint4*>(A + gr * Kc + kb * kBK + c * 16);
      if (kMode == kDgrad) {
        rb[p] = *reinterpret_cast<const uint4*>(B + (kb * kBK + r) * Nc + col0 + c * 16);
      } else {
        rb[p] = *reinterpret_cast<const uint4*>(B + (col0 + r) * Kc + kb * kBK + c * 16);
      }
    }
    if (t < kBM) {
      int64_t gr = row0 + t;
      gr = gr < Mr ? gr : Mr - 1;
      rsa = sa[kb * Mr + gr];
    } else if (kMode == kWgrad) {
      rsb = sb[kb * Nc + col0 + (t - kBM)];
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int id = t + kThreads * p, r = id >> 3, c = id & 7;
      *reinterpret_cast<uint4*>(&As[buf][lds_off(r, c)]) = ra[p];
      *reinterpret_cast<uint4*>(&Bs[buf][lds_off(r, c)]) = rb[p];
    }
    if (t < kBM) sas[buf][t] = rsa;
    else if (kMode == kWgrad) sbs[buf][t - kBM] = rsb;
  };

  v4f_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f_t{0.0f, 0.0f, 0.0f, 0.0f};

  load_tile(0);
  store_tile(0);
  __syncthreads();

  const int lr = l & 15;   // row (A) / column (B) inside a 16x16 sub-tile
  const int lk = l >> 4;   // which 32-byte slice of the 128-deep block
  for (int64_t kb = 0; kb < nkb; ++kb) {
    const int cur = (int)(kb & 1);
    if (kb + 1 < nkb) load_tile(kb + 1);

    // operand fragments
    v8i_t af[4], bf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wm * 64 + 16 * i + lr;
      const uint4 x0 = *reinterpret_cast<const uint4*>(&As[cur][lds_off(r, 2 * lk)]);
      const uint4 x1 = *reinterpret_cast<const uint4*>(&As[cur][lds_off(r, 2 * lk + 1)]);
      af[i] = v8i_t{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                    (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (kMode == kDgrad) {
        // LDS holds B[n][c] (n = contraction).  Lane (lr) supplies the address of
        // contraction row 32 lk + 8 q + (lr >> 1), bytes 8 (lr & 1) of the
        // sub-tile's 16 columns; it receives column lr of those 8 rows.
        const int chunk = 4 * wn + j;
        v2i_t part[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int n = 32 * lk + 8 * q4 + (lr >> 1);
          part[q4] = lds_tr8(&Bs[cur][lds_off(n, chunk) + 8 * (lr & 1)]);
        }
        bf[j] = v8i_t{part[0].x, part[0].y, part[1].x, part[1].y,
                      part[2].x, part[2].y, part[3].x, part[3].y};
      } else {
        const int r = wn * 64 + 16 * j + lr;
        const uint4 x0 = *reinterpret_cast<const uint4*>(&Bs[cur][lds_off(r, 2 * lk)]);
        const uint4 x1 = *reinterpret_cast<const uint4*>(&Bs[cur][lds_off(r, 2 * lk + 1)]);
        bf[j] = v8i_t{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                      (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
      }
    }

    // scales: this lane's output rows are wm*64 + 16 i + 4 lk + e, column wn*64 + 16 j + lr
    float sarow[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 s4 = *reinterpret_cast<const float4*>(&sas[cur][wm * 64 + 16 * i + 4 * lk]);
      sarow[i][0] = s4.x; sarow[i][1] = s4.y; sarow[i][2] = s4.z; sarow[i][3] = s4.w;
    }
    if (kMode == kWgrad) {
      float sbcol[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) sbcol[j] = sbs[cur][wn * 64 + 16 * j + lr];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const v4f_t p = mfma_fp8(af[i], bf[j]);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][j][e] = fmaf(p[e], sarow[i][e] * sbcol[j], acc[i][j][e]);
        }
    } else {
      const float sblk = (kMode == kFprop) ? sb[(col0 / kBN) * nkb + kb]
                                           : sb[kb * (Nc / kBN) + col0 / kBN];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) sarow[i][e] *= sblk;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const v4f_t p = mfma_fp8(af[i], bf[j]);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][j][e] = fmaf(p[e], sarow[i][e], acc[i][j][e]);
        }
    }

    if (kb + 1 < nkb) store_tile(cur ^ 1);
    __syncthreads();
  }

  // epilogue: fp32 -> bf16 (nearest even), masked on ragged rows
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t gr = row0 + wm * 64 + 16 * i + 4 * lk + e;
      if (gr < Mr) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t gc = col0 + wn * 64 + 16 * j + lr;
          C[gr * Nc + gc] = (uint16_t)f32_to_bf16_rne(acc[i][j][e]);
        }
      }
    }
}

__global__ void fill_zero_u16(uint16_t* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

static hipError_t launch_zero(uint16_t* p, int64_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(fill_zero_u16, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

template <int kMode>
static hipError_t launch_gemm(const uint8_t* A, const float* sa, const uint8_t* B, const float* sb,
                              int64_t Mr, int64_t Nc, int64_t Kc, uint16_t* C,
                              hipStream_t stream) {
  if (Mr == 0 || Nc == 0) return hipSuccess;
  if (Kc == 0) return launch_zero(C, Mr * Nc, stream);
  dim3 grid((unsigned)(Nc / kBN), (unsigned)((Mr + kBM - 1) / kBM));
  hipLaunchKernelGGL(gemm_fp8_kernel<kMode>, grid, dim3(kThreads), 0, stream, A, sa, B, sb, Mr, Nc,
                     Kc, C);
  return hipGetLastError();
}

hipError_t launch_gemm_fprop(const uint8_t* qx, const float* sx, const uint8_t* qw, const float* sw,
                             int64_t M, int64_t N, int64_t K, uint16_t* y, hipStream_t stream) {
  return launch_gemm<kFprop>(qx, sx, qw, sw, M, N, K, y, stream);
}

hipError_t launch_gemm_dgrad(const uint8_t* qdy, const float* sdy, const uint8_t* qw,
                             const float* sw, int64_t M, int64_t N, int64_t K, uint16_t* dx,
                             hipStream_t stream) {
  // contraction over N; output columns are the K input features
  return launch_gemm<kDgrad>(qdy, sdy, qw, sw, M, K, N, dx, stream);
}

hipError_t launch_gemm_wgrad(const uint8_t* qdyt, const float* sdyt, const uint8_t* qxt,
                             const float* sxt, int64_t M, int64_t N, int64_t K, uint16_t* dw,
                             hipStream_t stream) {
  // rows are the N output features, columns the K input features, contraction over M tokens
  return launch_gemm<kWgrad>(qdyt, sdyt, qxt, sxt, N, K, M, dw, stream);
}

}  // namespace jetfp8
