// SwiGLU + 1x128 quantisation of the down projection's input for gfx950.
//
//   y = [gate | up]  bf16 [M][2I]  (the gate+up projection's output)
//   h[m][i] = fl32(silu(gate[m][i]) * up[m][i])
//   silu(g) = fl32(g / fl32(1 + E)),  E = the fp32 value nearest to e^-g
//   (q, s)  = the 1x128 quantisation of h, exactly as quantize_act_1x128 does
//             for fp32 values (no bf16 rounding of h)
//
// The pages fuse the quantisation into the neighbouring kernels (Jet-RL pages,
// paper.rainbus.top summary, section "核心方法"); SiLU, its exponential and the
// gate/up layout are readings (the pages print no formula for them).
//
// HBM-bound: 4 bytes in, 1 + 4/128 out per output element.  silu depends only
// on the 16 bits of the bf16 gate: it is looked up (silu_lookup.hpp) in a
// 32 KB table that each workgroup copies into LDS, with closed forms outside
// the table's range.  No fp64 exponential runs in the kernel, which would make
// it ALU-bound.
//
// Workgroups of 256 threads, two per CU, walk tiles of 32 rows x 4 groups (512
// outputs; 4 or 8 rows for rollout batches); a lane holds 8 consecutive outputs
// of a group (quarter-wave = group) in 8 rows (1 or 2).  The loop is software-pipelined over two register buffers:
// the next tile's 16 loads per lane are in flight while the current tile is
// computed and stored.
#include "device_common.hpp"
#include "launch.hpp"
#include "silu_lookup.hpp"

namespace jetfp8 {

constexpr int kSwThreads = 256;

__device__ const uint32_t kSiluBits[kSiluTable] __attribute__((aligned(16))) = {
#include "silu_table.inc"
};

// kRows rows per tile (32 for training batches, fewer for rollout batches, so
// that their few rows still spread over many workgroups); kIters rows per wave
template <int kRows>
struct SwTile {
  static constexpr int kIters = kRows / (kSwThreads / 64);
  uint4 gv[kIters], uv[kIters];
};

template <int kRows>
struct SwGeom {
  static constexpr int kIters = SwTile<kRows>::kIters;
  const uint16_t* y;
  int64_t M, I, ctiles;
  int l, lane16, wave;
  __device__ __forceinline__ void at(int64_t tile, int64_t& g, bool& g_ok, int64_t& col, int64_t& row0) const {
    g = (tile % ctiles) * 4 + (l >> 4);
    g_ok = g * kGroup < I;  // ragged last column tile (I % 512 != 0)
    col = g * kGroup + lane16 * 8;
    row0 = (tile / ctiles) * kRows + wave;
  }
  __device__ __forceinline__ void load(int64_t tile, SwTile<kRows>& b) const {
    int64_t g, col, row0;
    bool g_ok;
    at(tile, g, g_ok, col, row0);
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
      const int64_t r = row0 + (kSwThreads / 64) * it;
      const bool ok = r < M && g_ok;
      b.gv[it] = ok ? ld_stream16(y + r * 2 * I + col) : make_uint4(0, 0, 0, 0);
      b.uv[it] = ok ? ld_stream16(y + r * 2 * I + I + col) : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void compute(int64_t tile, const SwTile<kRows>& b, const float* tab, uint8_t* q,
                                          float* s) const {
    int64_t g, col, row0;
    bool g_ok;
    at(tile, g, g_ok, col, row0);
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
      const int64_t r = row0 + (kSwThreads / 64) * it;
      float u[8], h[8];
      unpack_bf16x8(b.uv[it], u);
      const uint32_t gw[4] = {b.gv[it].x, b.gv[it].y, b.gv[it].z, b.gv[it].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        h[2 * j] = silu_of_bits(gw[j] & 0xFFFFu, tab) * u[2 * j];
        h[2 * j + 1] = silu_of_bits(gw[j] >> 16, tab) * u[2 * j + 1];
      }
      const float amax = quarter_wave_max(absmax8(h));
      const float sc = scale_from_amax(amax);
      const double inv = inv_scale(sc);
      const uint2 codes = quant8(h, inv);
      if (r < M && g_ok) {
        st_global8(q + r * I + col, codes);
        if (lane16 == 0) s[g * M + r] = sc;
      }
    }
  }
};

template <int kRows>
__global__ __launch_bounds__(kSwThreads) void swiglu_quant_kernel(const uint16_t* __restrict__ y, int64_t M,
                                                                  int64_t I, uint8_t* __restrict__ q,
                                                                  float* __restrict__ s, int64_t tiles) {
  __shared__ __attribute__((aligned(16))) float tab[kSiluTable];
  SwGeom<kRows> geo;
  geo.y = y; geo.M = M; geo.I = I;
  geo.ctiles = (I / kGroup + 3) / 4;
  geo.l = threadIdx.x & 63; geo.lane16 = geo.l & 15; geo.wave = threadIdx.x >> 6;
  const int64_t stride = gridDim.x;
  int64_t tile = blockIdx.x;
  SwTile<kRows> b0, b1;
  geo.load(tile, b0);  // the first tile's loads go out before the table copy
#pragma unroll
  for (int i = 0; i < kSiluTable / (4 * kSwThreads); ++i) {
    const int e = 4 * (threadIdx.x + kSwThreads * i);
    *reinterpret_cast<uint4*>(&tab[e]) = *reinterpret_cast<const uint4*>(&kSiluBits[e]);
  }
  __syncthreads();
  for (;;) {
    if (tile + stride < tiles) geo.load(tile + stride, b1);
    geo.compute(tile, b0, tab, q, s);
    tile += stride;
    if (tile >= tiles) break;
    if (tile + stride < tiles) geo.load(tile + stride, b0);
    geo.compute(tile, b1, tab, q, s);
    tile += stride;
    if (tile >= tiles) break;
  }
}

hipError_t launch_swiglu_quant(const uint16_t* y, int64_t M, int64_t I, uint8_t* q, float* s,
                               hipStream_t stream) {
  if (M == 0 || I == 0) return hipSuccess;
  // rows per tile: rollout batches spread over more workgroups (each copies the
  // 32 KB table once): measured at I = 12288, M = 16 / 64 / 128 / 256: 7.3 / 8.0
  // / 8.2 / 9.0 us with 32-row tiles, 3.2 / 3.7 / 4.5 us with 4 rows, 6.3 us with
  // 8 at M = 256; training batches (8192, 16384 rows) are fastest with 32
  const int rows = M <= 128 ? 4 : (M <= 512 ? 8 : 32);
  const int64_t tiles = ((I / kGroup + 3) / 4) * ((M + rows - 1) / rows);
  int64_t grid = 2 * (int64_t)device_cu_count();
  if (grid <= 0) grid = 512;
  if (grid > tiles) grid = tiles;
  if (rows == 4)
    hipLaunchKernelGGL(swiglu_quant_kernel<4>, dim3((unsigned)grid), dim3(kSwThreads), 0, stream, y, M, I, q, s,
                       tiles);
  else if (rows == 8)
    hipLaunchKernelGGL(swiglu_quant_kernel<8>, dim3((unsigned)grid), dim3(kSwThreads), 0, stream, y, M, I, q, s,
                       tiles);
  else
    hipLaunchKernelGGL(swiglu_quant_kernel<32>, dim3((unsigned)grid), dim3(kSwThreads), 0, stream, y, M, I, q, s,
                       tiles);
  return hipGetLastError();
}

}  // namespace jetfp8
