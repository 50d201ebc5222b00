// Quantisation kernels of the FP8 linear layer for gfx950 (HBM-bound).
//
//   quantize_act_1x128       1x128 per-group E4M3 quantisation (activations, gradients)
//   quantize_weight_128x128  128x128 per-block E4M3 quantisation (weights)
//   rmsnorm_quant            fused RMSNorm + 1x128 quantisation (optionally saving the
//                            per-row factor rstd for the backward)
//   requant_transpose_128x1  saved 1x128 FP8 -> 128x1 groups along tokens, stored transposed
//
// Definitions: Jet-RL pages, paper.rainbus.top summary, sections
// "FP8 量化 (E4M3 格式)", "Per-group / Per-block 量化粒度" and "方法步骤详情"
// (steps 1-5).  Every quantiser output is a bit-exact function of its input.
#include "device_common.hpp"
#include "launch.hpp"

namespace jetfp8 {

// ---------------------------------------------------------------------------
// 1x128 activation / gradient quantisation.
//
// A workgroup of 256 threads owns a tile of kActRows rows x 4 groups (512
// columns).  Every load instruction of a wave reads 1 KB of one row (lane l:
// bytes 16 l ..), so quarter-wave q holds group 4 c + q of that row; wave w
// takes rows w, w + 4, ..  Each lane issues all of its loads before any
// arithmetic.  The launch walks the column tiles of a row band fastest, so
// the workgroups in flight stream contiguous memory, and the scales of the
// tile's 32 rows of one group fill a 128-byte line of S[g][*].
constexpr int kActRows = 32;
constexpr int kActIters = kActRows / 4;

__global__ __launch_bounds__(256) void quant_act_1x128_kernel(const uint16_t* __restrict__ x,
                                                              int64_t M, int64_t K,
                                                              uint8_t* __restrict__ q,
                                                              float* __restrict__ s) {
  const int l = threadIdx.x & 63, lane16 = l & 15;
  const int wave = threadIdx.x >> 6;
  const int64_t ctiles = (K / kGroup + 3) / 4;
  const int64_t g = (int64_t)(blockIdx.x % ctiles) * 4 + (l >> 4);
  const bool g_ok = g * kGroup < K;  // ragged last column tile (K % 512 != 0)
  const int64_t col = g * kGroup + lane16 * 8;
  const int64_t row0 = (int64_t)(blockIdx.x / ctiles) * kActRows + wave;

  uint4 v[kActIters];
#pragma unroll
  for (int it = 0; it < kActIters; ++it) {
    const int64_t r = row0 + 4 * it;
    v[it] = (r < M && g_ok) ? ld_stream16(x + r * K + col) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int it = 0; it < kActIters; ++it) {
    const int64_t r = row0 + 4 * it;
    float f[8];
    unpack_bf16x8(v[it], f);
    const float amax = quarter_wave_max(absmax8(f));
    const float sc = scale_from_amax(amax);
    const double inv = inv_scale(sc);
    const uint2 codes = quant8(f, inv);
    if (r < M && g_ok) {
      st_global8(q + r * K + col, codes);
      if (lane16 == 0) s[g * M + r] = sc;
    }
  }
}

// ---------------------------------------------------------------------------
// 128x128 weight quantisation: one workgroup per block.  Each thread keeps its
// 64 elements (eight 16-byte loads) in registers across the block-wide amax.
__global__ __launch_bounds__(256) void quant_weight_128x128_kernel(const uint16_t* __restrict__ w,
                                                                   int64_t N, int64_t K,
                                                                   uint8_t* __restrict__ q,
                                                                   float* __restrict__ s) {
  __shared__ float wave_amax[4];
  const int lane16 = threadIdx.x & 15;
  const int rsub = threadIdx.x >> 4;  // 0..15
  const int64_t kb = blockIdx.x, nb = blockIdx.y;
  const uint16_t* base = w + (nb * kGroup) * K + kb * kGroup + lane16 * 8;

  uint4 v[8];
#pragma unroll
  for (int it = 0; it < 8; ++it)
    v[it] = ld_stream16(base + (int64_t)(rsub + 16 * it) * K);
  float amax = 0.0f;
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    float f[8];
    unpack_bf16x8(v[it], f);
    amax = fmaxf(amax, absmax8(f));
  }
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) wave_amax[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wave_amax[0], wave_amax[1]), fmaxf(wave_amax[2], wave_amax[3]));
  const float sc = scale_from_amax(amax);
  const double inv = inv_scale(sc);
  uint8_t* qbase = q + (nb * kGroup) * K + kb * kGroup + lane16 * 8;
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    float f[8];
    unpack_bf16x8(v[it], f);
    st_global8(qbase + (int64_t)(rsub + 16 * it) * K, quant8(f, inv));
  }
  if (threadIdx.x == 0) s[nb * (K / kGroup) + kb] = sc;
}

// ---------------------------------------------------------------------------
// Fused RMSNorm + 1x128 quantisation: one workgroup (256 threads) per row.
//
// The sum of squares follows the pairwise tree over the row zero-padded to a
// power of two.  Pass j covers elements [2048 j, 2048 j + 2048): thread t owns
// the 8 contiguous elements starting at 2048 j + 8 t and sums them as a
// balanced tree; a xor-butterfly over the wave (offsets 1..32) builds the
// 512-element subtrees, and the four wave sums are combined as (w0+w1)+(w2+w3).
// The per-pass sums are then combined by the same pairwise rule.  Every
// partial is a node of the canonical tree, so the fp32 result is exactly the
// oracle's.  Then each quarter-wave quantises 128-element groups.
constexpr int kNormPass = 2048;
constexpr int kNormMaxPasses = 32;  // K <= 65536

__device__ __forceinline__ float tree8_sq(const float (&f)[8]) {
  const float a = f[0] * f[0] + f[1] * f[1];  // contraction is disabled for this file
  const float b = f[2] * f[2] + f[3] * f[3];
  const float c = f[4] * f[4] + f[5] * f[5];
  const float d = f[6] * f[6] + f[7] * f[7];
  return (a + b) + (c + d);
}

// Rows of up to 8192 elements: one wave per row, the row held in registers.
// Pass p covers elements [512 p, 512 p + 512): lane l owns the 8 elements at
// 512 p + 8 l, summed as a balanced tree, then a xor-butterfly over the wave
// (offsets 1..32) gives the pass's 512-element subtree; the pass sums are
// combined by the pairwise rule (odd tail carried).  Each partial is a node of
// the canonical tree of the row zero-padded to a power of two.  kP (passes) is
// a template parameter so that all loads -- the row and gamma -- are issued
// unconditionally up front; only the last pass can be partial.
constexpr int kRowPasses = 16;  // K <= 8192

template <int kP>
__global__ __launch_bounds__(256) void rmsnorm_quant_rows_kernel(const uint16_t* __restrict__ x,
                                                                 const uint16_t* __restrict__ gamma,
                                                                 int64_t M, int64_t K, float eps,
                                                                 uint8_t* __restrict__ q,
                                                                 float* __restrict__ s,
                                                                 float* __restrict__ rstd) {
  const int l = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;  // whole waves only
  const uint16_t* xr = x + row * K;

  uint4 xv[kP], gv[kP];
#pragma unroll
  for (int p = 0; p < kP; ++p) {
    const int64_t e = 512 * p + 8 * l;
    const bool in = p < kP - 1 || e < K;
    xv[p] = in ? ld_stream16(xr + e) : make_uint4(0, 0, 0, 0);
    gv[p] = in ? *reinterpret_cast<const uint4*>(gamma + e) : make_uint4(0, 0, 0, 0);
  }
  float ps[kP];
#pragma unroll
  for (int p = 0; p < kP; ++p) {
    float f[8];
    unpack_bf16x8(xv[p], f);
    float v = tree8_sq(f);
    v = wave_sum_tree(v);
    ps[p] = v;
  }
  // pairwise tree over the pass sums (all lanes hold the same values)
#pragma unroll
  for (int n = kP; n > 1; n = n / 2 + (n & 1)) {
    const int h = n / 2;
#pragma unroll
    for (int j = 0; j < h; ++j) ps[j] = ps[2 * j] + ps[2 * j + 1];
    if (n & 1) ps[h] = ps[n - 1];
  }
  const float ms = ps[0] / (float)K;
  const float inv = recip_f32_rn(sqrt_rn(ms + eps));
  if (rstd != nullptr && l == 0) rstd[row] = inv;

  const int lane16 = l & 15, quarter = l >> 4;
#pragma unroll
  for (int p = 0; p < kP; ++p) {
    const int64_t g = 4 * p + quarter;
    if (p < kP - 1 || g * kGroup < K) {
      const int64_t e = g * kGroup + lane16 * 8;
      float f[8], gm[8];
      unpack_bf16x8(xv[p], f);
      unpack_bf16x8(gv[p], gm);
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = (f[i] * inv) * gm[i];
      const float amax = quarter_wave_max(absmax8(f));
      const float sc = scale_from_amax(amax);
      const double dinv = inv_scale(sc);
      st_global8(q + row * K + e, quant8(f, dinv));
      if (lane16 == 0) s[g * M + row] = sc;
    }
  }
}

template <int kP>
static void launch_rows(const uint16_t* x, const uint16_t* gamma, int64_t M, int64_t K, float eps,
                        uint8_t* q, float* s, float* rstd, hipStream_t stream) {
  hipLaunchKernelGGL(rmsnorm_quant_rows_kernel<kP>, dim3((unsigned)((M + 3) / 4)), dim3(256), 0, stream,
                     x, gamma, M, K, eps, q, s, rstd);
}

// Rows of K = 2048 kQ elements (kQ = 1, 2, 4: the 2048-, 4096- and
// 8192-wide models): the four waves of a workgroup share each row, and a
// workgroup walks a strided set of rows (below).  Wave w owns the
// kQ passes kQ w .. kQ w + kQ - 1 of 512 elements (lane l: the 8 elements at
// 512 p + 8 l), so its pass sums combine pairwise into the subtree of its
// 512 kQ elements and the four wave subtrees meet in LDS as (w0 + w1) +
// (w2 + w3): the same canonical tree as the one-wave kernel.  gamma is
// loaded and widened to fp32 once per workgroup, the row's fp32 values are
// kept for the quantisation (one widening per element), and the next row's
// loads are issued before the current row is reduced.
template <int kQ>
__global__ __launch_bounds__(256) void rmsnorm_quant_split_kernel(const uint16_t* __restrict__ x,
                                                                  const uint16_t* __restrict__ gamma,
                                                                  int64_t M, int64_t K, float eps,
                                                                  uint8_t* __restrict__ q,
                                                                  float* __restrict__ s,
                                                                  float* __restrict__ rstd) {
  // K = 2048 kQ is a power of two, so ss / K is exactly ss * (1 / K)
  constexpr float kInvK = 1.0f / (float)(2048 * kQ);
  __shared__ float wsum[2][4];  // per row parity: the four wave subtrees
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int lane16 = l & 15, quarter = l >> 4;
  const int64_t e0 = 512 * kQ * w + 8 * l;  // element of pass j: e0 + 512 j

  float g[kQ][8];
#pragma unroll
  for (int j = 0; j < kQ; ++j) unpack_bf16x8(*reinterpret_cast<const uint4*>(gamma + e0 + 512 * j), g[j]);

  // one row: reduce, normalise, quantise; `nxt` receives the loads of row + stride
  auto do_row = [&](int64_t row, int64_t end, int64_t stride, const uint4 (&cur)[kQ], uint4 (&nxt)[kQ],
                    int par) {
    float f[kQ][8];
#pragma unroll
    for (int j = 0; j < kQ; ++j) unpack_bf16x8(cur[j], f[j]);
    const int64_t next = row + stride;
    if (next < end) {
#pragma unroll
      for (int j = 0; j < kQ; ++j) nxt[j] = ld_stream16(x + next * K + e0 + 512 * j);
    }
    float ps[kQ];
#pragma unroll
    for (int j = 0; j < kQ; ++j) ps[j] = wave_sum_tree(tree8_sq(f[j]));
#pragma unroll
    for (int n = kQ; n > 1; n /= 2)
#pragma unroll
      for (int j = 0; j < n / 2; ++j) ps[j] = ps[2 * j] + ps[2 * j + 1];
    if (l == 0) wsum[par][w] = ps[0];
    __syncthreads();
    const float tot = (wsum[par][0] + wsum[par][1]) + (wsum[par][2] + wsum[par][3]);
    const float inv = recip_f32_rn(sqrt_rn(tot * kInvK + eps));
    if (rstd != nullptr && threadIdx.x == 0) rstd[row] = inv;
#pragma unroll
    for (int j = 0; j < kQ; ++j) {
      float y[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = (f[j][i] * inv) * g[j][i];
      const float amax = quarter_wave_max(absmax8(y));
      const float sc = scale_from_amax(amax);
      st_global8(q + row * K + e0 + 512 * j, quant8(y, inv_scale(sc)));
      const int64_t grp = 4 * (kQ * w + j) + quarter;
      if (lane16 == 0) s[grp * M + row] = sc;
    }
  };

  // Rows of this workgroup: with a grid of 8 g workgroups (dealt to the 8
  // XCDs round-robin), XCD x owns rows [x M / 8, (x + 1) M / 8) and its
  // workgroups walk them with stride g, so the rows in flight on one XCD are
  // consecutive and the 4-byte scale stores of a group fill whole lines in
  // that XCD's L2 (interleaved over the XCDs, each line was written back in
  // pieces from eight caches: 21 % more bytes written).  Other grids: one row
  // per workgroup.
  int64_t row, end, stride;
  if (gridDim.x % 8 == 0 && (int64_t)gridDim.x < M) {
    const int64_t xcd = blockIdx.x % 8;
    row = xcd * M / 8 + blockIdx.x / 8;
    end = (xcd + 1) * M / 8;
    stride = gridDim.x / 8;
  } else {
    row = blockIdx.x;
    end = M;
    stride = gridDim.x;
  }
  if (row >= end) return;  // whole workgroup: no barrier is left waiting
  // rows alternate between two register buffers (no copies between them)
  uint4 xa[kQ], xb[kQ];
#pragma unroll
  for (int j = 0; j < kQ; ++j) xa[j] = ld_stream16(x + row * K + e0 + 512 * j);
  while (true) {
    do_row(row, end, stride, xa, xb, 0);
    row += stride;
    if (row >= end) break;
    do_row(row, end, stride, xb, xa, 1);
    row += stride;
    if (row >= end) break;
  }
}

template <int kQ>
static void launch_split(const uint16_t* x, const uint16_t* gamma, int64_t M, int64_t K, float eps,
                         uint8_t* q, float* s, float* rstd, hipStream_t stream) {
  // about eight workgroups per CU; each walks M / grid rows
  const int64_t grid = M < 2048 ? M : 2048;
  hipLaunchKernelGGL(rmsnorm_quant_split_kernel<kQ>, dim3((unsigned)grid), dim3(256), 0, stream, x, gamma,
                     M, K, eps, q, s, rstd);
}

// Wider rows: one workgroup (256 threads) per row, two passes over the row.
__global__ __launch_bounds__(256) void rmsnorm_quant_kernel(const uint16_t* __restrict__ x,
                                                            const uint16_t* __restrict__ gamma,
                                                            int64_t M, int64_t K, float eps,
                                                            uint8_t* __restrict__ q,
                                                            float* __restrict__ s,
                                                            float* __restrict__ rstd) {
  __shared__ float part[kNormMaxPasses][4];
  __shared__ float inv_sh;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int64_t row = blockIdx.x;
  const uint16_t* xr = x + row * K;
  const int passes = (int)((K + kNormPass - 1) / kNormPass);

  for (int j = 0; j < passes; ++j) {
    const int64_t e = (int64_t)j * kNormPass + 8 * t;
    float v = 0.0f;
    if (e < K) {
      float f[8];
      unpack_bf16x8(*reinterpret_cast<const uint4*>(xr + e), f);
      v = tree8_sq(f);
    }
    v = wave_sum_tree(v);
    if (lane == 0) part[j][wave] = v;
  }
  __syncthreads();
  if (t == 0) {
    float ps[kNormMaxPasses];
    int n = passes;
    for (int j = 0; j < n; ++j) ps[j] = (part[j][0] + part[j][1]) + (part[j][2] + part[j][3]);
    while (n > 1) {  // pairwise tree over the per-pass sums, odd tail carried
      const int h = n / 2;
      for (int j = 0; j < h; ++j) ps[j] = ps[2 * j] + ps[2 * j + 1];
      if (n & 1) ps[h] = ps[n - 1];
      n = h + (n & 1);
    }
    const float ms = ps[0] / (float)K;
    const float d = ms + eps;
    inv_sh = recip_f32_rn(sqrt_rn(d));
    if (rstd != nullptr) rstd[row] = inv_sh;
  }
  __syncthreads();
  const float inv = inv_sh;

  // quantisation: quarter-wave qw handles groups qw, qw + 16, ...
  const int lane16 = t & 15, quarter = t >> 4;
  const int64_t ngroups = K / kGroup;
  for (int64_t g = quarter; g < ngroups; g += 16) {
    const int64_t e = g * kGroup + lane16 * 8;
    float f[8], gm[8];
    unpack_bf16x8(*reinterpret_cast<const uint4*>(xr + e), f);
    unpack_bf16x8(*reinterpret_cast<const uint4*>(gamma + e), gm);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = (f[i] * inv) * gm[i];
    const float amax = quarter_wave_max(absmax8(f));
    const float sc = scale_from_amax(amax);
    const double dinv = inv_scale(sc);
    *reinterpret_cast<uint2*>(q + row * K + e) = quant8(f, dinv);
    if (lane16 == 0) s[g * M + row] = sc;
  }
}

// ---------------------------------------------------------------------------
// Requantisation 1x128 -> 128x1 with transposed store.
//
// A workgroup of 256 threads owns a 128-token x 128-feature tile.  It stages
// the 16 KB of codes and the tile's 128 input scales in LDS; two threads own
// each column k (tokens 0..63 and 64..127).  A thread reads its 64 codes with
// the gfx950 LDS transpose read (ds_read_b64_tr_b8: within each 16-lane
// group, lane i receives byte (i & 7) of the 8-byte rows addressed by lanes
// 2j + (i >> 3), j = 0..7 -- one column of an 8 x 16 byte block) and keeps
// them as codes (16 registers).  Pass 1 decodes them (v_cvt_pk_f32_fp8),
// multiplies by the token scales and takes the column amax; the two halves'
// amax meet in LDS.  Pass 2 recomputes the same fp32 products and writes the
// requantised codes into the same LDS tile, now holding Qt (every read of the
// input tile happens before the barrier between the passes), which the
// workgroup stores with full 128-byte rows.  One 18.4 KB tile and about 40
// registers per thread let eight workgroups share a CU.
constexpr int kRqPitch = 128 + 16;  // LDS row pitch in bytes (16-byte pad)

typedef int v2i_t __attribute__((ext_vector_type(2)));
typedef float v2f_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ v2i_t lds_read_tr8(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (__attribute__((address_space(3))) v2i_t*)((__attribute__((address_space(3))) uint8_t*)(p)));
}

// Four E4M3 codes packed in a dword -> fp32 (exact).
__device__ __forceinline__ void decode4(uint32_t w, float (&v)[4]) {
  const v2f_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const v2f_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  v[0] = lo.x; v[1] = lo.y; v[2] = hi.x; v[3] = hi.y;
}

// The eight dequantised values fl32(decode(code) * s) of one transpose read
// (tokens r0 .. r0 + 7 of the thread's column); the scales come from LDS.
__device__ __forceinline__ void dequant8(v2i_t r, const float* sc, float (&v)[8]) {
  float d[8];
  decode4((uint32_t)r.x, *reinterpret_cast<float(*)[4]>(&d[0]));
  decode4((uint32_t)r.y, *reinterpret_cast<float(*)[4]>(&d[4]));
  const float4 s0 = *reinterpret_cast<const float4*>(sc);
  const float4 s1 = *reinterpret_cast<const float4*>(sc + 4);
  v[0] = d[0] * s0.x; v[1] = d[1] * s0.y; v[2] = d[2] * s0.z; v[3] = d[3] * s0.w;
  v[4] = d[4] * s1.x; v[5] = d[5] * s1.y; v[6] = d[6] * s1.z; v[7] = d[7] * s1.w;
}

__global__ __launch_bounds__(256) void requant_transpose_kernel(const uint8_t* __restrict__ q,
                                                                const float* __restrict__ s,
                                                                int64_t M, int64_t K,
                                                                uint8_t* __restrict__ qt,
                                                                float* __restrict__ st) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[kGroup * kRqPitch];  // [m][k], then [k][m]
  __shared__ __attribute__((aligned(16))) float sc_in[kGroup];
  __shared__ float half_amax[2][kGroup];
  const int t = threadIdx.x;
  // Token blocks run fastest: the workgroups in flight share a few feature
  // groups, so their stores fill long contiguous stretches of each Qt row
  // (the loads still cover whole rows of Q per feature group).  With feature
  // groups fastest, the stores of a 16384-token tensor ran 30 % slower.
  const int64_t mb = blockIdx.x;  // token block (128 rows)
  const int64_t kg = blockIdx.y;  // feature group (128 columns)
  const uint8_t* src = q + (mb * kGroup) * K + kg * kGroup;

  // 128 rows x 8 chunks of 16 bytes = 1024 chunks, 4 per thread
  uint4 c[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int id = t + 256 * it, r = id >> 3, ch = id & 7;
    c[it] = ld_stream16(src + (int64_t)r * K + ch * 16);
  }
  if (t < kGroup) sc_in[t] = s[kg * M + mb * kGroup + t];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int id = t + 256 * it, r = id >> 3, ch = id & 7;
    *reinterpret_cast<uint4*>(tile + r * kRqPitch + ch * 16) = c[it];
  }
  __syncthreads();

  // thread -> (column, half): 16-lane group gi covers columns 16 gi .. + 15
  const int li = t & 15, gi = (t >> 4) & 7, h = t >> 7;
  const int col = 16 * gi + li;
  // address this lane supplies for row block j: row 64 h + 8 j + (li >> 1), bytes 8 (li & 1)
  const uint8_t* abase = tile + (64 * h + (li >> 1)) * kRqPitch + 16 * gi + 8 * (li & 1);
  const float* sch = sc_in + 64 * h;
  v2i_t r[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = lds_read_tr8(abase + 8 * j * kRqPitch);
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float v[8];
    dequant8(r[j], sch + 8 * j, v);
#pragma unroll
    for (int b = 0; b < 8; ++b) amax = fmaxf(amax, fabsf(v[b]));
  }
  half_amax[h][col] = amax;
  __syncthreads();  // also ends every read of the input tile
  // Opaque to the compiler: pass 2 decodes the codes again instead of keeping
  // pass 1's 64 decoded values alive across the barrier.
#pragma unroll
  for (int j = 0; j < 8; ++j) __asm__ volatile("" : "+v"(r[j]));
  amax = fmaxf(half_amax[0][col], half_amax[1][col]);
  const float sc = scale_from_amax(amax);
  const double inv = inv_scale(sc);
#pragma unroll
  for (int i = 0; i < 4; ++i) {  // 16 codes per 16-byte LDS store
    uint32_t o[4];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      float v[8];
      dequant8(r[2 * i + jj], sch + 8 * (2 * i + jj), v);
      const uint2 p = quant8(v, inv);
      o[2 * jj] = p.x;
      o[2 * jj + 1] = p.y;
    }
    *reinterpret_cast<uint4*>(tile + col * kRqPitch + 64 * h + 16 * i) = make_uint4(o[0], o[1], o[2], o[3]);
  }
  if (h == 0) st[mb * K + kg * kGroup + col] = sc;
  __syncthreads();
  // store Qt rows kg*128 + r, tokens mb*128 .. +128: 8 threads per 128-byte row
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int id = t + 256 * it, rr = id >> 3, ch = id & 7;
    st_global16(qt + (kg * kGroup + rr) * M + mb * kGroup + ch * 16,
                *reinterpret_cast<const uint4*>(tile + rr * kRqPitch + ch * 16));
  }
}

// ---------------------------------------------------------------------------
// launchers (shapes validated by the caller)

hipError_t launch_quant_act(const uint16_t* x, int64_t M, int64_t K, uint8_t* q, float* s,
                            hipStream_t stream) {
  if (M == 0 || K == 0) return hipSuccess;
  const int64_t tiles = ((K / kGroup + 3) / 4) * ((M + kActRows - 1) / kActRows);  // < 2^32
  hipLaunchKernelGGL(quant_act_1x128_kernel, dim3((unsigned)tiles), dim3(256), 0, stream, x, M, K, q, s);
  return hipGetLastError();
}

hipError_t launch_quant_weight(const uint16_t* w, int64_t N, int64_t K, uint8_t* q, float* s,
                               hipStream_t stream) {
  if (N == 0 || K == 0) return hipSuccess;
  dim3 grid((unsigned)(K / kGroup), (unsigned)(N / kGroup));
  hipLaunchKernelGGL(quant_weight_128x128_kernel, grid, dim3(256), 0, stream, w, N, K, q, s);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_quant(const uint16_t* x, const uint16_t* gamma, int64_t M, int64_t K,
                                float eps, uint8_t* q, float* s, float* rstd, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  if (K == 2048 || K == 4096 || K == 8192) {
    if (K == 2048) launch_split<1>(x, gamma, M, K, eps, q, s, rstd, stream);
    else if (K == 4096) launch_split<2>(x, gamma, M, K, eps, q, s, rstd, stream);
    else launch_split<4>(x, gamma, M, K, eps, q, s, rstd, stream);
    return hipGetLastError();
  }
  if (K <= 512 * kRowPasses) {
    switch ((K + 511) / 512) {
      case 1: launch_rows<1>(x, gamma, M, K, eps, q, s, rstd, stream); break;
      case 2: launch_rows<2>(x, gamma, M, K, eps, q, s, rstd, stream); break;
      case 3: launch_rows<3>(x, gamma, M, K, eps, q, s, rstd, stream); break;
      case 4: launch_rows<4>(x, gamma, M, K, eps, q, s, rstd, stream); break;
      case 5: launch_rows<5>(x, gamma, M, K, eps, q, s, rstd, stream); break;
      case 6: launch_rows<6>(x, gamma, M, K, eps, q, s, rstd, stream); break;
      case 7: launch_rows<7>(x, gamma, M, K, eps, q, s, rstd, stream); break;
      case 8: launch_rows<8>(x, gamma, M, K, eps, q, s, rstd, stream); break;
      case 9: launch_rows<9>(x, gamma, M, K, eps, q, s, rstd, stream); break;
      case 10: launch_rows<10>(x, gamma, M, K, eps, q, s, rstd, stream); break;
      case 11: launch_rows<11>(x, gamma, M, K, eps, q, s, rstd, stream); break;
      case 12: launch_rows<12>(x, gamma, M, K, eps, q, s, rstd, stream); break;
      case 13: launch_rows<13>(x, gamma, M, K, eps, q, s, rstd, stream); break;
      case 14: launch_rows<14>(x, gamma, M, K, eps, q, s, rstd, stream); break;
      case 15: launch_rows<15>(x, gamma, M, K, eps, q, s, rstd, stream); break;
      default: launch_rows<16>(x, gamma, M, K, eps, q, s, rstd, stream); break;
    }
    return hipGetLastError();
  }
  hipLaunchKernelGGL(rmsnorm_quant_kernel, dim3((unsigned)M), dim3(256), 0, stream, x, gamma, M, K,
                     eps, q, s, rstd);
  return hipGetLastError();
}

hipError_t launch_requant(const uint8_t* q, const float* s, int64_t M, int64_t K, uint8_t* qt,
                          float* st, hipStream_t stream) {
  if (M == 0 || K == 0) return hipSuccess;
  dim3 grid((unsigned)(M / kGroup), (unsigned)(K / kGroup));
  hipLaunchKernelGGL(requant_transpose_kernel, grid, dim3(256), 0, stream, q, s, M, K, qt, st);
  return hipGetLastError();
}

}  // namespace jetfp8
