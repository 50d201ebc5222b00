// Block-scaled FP8 GEMMs of the FP8 linear layer for gfx950.
//
//   FProp  Y  = X W^T   (1x128) x (128x128)
//   DGrad  dX = dY W    (1x128) x (128x128), weight blocks used transposed
//   WGrad  dW = dY^T X  (1x128) x (128x1), both operands from the 128x1 requantiser
//
// (Jet-RL pages, paper.rainbus.top summary, sections "GEMM 量化布局", "核心方法",
// "方法步骤详情" steps 2 and 4.)
//
// Every kernel here computes
//   C[i][j] = sum_kb  sa[kb][i] * sb(kb, j) * P_kb[i][j],
//   P_kb[i][j] = sum_{k in block kb} A[i][k] * Bop[k][j]       (one MFMA result, fp32)
// where A is [rows][Kc] with the contraction contiguous, and Bop is either
// B[cols][Kc] (contraction contiguous; FProp, WGrad) or B[Kc][cols] (DGrad: the
// weight as stored, transposed while reading LDS).  sb(kb, j) is a per-block
// scalar (FProp, DGrad) or a per-column value (WGrad).
//
// Each 128-deep block product P_kb of a 16x16 sub-tile is exactly one
// v_mfma_f32_16x16x128_f8f6f4 with a zero accumulator; the fp32 partial is
// multiplied by the product of the two scales and added to the running fp32
// accumulator in registers (one FMA per output element per K-block).
// P_kb is not the exact sum of its products: the instruction adds each lane's
// 32-product slice with reduced internal precision (products below about 2^-14
// of the slice's largest can be lost), then combines the slices in fp32.  On
// codes of quantised bell-shaped data the resulting error is far inside the
// bf16 tolerance; with arbitrary full-range codes it stays below 2^-9 of the
// output's absolute product sum, which exceeds 1e-3 rms where large products
// cancel (the normwise bound holds).
//
// Kernels (chosen in launch_gemm):
//   gemm_fp8_decode_kernel       FProp with M <= 32 (weight streaming; up to 64
//                                rows where the weight-sharing kernel is not
//                                chosen);
//   gemm_fp8_decode_ws_kernel    FProp with 33 .. 256 rows (weight chunks staged
//                                in LDS once per workgroup for several waves of
//                                tokens);
//                                both also over the rollout-packed weight
//                                (gemm_fprop_packed; pack_weight_rollout_kernel
//                                writes that weight);
//   gemm_fp8_large_kernel<mode>  256 x 256 tiles: problems with >= 256 of them
//                                (FProp and DGrad: one workgroup per CU looping
//                                over the tiles; a last round of at most half
//                                the CUs' tiles goes to the 128 x 128 kernel);
//                                FProp also with the SwiGLU + 1x128
//                                quantisation epilogue (gemm_fprop_swiglu_quant);
//   gemm_fp8_med_kernel<mode>    128 x 128 tiles, same machinery: everything else
//                                (four operand stages when the tiles do not
//                                fill the CUs, two otherwise).
// gemm_fprop_splitk (launch_gemm_fprop_splitk) runs the 128 x 128 kernel on K
// shares with fp32 partials in a caller workspace, then
// splitk_reduce_bf16_kernel.
// Byte offsets are 32-bit (buffer resources): launch_gemm runs a problem whose
// row operand or output reaches 2^31 bytes as launches over row ranges that
// stay below it.
// Every kernel but the split-K FProp's folds the K-blocks of an output in
// ascending order with the same fp32 operations, so a row's FProp output does
// not depend on the kernel (nor on the batch it is computed in).
#include <atomic>
#include <mutex>
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"
#include "silu_lookup.hpp"

namespace jetfp8 {

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v4f_t __attribute__((ext_vector_type(4)));
typedef int v2i_t __attribute__((ext_vector_type(2)));
typedef int v4i_t __attribute__((ext_vector_type(4)));

enum GemmMode { kFprop = 0, kDgrad = 1, kWgrad = 2 };

constexpr int kBN = 128, kBK = 128;  // weight block width, K-block depth
constexpr uint32_t kPackChunk = 2048;  // rollout-packed weight: bytes of one 16-row strip's K-block

__device__ __forceinline__ v2i_t lds_tr8(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (__attribute__((address_space(3))) v2i_t*)((__attribute__((address_space(3))) uint8_t*)(p)));
}

// Two fp32 values to a packed pair of bf16 (lo in bits 0..15), rounded to
// nearest even by v_cvt_pk_bf16_f32.  It agrees with f32_to_bf16_rne on every
// non-NaN fp32 value: tests/test_gpu_casts.py compares the same conversion,
// compiled with this library's flags, with the integer rounding on all 2^32
// bit patterns.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

__device__ __forceinline__ v4f_t mfma_fp8(const v8i_t& a, const v8i_t& b) {
  const v4f_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
  // cbsz = blgp = 0: both operands OCP E4M3; zero scale operands select the
  // unscaled instruction.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Large-tile kernel: 256 x 256 output tile, 8 waves (2 x 4) of 128 x 64, two
// waves per SIMD.  Operand tiles move global -> LDS with buffer loads that
// write LDS directly (buffer_load_dwordx4 ... lds: each lane's 16 bytes land
// at the wave's LDS base + 16 * lane), double-buffered: the next K-block's
// loads are in flight while the current one is multiplied.  A workgroup reads
// 64 KB of operands per 128-deep K-block for 16.8 MFLOP (256 FLOP per byte
// from L2, against 128 for a 128 x 128 tile), and each wave reads 24 KB of
// fragments from LDS for 4.2 MFLOP.  Buffer resources give 32-bit offsets and
// the hardware range check: rows past the end of A read as zero and stores
// past the end of C are dropped.
//
// LDS rows are 128 bytes (one K-block of one operand row); 16-byte chunk c of
// row r lives at chunk position c ^ f(r), f(r) = (r & 7) ^ bit3(r) ^ bit5(r).
// With that, the 16 rows read by one quarter-wave's ds_read_b128 hit 16
// distinct 4-bank groups, and the 8-row blocks read by ds_read_b64_tr_b8 in two
// quarter-waves hit distinct 2-bank pairs.
constexpr int kLBM = 256, kLBN = 256;
constexpr int kLThreads = 512;
constexpr int kLStage = kLBM * kBK + kLBN * kBK;  // 64 KB per stage (A then B)
constexpr int kGroupM = 8;                        // tile-row group of the launch order
constexpr uint32_t kRsrcWord3 = 0x00020000u;      // raw buffer, 32-bit dwords
// Cache-policy operand of a buffer store: nt (non-temporal, streaming).  The
// large kernel's epilogue writes each output line once and nothing in the
// kernel reads it back; every CU writes its 128 KB tile at about the same
// moment, and each wave's next barrier waits for its stores to be taken.
// Streaming also keeps FProp's and DGrad's large outputs from displacing the
// FP8 operands that the next GEMMs of the training step read from the caches:
// in the 8B step, streaming stores in FProp and DGrad took it 1 % below plain
// stores, while streaming WGrad's output as well gained nothing.  (Timed
// alone, back to back, all three kernels ran 3-5 % faster with them.)
constexpr int kStoreStream = 2;

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ int lf(int r) { return (r & 7) ^ ((r >> 3) & 1) ^ ((r >> 5) & 1); }
__device__ __forceinline__ int loff(int r, int c) { return r * 128 + ((c ^ lf(r)) << 4); }

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, (int)kRsrcWord3);
}

__device__ __forceinline__ void buf_to_lds16(rsrc_t r, uint8_t* lds_wave_base, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(lds_wave_base), 16,
                                           voff, soff, 0, 0);
}

// vmcnt(0): wait for every outstanding vector-memory load of this wave
// (including the LDS-direct loads); expcnt and lgkmcnt left at their maxima.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// vmcnt(n), n <= 63: wait until at most n of this wave's vector-memory loads
// are outstanding (they complete in issue order for this count).
template <int kN>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(kN >= 0 && kN <= 63, "vmcnt is a 6-bit field");
  __builtin_amdgcn_s_waitcnt((kN & 15) | ((kN >> 4) << 14) | 0x0F70);
}

// Workgroup barrier for LDS traffic: waits for this wave's LDS operations,
// not for its outstanding global loads (__syncthreads() is also a release
// fence, which waits for every load in flight, direct-to-LDS ones included).
__device__ __forceinline__ void lds_barrier() { __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// f(std::integral_constant<int, 0>{}), .., f(std::integral_constant<int, kN - 1>{})
template <int kN, int kI = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (kI < kN) {
    f(std::integral_constant<int, kI>{});
    static_for<kN, kI + 1>(f);
  }
}

// One stage of operand tiles (A then B) and its scales, as separate LDS
// objects: the loop below is unrolled over the two stages so that every LDS
// access names its stage statically, which lets the compiler see that the
// fragment reads of one stage do not alias the in-flight direct loads into
// the other (otherwise it waits for those loads before every read).
// Row factors are stored transposed, row r at [(r % 16) * kLScPitch + r / 16]:
// lane lr then reads its eight row sub-tiles' factors as two float4s at
// lr * kLScPitch + 8 wm, and with a pitch of 20 floats (not 16) the sixteen
// lanes of a quarter-wave cover disjoint four-bank groups (20 lr mod 64 runs
// over the multiples of 4), as do the 64 lanes' 4-byte stores.  With a pitch of
// 16, lanes lr and lr + 4 shared banks: a 4-way conflict on every read, which
// cost 9-20 % of the GEMMs' time (measured with SQ_LDS_BANK_CONFLICT: 13-17 M
// conflict cycles per 8B-step GEMM, 0.5-1.6 M without these accesses).
constexpr int kLScPitch = 20;
struct LStage {
  uint8_t ab[kLStage];
  // FProp, DGrad: sc[h] holds fl32(sa(row) * sb(block h)) for the tile's two
  // 128-column halves h, so the rescale needs no multiply; WGrad: sc[0] holds
  // the A-row scales, sc[1] the 256 B-column scales in column order.
  float sc[2][16 * kLScPitch];
};

// The MFMAs take the B-tile fragment as their first operand and the A-tile
// fragment as their second, so D = (B-sub-tile) x (A-sub-tile)^T: lane l holds
// output row 16 i + (l % 16) of its A sub-tile and the four consecutive output
// columns 16 j + 4 (l / 16) .. + 3 of its B sub-tile.  One row scale then
// covers a whole 4-value partial, and the epilogue writes 8-byte pieces.
template <int kMode, bool kSwiglu = false>
struct LargeTile {
  int t, l, w, wm, wn, lr, lk;
  uint32_t M, N, K, lds, row0, col0, nkb, t8, arow;  // lds: row stride of the A scales
  // kSwiglu (FProp fused with SwiGLU): the tile's output columns are the
  // h-columns col0 .. col0 + 127 (tile columns step by 128), and B row r of
  // the stage is weight row col0 + r (gate) for r < 128, col0 + bskip + r (up,
  // bskip = N / 2 - 128) otherwise.
  uint32_t bskip = 0;
  bool b_half;
  rsrc_t ra, rb;
  uint32_t va[4], vb[4];
  const float* sa;
  const float* sb;
  // LDS byte offsets inside a stage (see compute())
  uint32_t a_even, a_odd, b_even, b_odd, s_row;
  uint32_t dv[4];

  __device__ __forceinline__ void setup_offsets() {
    const uint32_t f0 = (uint32_t)((lr & 7) ^ ((lr >> 3) & 1));
    const uint32_t ra0 = (uint32_t)(wm * 128 + lr) * 128u;
    a_even = ra0 + (((uint32_t)(2 * lk) ^ f0) << 4);
    a_odd = ra0 + (((uint32_t)(2 * lk + 1) ^ f0) << 4);
    const uint32_t rb0 = (uint32_t)(kLBM * kBK) + (uint32_t)(wn * 64 + lr) * 128u;
    b_even = rb0 + (((uint32_t)(2 * lk) ^ f0) << 4);
    b_odd = rb0 + (((uint32_t)(2 * lk + 1) ^ f0) << 4);
    s_row = (uint32_t)(lr * kLScPitch + wm * 8) * 4u;
    // DGrad: transposed reads of B[n][c]; n = 32 lk + 8 q + lr / 2, chunk 4 (wn % 2) + j
    const uint32_t x = (uint32_t)(((lr >> 1) & 7) ^ (lk & 1) ^ (4 * (wn & 1)));
    const uint32_t dbase = (uint32_t)(kLBM * kBK) + (uint32_t)(wn >> 1) * (128u * 128u) +
                           (uint32_t)(32 * lk + (lr >> 1)) * 128u + 8u * (uint32_t)(lr & 1);
#pragma unroll
    for (int v = 0; v < 4; ++v) dv[v] = dbase + (((uint32_t)v ^ x) << 4);
  }

  // Tile id -> output tile origin (tile-row groups of kGroupM rows walked
  // column by column) and the per-tile load offsets.
  __device__ __forceinline__ void set_tile(uint32_t id, uint32_t ntm, uint32_t ntn) {
    const uint32_t per_group = kGroupM * ntn;
    const uint32_t g0 = (id / per_group) * kGroupM;
    const uint32_t gm = (ntm - g0) < (uint32_t)kGroupM ? (ntm - g0) : (uint32_t)kGroupM;
    row0 = (g0 + (id % per_group) % gm) * kLBM;
    col0 = ((id % per_group) / gm) * (kSwiglu ? 128u : (uint32_t)kLBN);
    arow = (row0 + t8) < M ? (row0 + t8) : (M - 1);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int r = 32 * w + 8 * p + (l >> 3);
      va[p] = (row0 + r) * K + (((l & 7) ^ lf(r)) << 4);
      if (kMode == kDgrad) {
        // B tile = W[kb*128 + rr][col0 + 128 h + ...]: two 128-column halves of
        // 128 contraction rows; this wave fills half h = w / 4, rows 32 (w % 4) ..
        const int rr = 32 * (w & 3) + 8 * p + (l >> 3);
        vb[p] = rr * N + col0 + 128 * (w >> 2) + (((l & 7) ^ lf(rr)) << 4);
      } else {
        vb[p] = (col0 + r + (kSwiglu && r >= 128 ? bskip : 0u)) * K + (((l & 7) ^ lf(r)) << 4);
      }
    }
  }

  // Direct loads of K-block kb into stage st: wave w fills 32 rows of each
  // operand tile, 8 rows (1 KB) per instruction; lane l covers row l / 8 of
  // the 8, chunk position l % 8, i.e. logical chunk (l % 8) ^ f(row).
  // Piece p < 4 is A rows 32 w + 8 p .., piece 4 + p the matching B rows.
  __device__ __forceinline__ void issue_piece(uint32_t kb, LStage& st, int piece) const {
    uint8_t* As = st.ab;
    uint8_t* Bs = st.ab + kLBM * kBK;
    const int p = piece & 3;
    if (piece < 4)
      buf_to_lds16(ra, As + (32 * w + 8 * p) * 128, va[p], kb * kBK);
    else if (kMode == kDgrad)
      buf_to_lds16(rb, Bs + (w >> 2) * (128 * 128) + (32 * (w & 3) + 8 * p) * 128, vb[p], kb * kBK * N);
    else
      buf_to_lds16(rb, Bs + (32 * w + 8 * p) * 128, vb[p], kb * kBK);
  }
  __device__ __forceinline__ void issue(uint32_t kb, LStage& st) const {
#pragma unroll
    for (int piece = 0; piece < 8; ++piece) issue_piece(kb, st, piece);
  }
  // Scales of one K-block, staged in LDS with the tiles.  FProp, DGrad:
  // thread t forms fl32(sa(row t % 256) * sb(block of column half t / 256)),
  // the factor the rescale applies.  WGrad: threads 0..255 fetch the A-row
  // scales, threads 256..511 the 256 B-column scales.  All compute-side reads
  // are then in-order LDS reads.  No divergent branches.  The product is
  // formed in store_scale, after the block's MFMAs, so that the loads' latency
  // is never waited for up front.
  __device__ __forceinline__ float2 load_scale(uint32_t kb) const {
    if (kMode == kWgrad) return make_float2(b_half ? sb[kb * N + col0 + t8] : sa[kb * lds + arow], 1.0f);
    const uint32_t cb = kSwiglu ? (col0 + (t >= 256 ? 128u + bskip : 0u)) / kBN : col0 / kBN + ((uint32_t)t >> 8);
    const uint32_t bi = (kMode == kFprop) ? cb * nkb + kb : kb * (N / kBN) + cb;
    return make_float2(sa[kb * lds + arow], sb[bi]);
  }
  __device__ __forceinline__ void store_scale(LStage& st, float2 x) const {
    const uint32_t tr = (t8 & 15u) * (uint32_t)kLScPitch + (t8 >> 4);
    st.sc[t >> 8][(kMode == kWgrad && t >= kLBM) ? t8 : tr] = (kMode == kWgrad) ? x.x : x.x * x.y;
  }

  __device__ __forceinline__ static v8i_t frag(const uint8_t* base, uint32_t o0, uint32_t o1) {
    const uint4 x0 = *reinterpret_cast<const uint4*>(base + o0);
    const uint4 x1 = *reinterpret_cast<const uint4*>(base + o1);
    return v8i_t{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
  }

  // Registers carried from one K-block into the next: the first A fragment,
  // the first two B fragments and the row factors of the block, read from its
  // stage right after the barrier that publishes it.
  struct Head {
    v8i_t af0, bf0, bf1;
    float srow[8];
  };

  // B fragment j of the stage at S.  DGrad: transposed reads of W's rows.
  __device__ __forceinline__ v8i_t read_b(const uint8_t* S, int j) const {
    if (kMode == kDgrad) {
      v2i_t part[4];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) part[q4] = lds_tr8(S + dv[j ^ (q4 & 1)] + 1024 * q4);
      return v8i_t{part[0].x, part[0].y, part[1].x, part[1].y, part[2].x, part[2].y, part[3].x, part[3].y};
    }
    const bool sw = (j >> 1) & 1;
    return frag(S + 2048 * j, sw ? b_odd : b_even, sw ? b_even : b_odd);
  }
  // Row factors of the 8 row sub-tiles (transposed layout: 8 contiguous
  // floats); FProp, DGrad: the products for the column half holding the
  // wave's 64 columns.
  __device__ __forceinline__ void read_srow(const LStage& st, float (&srow)[8]) const {
    const uint8_t* sr = reinterpret_cast<const uint8_t*>(st.sc[kMode == kWgrad ? 0 : (wn >> 1)]) + s_row;
    const float4 s0 = *reinterpret_cast<const float4*>(sr);
    const float4 s1 = *reinterpret_cast<const float4*>(sr + 16);
    srow[0] = s0.x; srow[1] = s0.y; srow[2] = s0.z; srow[3] = s0.w;
    srow[4] = s1.x; srow[5] = s1.y; srow[6] = s1.z; srow[7] = s1.w;
  }
  // The first A fragment is read before the B fragments: the block's first
  // MFMA then waits for four reads instead of the whole set.
  __device__ __forceinline__ void read_head(const LStage& st, Head& h) const {
    h.af0 = frag(st.ab, a_even, a_odd);
    h.bf0 = read_b(st.ab, 0);
    h.bf1 = read_b(st.ab, 1);
    read_srow(st, h.srow);
  }

  // Multiply the K-block held in stage st into the accumulators, load K-block
  // kn into stage nxt, and publish nxt (with its scale factors xs) to all
  // waves: store the factors, wait for this wave's loads, barrier, read the
  // head of nxt.
  //
  // Row sub-tile i of the A tile: lane reads row wm*128 + 16 i + lr, logical
  // chunks 2 lk and 2 lk + 1.  The swizzle f(row) equals f0(lr) ^ bit1(i), so
  // the two chunk positions are fixed per lane and merely swap when bit 1 of i
  // is set: two base offsets plus an immediate 2048 i.  The same holds for
  // the B sub-tiles j.
  // The next K-block's direct loads (into the other stage) are issued one
  // piece every two MFMAs over the first half of the block: late enough not
  // to crowd the block's first fragment reads, early enough that the last
  // piece has half a block to arrive before the wait (issued through the
  // whole block, its latency showed in every block; in one burst, the
  // fragment reads stalled behind it).
  // WGrad publishes nxt at step kBar = 27, once the block's last LDS read (A
  // row 7, step 24) is done: the barrier and the next block's head reads then
  // overlap the last MFMAs and rescales, whose VALU work is largest in WGrad.
  // FProp and DGrad publish after the block, which leaves the loads more time
  // (measured better with cold caches).
  __device__ __forceinline__ void compute(const LStage& st, v4f_t (&acc)[8][4], uint32_t kn, LStage& nxt,
                                          float2 xs, Head& h) const {
    constexpr int kBar = kMode == kWgrad ? 27 : 34;
    const uint8_t* S = st.ab;
    v8i_t bf[4], af[2];
    bf[0] = h.bf0;
    bf[1] = h.bf1;
    af[0] = h.af0;
    float srow[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) srow[r] = h.srow[r];
    float scol[4][4];
    if (kMode == kWgrad) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 c4 = *reinterpret_cast<const float4*>(&st.sc[1][wn * 64 + 16 * j + 4 * lk]);
        scol[j][0] = c4.x; scol[j][1] = c4.y; scol[j][2] = c4.z; scol[j][3] = c4.w;
      }
    }
    auto publish = [&]() {
      store_scale(nxt, xs);
      wait_vmem();
      __syncthreads();
    };

    // Software pipeline over the 32 (row, column) sub-tiles, row-major: step q
    // issues the MFMA of sub-tile q, then rescales the partial of sub-tile
    // q - 2 into its accumulators, so two MFMAs separate every partial from
    // its use; the A fragment of the next row sub-tile is read a row ahead,
    // B fragments 2 and 3 at steps 0 and 1.  Scheduling barriers pin the order.
    v4f_t part[3];
#pragma unroll
    for (int q = 0; q < 34; ++q) {
      const int i = q >> 2, j = q & 3;
      if (q < 2) bf[q + 2] = read_b(S, q + 2);
      if (q < 32 && j == 0 && i + 1 < 8) {
        const int n = i + 1;
        const bool sw = (n >> 1) & 1;
        af[n & 1] = frag(S + 2048 * n, sw ? a_odd : a_even, sw ? a_even : a_odd);
      }
      if (q < 32) part[q % 3] = mfma_fp8(bf[j], af[i & 1]);
      // a wave in the first three quarters of its block issues ahead of one in
      // its tail (rescales, publish, barrier): measured 1-3 % faster
      if (q == 0) __builtin_amdgcn_s_setprio(1);
      if (q == 24) __builtin_amdgcn_s_setprio(0);
      if (q < 16 && !(q & 1)) issue_piece(kn, nxt, q >> 1);
      if (q == kBar) publish();
      if (q == kBar + 1) h.af0 = frag(nxt.ab, a_even, a_odd);
      if (q == kBar + 2) h.bf0 = read_b(nxt.ab, 0);
      if (q == kBar + 3) h.bf1 = read_b(nxt.ab, 1);
      if (q == kBar + 4) read_srow(nxt, h.srow);
      __builtin_amdgcn_sched_barrier(0);
      if (q >= 2) {
        const int qp = q - 2, pi = qp >> 2, pj = qp & 3;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float sc = (kMode == kWgrad) ? srow[pi] * scol[pj][e] : srow[pi];
          acc[pi][pj][e] = fmaf(part[qp % 3][e], sc, acc[pi][pj][e]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (kBar >= 34) {
      publish();
      read_head(nxt, h);
    }
  }
};

// Output element kinds of the tile kernels: bf16 (every entry point), fp32
// written, fp32 added to what the output already holds (WGrad into an fp32
// gradient buffer).
// kOutSwiglu (FProp only): the tile's gate and up columns are combined into
// SiLU(gate) * up and written as its 1x128 FP8 quantisation (codes + scales).
enum OutKind { kOutBf16 = 0, kOutF32 = 1, kOutF32Add = 2, kOutSwiglu = 3 };

// swiglu_quant's SiLU table (silu_lookup.hpp; the same generated entries),
// which the fused epilogue copies into its staging stage once per tile.
__device__ const uint32_t kSiluBitsEp[kSiluTable] __attribute__((aligned(16))) = {
#include "silu_table.inc"
};

// fp32 output straight from the accumulators: each lane's four consecutive
// columns of a 16 x 16 sub-tile go out as one 16-byte store (a quarter-wave
// covers 64 contiguous bytes of a row); rows past the end fall outside the
// buffer, read as zero and are not written.
template <int kOut>
__device__ __forceinline__ void store_f32(rsrc_t rc, uint32_t byte_off, v4f_t v) {
  if (kOut == kOutF32Add) v += __builtin_bit_cast(v4f_t, __builtin_amdgcn_raw_buffer_load_b128(rc, byte_off, 0, 0));
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i_t, v), rc, byte_off, 0, 0);
}

template <int kMode, int kOut = kOutBf16>
__global__ __launch_bounds__(kLThreads) void gemm_fp8_large_kernel(const uint8_t* __restrict__ A,
                                                                    const float* __restrict__ sa,
                                                                    const uint8_t* __restrict__ B,
                                                                    const float* __restrict__ sb,
                                                                    uint32_t M, uint32_t N, uint32_t K,
                                                                    uint32_t lds, void* __restrict__ Cv,
                                                                    float* __restrict__ Sv) {
  static_assert(kOut != kOutSwiglu || kMode == kFprop, "the SwiGLU epilogue follows FProp");
  __shared__ __attribute__((aligned(16))) LStage st0;
  __shared__ __attribute__((aligned(16))) LStage st1;

  LargeTile<kMode, kOut == kOutSwiglu> g;
  if constexpr (kOut == kOutSwiglu) g.bskip = N / 2 - 128;
  g.t = threadIdx.x;
  g.l = g.t & 63;
  g.w = __builtin_amdgcn_readfirstlane(g.t >> 6);  // wave index, held in a scalar register
  g.wm = g.w >> 2;                                  // wave tile: rows wm*128 .. +128,
  g.wn = g.w & 3;                                   //            cols wn*64 .. +64
  g.lr = g.l & 15;
  g.lk = g.l >> 4;
  g.M = M; g.N = N; g.K = K; g.lds = lds;
  g.sa = sa; g.sb = sb;
  g.setup_offsets();
  g.nkb = K / kBK;
  g.t8 = (uint32_t)g.t & 255u;
  g.b_half = (kMode == kWgrad) && g.t >= kLBM;
  g.ra = make_rsrc(A, M * K);
  g.rb = make_rsrc(B, N * K);

  // Tiles of this workgroup.  The grid is a multiple of 8 workgroups, dealt to
  // the 8 XCDs round-robin; each XCD works through one contiguous range of
  // tile ids (its share of the operands stays in its L2), its workgroups
  // taking ids local, local + (workgroups per XCD), ...  With as many
  // workgroups as tiles each takes one; with fewer (one per CU) each loops
  // over several, and the last K-block of a tile already loads the first
  // block of the next one (FProp and DGrad with an even block count; see the
  // launcher).  WGrad keeps one tile per workgroup: the loop's extra live
  // registers made it spill (measured 4-6 % slower), while FProp gained 2-4 %.
  constexpr bool kPersist = kMode != kWgrad;
  const uint32_t ntm = (M + kLBM - 1) / kLBM, ntn = N / kLBN, total = ntm * ntn;
  const bool xcd_split = (total & 7) == 0;
  const uint32_t per_xcd = total >> 3, wg_per_xcd = gridDim.x >> 3;
  const uint32_t xcd = blockIdx.x & 7;
  uint32_t local = xcd_split ? (blockIdx.x >> 3) : blockIdx.x;
  const uint32_t stride = xcd_split ? wg_per_xcd : gridDim.x;
  const uint32_t range = xcd_split ? per_xcd : total;
  auto tile_id = [&](uint32_t loc) { return xcd_split ? xcd * per_xcd + loc : loc; };
  if (local >= range) return;  // (the launcher never makes such workgroups)
  g.set_tile(tile_id(local), ntm, ntn);

  g.store_scale(st0, g.load_scale(0));
  g.issue(0, st0);
  wait_vmem();
  __syncthreads();
  typename LargeTile<kMode, kOut == kOutSwiglu>::Head head;
  g.read_head(st0, head);

  const uint32_t last = g.nkb - 1;
#pragma clang loop unroll(disable)
  for (;;) {
    const uint32_t row0 = g.row0, col0 = g.col0;
    const bool has_next = kPersist && (g.nkb & 1) == 0 && local + stride < range;
    v4f_t acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = v4f_t{0.0f, 0.0f, 0.0f, 0.0f};

    // Two K-blocks per trip: compute stage 0 while stage 1 loads, then the
    // reverse.  After the tile's last block the prefetch moves on to the next
    // tile's first block, or, for the last tile, reloads the last block (the
    // loop stays free of branches on the data path; nkb >= 1).
#pragma clang loop unroll(disable)
    for (uint32_t kb = 0; kb < g.nkb; kb += 2) {
      {
        const uint32_t kn = kb + 1 <= last ? kb + 1 : last;
        g.compute(st0, acc, kn, st1, g.load_scale(kn), head);
      }
      if (kb + 1 <= last) {
        uint32_t kn = kb + 2;
        if (kn > last) {
          kn = last;
          if (has_next) {
            local += stride;
            g.set_tile(tile_id(local), ntm, ntn);
            kn = 0;
          }
        }
        g.compute(st1, acc, kn, st0, g.load_scale(kn), head);
      }
    }

    if constexpr (kOut == kOutSwiglu) {
      // SwiGLU + 1x128 quantisation of the tile: h-columns col0 .. col0 + 127
      // (gate in tile columns 0..127, up in 128..255), bit for bit what
      // swiglu_quant computes from gemm_fprop's bf16 output.  The accumulators
      // are first rounded to bf16 as gemm_fprop rounds them (packed, which frees
      // the fp32 registers).  Stage 1 holds the SiLU table (32 KB, copied in
      // with direct loads as the epilogue starts) and a 64-row slice of the
      // tile at a time: thread t takes row t / 8 of it, h-columns
      // 16 (t % 8) .. + 15: silu from the table, h = fl32(silu * up), the group
      // amax across the row's eight threads, the scale and the codes (one
      // 16-byte store).  Rows past M fall outside the codes' buffer and are
      // dropped; their scales are not written.
      const uint32_t I = N / 2;
      uint32_t pk[8][4][2];
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          pk[i][j][0] = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
          pk[i][j][1] = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
        }
      constexpr int kPitch = kLBN * 2 + 16;
      constexpr int kTab = 64 * kPitch;  // byte offset of the table in the stage
      static_assert(kTab + 4 * kSiluTable <= (int)sizeof(LStage), "epilogue staging and table must fit one stage");
      const rsrc_t rq = make_rsrc(Cv, M * I);
      uint8_t* stage = reinterpret_cast<uint8_t*>(&st1);
      {
        // every wave copies 4 KB of the table (four 1 KB direct loads)
        const rsrc_t rt = make_rsrc(kSiluBitsEp, 4u * kSiluTable);
#pragma unroll
        for (int p = 0; p < 4; ++p)
          buf_to_lds16(rt, stage + kTab + 1024 * (4 * g.w + p), 16u * (uint32_t)g.l, 1024u * (uint32_t)(4 * g.w + p));
      }
      const float* tab = reinterpret_cast<const float*>(stage + kTab);
      const int er = g.t >> 3, eo = g.t & 7;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          if (g.wm == h) {
#pragma unroll
            for (int i = 4 * q; i < 4 * q + 4; ++i) {
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const int r = 16 * (i - 4 * q) + g.lr, c = g.wn * 64 + 16 * j + 4 * g.lk;
                *reinterpret_cast<uint2*>(stage + r * kPitch + 2 * c) = make_uint2(pk[i][j][0], pk[i][j][1]);
              }
              __builtin_amdgcn_sched_barrier(0);
            }
          }
          if (h == 0 && q == 0) wait_vmem();  // this wave's part of the table has landed
          __syncthreads();
          const uint8_t* rowp = stage + er * kPitch + 2 * 16 * eo;
          uint4 gv[2], uv[2];
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            gv[c] = *reinterpret_cast<const uint4*>(rowp + 16 * c);
            uv[c] = *reinterpret_cast<const uint4*>(rowp + 2 * 128 + 16 * c);
          }
          float hv[2][8];
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            float u[8];
            unpack_bf16x8(uv[c], u);
            const uint32_t gw[4] = {gv[c].x, gv[c].y, gv[c].z, gv[c].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              hv[c][2 * e] = silu_of_bits(gw[e] & 0xFFFFu, tab) * u[2 * e];
              hv[c][2 * e + 1] = silu_of_bits(gw[e] >> 16, tab) * u[2 * e + 1];
            }
          }
          uint32_t am = max(__float_as_uint(absmax8(hv[0])), __float_as_uint(absmax8(hv[1])));
          am = max(am, dpp_u32<kXor1>(am));
          am = max(am, dpp_u32<kXor2>(am));
          am = max(am, dpp_u32<kHalfMirror>(am));
          const float sc = scale_from_amax(__uint_as_float(am));
          const double inv = inv_scale(sc);
          const uint2 c0 = quant8(hv[0], inv), c1 = quant8(hv[1], inv);
          const uint32_t grow = row0 + 128 * h + 64 * q + er;
          const uint32_t qoff = grow * I + col0 + 16 * eo;
          __builtin_amdgcn_raw_buffer_store_b128(v4i_t{(int)c0.x, (int)c0.y, (int)c1.x, (int)c1.y}, rq, qoff, 0, 0);
          if (eo == 0 && grow < M) Sv[(col0 / kGroup) * lds + grow] = sc;
          __syncthreads();
        }
      }
    } else if constexpr (kOut != kOutBf16) {
      const rsrc_t rc = make_rsrc(Cv, M * N * 4u);
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t r = row0 + g.wm * 128 + 16 * i + g.lr, c = col0 + g.wn * 64 + 16 * j + 4 * g.lk;
          store_f32<kOut>(rc, (r * N + c) * 4u, acc[i][j]);
        }
    } else {
      // bf16 epilogue, staged through stage 1 (free once the last block's
      // barrier has passed; stage 0 may already hold the next tile's first
      // block) in two halves of 128 rows with a row pitch of 512 + 16 bytes,
      // then written with 16-byte buffer stores, streaming in FProp and DGrad
      // (rows past M fall outside the buffer and are dropped)
      constexpr int kPitch = kLBN * 2 + 16;
      static_assert(128 * kPitch <= sizeof(LStage), "epilogue staging must fit one stage");
      uint16_t* C = static_cast<uint16_t*>(Cv);
      const rsrc_t rc = make_rsrc(C, M * N * 2u);
      uint8_t* stage = reinterpret_cast<uint8_t*>(&st1);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (g.wm == h) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int r = 16 * i + g.lr, c = g.wn * 64 + 16 * j + 4 * g.lk;
              // the hardware conversion saves about 3 VALU per element (FProp
              // 1-2 % faster); DGrad keeps the integer rounding, with which
              // its register allocation stays spill-free
              uint32_t lo, hi;
              if (kMode != kDgrad) {
                lo = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
                hi = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
              } else {
                lo = f32_to_bf16_rne(acc[i][j][0]) | (f32_to_bf16_rne(acc[i][j][1]) << 16);
                hi = f32_to_bf16_rne(acc[i][j][2]) | (f32_to_bf16_rne(acc[i][j][3]) << 16);
              }
              *reinterpret_cast<uint2*>(stage + r * kPitch + 2 * c) = make_uint2(lo, hi);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        __syncthreads();
#pragma unroll
        for (int p = 0; p < 8; ++p) {
          const int id16 = g.t + kLThreads * p;  // 16-byte chunk id: 32 per row
          const int r = id16 >> 5, c16 = id16 & 31;
          const uint4 v = *reinterpret_cast<const uint4*>(stage + r * kPitch + 16 * c16);
          const v4i_t d = {(int)v.x, (int)v.y, (int)v.z, (int)v.w};
          __builtin_amdgcn_raw_buffer_store_b128(d, rc, ((row0 + 128 * h + r) * N + col0 + 8 * c16) * 2u, 0,
                                                 kMode != kWgrad ? kStoreStream : 0);
        }
        __syncthreads();
      }
    }
    if (!has_next) break;
  }
}


// ---------------------------------------------------------------------------
// Medium-tile kernel: 128 x 128 output tile, 4 waves (2 x 2) of 64 x 64, two
// workgroups per CU.  The large kernel's machinery at a quarter of the tile:
// direct-to-LDS operand loads (double-buffered, issued early in each block),
// the same XOR swizzle, LDS-staged scale factors, the same fold per output
// element.  For problems with fewer than 256 tiles of 256 x 256 it keeps every
// CU busy where the large kernel would leave most idle.
constexpr int kMBM = 128, kMBN = 128;
constexpr int kMThreads = 256;

// Row factors transposed, r at [(r % 16) * kMScPitch + r / 16]: a pitch of 12
// floats (not 8) puts the sixteen float4 reads of a quarter-wave (lane lr at
// lr * kMScPitch + 4 wm) on disjoint bank groups, as in the large kernel.
constexpr int kMScPitch = 12;
struct MStage {
  uint8_t ab[kMBM * kBK + kMBN * kBK];  // 32 KB: A rows then B rows
  // FProp, DGrad: sc[0] holds fl32(sa(row) * sb(block)) (the tile's 128
  // columns are one weight block); WGrad: sc[0] the A-row scales, sc[1] the
  // 128 B-column scales in column order.
  float sc[2][16 * kMScPitch];
};

template <int kMode>
struct MedTile {
  int t, l, w, wm, wn, lr, lk;
  // nkb K-blocks starting at block kb0 (a K-split share; kb0 = 0 and
  // nkb = nkbt, all K / 128 blocks, otherwise); the block arguments below are
  // relative to kb0
  uint32_t M, N, K, lds, row0, col0, nkb, nkbt, kb0, arow;  // lds: row stride of the A scales
  rsrc_t ra, rb;
  uint32_t va[4], vb[4];
  const float* sa;
  const float* sb;
  uint32_t a_even, a_odd, b_even, b_odd, s_row;
  uint32_t dv[4];

  __device__ __forceinline__ void setup_offsets() {
    // row wm*64 + 16 i + lr: f(row) = f0(lr) ^ bit1(i) (as in the large kernel)
    const uint32_t f0 = (uint32_t)((lr & 7) ^ ((lr >> 3) & 1));
    const uint32_t ra0 = (uint32_t)(wm * 64 + lr) * 128u;
    a_even = ra0 + (((uint32_t)(2 * lk) ^ f0) << 4);
    a_odd = ra0 + (((uint32_t)(2 * lk + 1) ^ f0) << 4);
    const uint32_t rb0 = (uint32_t)(kMBM * kBK) + (uint32_t)(wn * 64 + lr) * 128u;
    b_even = rb0 + (((uint32_t)(2 * lk) ^ f0) << 4);
    b_odd = rb0 + (((uint32_t)(2 * lk + 1) ^ f0) << 4);
    s_row = (uint32_t)(lr * kMScPitch + wm * 4) * 4u;
    // DGrad: transposed reads of B[n][c]; n = 32 lk + 8 q + lr / 2, chunk 4 wn + j
    const uint32_t x = (uint32_t)(((lr >> 1) & 7) ^ (lk & 1) ^ (4 * wn));
    const uint32_t dbase = (uint32_t)(kMBM * kBK) + (uint32_t)(32 * lk + (lr >> 1)) * 128u + 8u * (uint32_t)(lr & 1);
#pragma unroll
    for (int v = 0; v < 4; ++v) dv[v] = dbase + (((uint32_t)v ^ x) << 4);
  }

  // Piece p < 4: A rows 32 w + 8 p ..; piece 4 + p: the matching B rows
  // (DGrad: contraction rows of the weight's 128-column block).
  __device__ __forceinline__ void issue_piece(uint32_t kb, MStage& st, int piece) const {
    uint8_t* As = st.ab;
    uint8_t* Bs = st.ab + kMBM * kBK;
    const int p = piece & 3;
    kb += kb0;
    if (piece < 4)
      buf_to_lds16(ra, As + (32 * w + 8 * p) * 128, va[p], kb * kBK);
    else if (kMode == kDgrad)
      buf_to_lds16(rb, Bs + (32 * w + 8 * p) * 128, vb[p], kb * kBK * N);
    else
      buf_to_lds16(rb, Bs + (32 * w + 8 * p) * 128, vb[p], kb * kBK);
  }
  __device__ __forceinline__ void issue(uint32_t kb, MStage& st) const {
#pragma unroll
    for (int piece = 0; piece < 8; ++piece) issue_piece(kb, st, piece);
  }
  // threads 0..127: the row factor of row t (FProp, DGrad: with the block
  // scale folded in); threads 128..255: WGrad column scales.  The product is
  // formed in store_scale, after the block's MFMAs.
  __device__ __forceinline__ float2 load_scale(uint32_t kb) const {
    kb += kb0;
    if (kMode == kWgrad) return make_float2(t >= kMBM ? sb[kb * N + col0 + (t - kMBM)] : sa[kb * lds + arow], 1.0f);
    const uint32_t cb = col0 / kBN;
    const uint32_t bi = (kMode == kFprop) ? cb * nkbt + kb : kb * (N / kBN) + cb;
    return make_float2(sa[kb * lds + arow], sb[bi]);
  }
  __device__ __forceinline__ void store_scale(MStage& st, float2 x) const {
    if (t < kMBM) st.sc[0][(t & 15) * kMScPitch + (t >> 4)] = (kMode == kWgrad) ? x.x : x.x * x.y;
    else if (kMode == kWgrad) st.sc[1][t - kMBM] = x.x;
  }

  __device__ __forceinline__ static v8i_t frag(const uint8_t* base, uint32_t o0, uint32_t o1) {
    const uint4 x0 = *reinterpret_cast<const uint4*>(base + o0);
    const uint4 x1 = *reinterpret_cast<const uint4*>(base + o1);
    return v8i_t{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
  }

  __device__ __forceinline__ void compute(const MStage& st, v4f_t (&acc)[4][4], uint32_t kn, MStage& nxt) const {
    const uint8_t* S = st.ab;
    v8i_t bf[4];
    auto read_b = [&](int j) {
      if (kMode == kDgrad) {
        v2i_t part[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) part[q4] = lds_tr8(S + dv[j ^ (q4 & 1)] + 1024 * q4);
        bf[j] = v8i_t{part[0].x, part[0].y, part[1].x, part[1].y,
                      part[2].x, part[2].y, part[3].x, part[3].y};
      } else {
        const bool sw = (j >> 1) & 1;
        bf[j] = frag(S + 2048 * j, sw ? b_odd : b_even, sw ? b_even : b_odd);
      }
    };
    v8i_t af[2];
    af[0] = frag(S, a_even, a_odd);
    read_b(0);
    read_b(1);
    float srow[4];
    {
      const float4 s0 = *reinterpret_cast<const float4*>(reinterpret_cast<const uint8_t*>(st.sc[0]) + s_row);
      srow[0] = s0.x; srow[1] = s0.y; srow[2] = s0.z; srow[3] = s0.w;
    }
    float scol[4][4];
    if (kMode == kWgrad) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 c4 = *reinterpret_cast<const float4*>(&st.sc[1][wn * 64 + 16 * j + 4 * lk]);
        scol[j][0] = c4.x; scol[j][1] = c4.y; scol[j][2] = c4.z; scol[j][3] = c4.w;
      }
    }
    // pipeline over the 16 (row, column) sub-tiles as in the large kernel; the
    // next block's 8 direct loads go out on the odd steps
    v4f_t part[3];
#pragma unroll
    for (int q = 0; q < 18; ++q) {
      const int i = q >> 2, j = q & 3;
      if (q < 2) read_b(q + 2);
      if (q < 16 && j == 0 && i + 1 < 4) {
        const int n = i + 1;
        const bool sw = (n >> 1) & 1;
        af[n & 1] = frag(S + 2048 * n, sw ? a_odd : a_even, sw ? a_even : a_odd);
      }
      if (q < 16) part[q % 3] = mfma_fp8(bf[j], af[i & 1]);
      // the next K-block's loads: two pieces per MFMA over the first four, so
      // that they have most of the (16-MFMA) block to arrive
      if (q < 4) {
        issue_piece(kn, nxt, 2 * q);
        issue_piece(kn, nxt, 2 * q + 1);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (q >= 2) {
        const int qp = q - 2, pi = qp >> 2, pj = qp & 3;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float sc = (kMode == kWgrad) ? srow[pi] * scol[pj][e] : srow[pi];
          acc[pi][pj][e] = fmaf(part[qp % 3][e], sc, acc[pi][pj][e]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
};

// kSt operand stages: 2 (double buffering, two workgroups per CU) or 4 (loads
// issued three K-blocks ahead, one workgroup per CU).  With one tile or less
// per CU, a tile's chain of K-blocks waits on memory latency at every block
// when only one block is in flight; four stages keep three in flight.
template <int kStages>
struct MedStages {
  static constexpr int kMinBlocks = kStages == 2 ? 2 : 1;
};

template <int kMode, int kOut = kOutBf16, int kSt = 2>
__global__ __launch_bounds__(kMThreads, MedStages<kSt>::kMinBlocks) void gemm_fp8_med_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ sa, const uint8_t* __restrict__ B,
    const float* __restrict__ sb, uint32_t M, uint32_t N, uint32_t K, uint32_t lds, void* __restrict__ Cv) {
  static_assert(kSt == 2 || kSt == 4, "two or four operand stages");
  // separate LDS objects, named statically below (see LStage); st2 and st3
  // exist only with four stages
  __shared__ __attribute__((aligned(16))) MStage st0;
  __shared__ __attribute__((aligned(16))) MStage st1;
  typedef typename std::conditional<kSt == 4, MStage, char>::type MStageOpt;
  __shared__ __attribute__((aligned(16))) MStageOpt st2;
  __shared__ __attribute__((aligned(16))) MStageOpt st3;

  MedTile<kMode> g;
  g.t = threadIdx.x;
  g.l = g.t & 63;
  g.w = __builtin_amdgcn_readfirstlane(g.t >> 6);
  g.wm = g.w >> 1;  // wave tile: rows wm*64 .. +64, cols wn*64 .. +64
  g.wn = g.w & 1;
  g.lr = g.l & 15;
  g.lk = g.l >> 4;
  g.M = M; g.N = N; g.K = K; g.lds = lds;
  g.sa = sa; g.sb = sb;
  g.setup_offsets();

  // launch order as in the large kernel: one contiguous tile range per XCD,
  // tile-row groups of kGroupM rows walked column by column
  const uint32_t ntm = (M + kMBM - 1) / kMBM, ntn = N / kMBN, total = ntm * ntn;
  uint32_t id = blockIdx.x;
  if ((total & 7) == 0) id = (id & 7) * (total >> 3) + (id >> 3);
  const uint32_t per_group = kGroupM * ntn;
  const uint32_t g0 = (id / per_group) * kGroupM;
  const uint32_t gm = (ntm - g0) < (uint32_t)kGroupM ? (ntm - g0) : (uint32_t)kGroupM;
  g.row0 = (g0 + (id % per_group) % gm) * kMBM;
  g.col0 = ((id % per_group) / gm) * kMBN;
  // K-split share: blockIdx.y of gridDim.y equal ranges (the launcher makes
  // gridDim.y divide the block count; it is 1 except for split FProp)
  g.nkbt = K / kBK;
  g.nkb = g.nkbt / gridDim.y;
  g.kb0 = blockIdx.y * g.nkb;
  const uint32_t t7 = (uint32_t)g.t & 127u;
  g.arow = (g.row0 + t7) < M ? (g.row0 + t7) : (M - 1);
  g.ra = make_rsrc(A, M * K);
  g.rb = make_rsrc(B, N * K);
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int r = 32 * g.w + 8 * p + (g.l >> 3);
    g.va[p] = (g.row0 + r) * K + (((g.l & 7) ^ lf(r)) << 4);
    if (kMode == kDgrad)
      g.vb[p] = r * N + g.col0 + (((g.l & 7) ^ lf(r)) << 4);  // contraction row r of the block
    else
      g.vb[p] = (g.col0 + r) * K + (((g.l & 7) ^ lf(r)) << 4);
  }

  v4f_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f_t{0.0f, 0.0f, 0.0f, 0.0f};

  auto stage = [&](auto c) -> MStage& {
    constexpr int i = decltype(c)::value;
    if constexpr (i == 0) return st0;
    else if constexpr (i == 1) return st1;
    else if constexpr (i == 2) return *reinterpret_cast<MStage*>(&st2);  // (kSt == 4 only)
    else return *reinterpret_cast<MStage*>(&st3);
  };
  const uint32_t last = g.nkb - 1;
  // Block kb lives in stage kb % kSt.  Its scale factors are fetched into
  // registers when its loads are issued (kSt - 1 blocks ahead) and stored to
  // its stage at the end of the block before it.
  float2 xs[kSt];
  static_for<kSt - 1>([&](auto c) {
    constexpr int p = decltype(c)::value;
    const uint32_t kp = (uint32_t)p <= last ? (uint32_t)p : last;
    xs[p] = g.load_scale(kp);
    g.issue(kp, stage(c));
  });
  // Publishing a block: with four stages the barrier must not be a fence,
  // which would wait for the later blocks' loads too; each wave's vmcnt wait
  // covers its own pieces of the block, the barrier everyone's.
  auto publish = [&]() {
    wait_vmem_le<8 * (kSt - 2)>();
    if constexpr (kSt == 2) __syncthreads();
    else lds_barrier();
  };
  g.store_scale(st0, xs[0]);
  publish();  // block 0's pieces (blocks 1 .. kSt - 2 may be in flight)

  // One K-block in stage s: issue block kb + kSt - 1 (clamped to the last:
  // the extra loads fill a stage no remaining block uses), multiply, then
  // publish block kb + 1: its factors into its stage, wait for this wave's
  // pieces of it (8 pieces per block are issued after them for each of the
  // kSt - 2 later blocks), barrier.
  auto step = [&](auto c, uint32_t kb) {
    constexpr int st = decltype(c)::value;
    constexpr int sn = (st + kSt - 1) % kSt, s1 = (st + 1) % kSt;
    const uint32_t kn = kb + kSt - 1 <= last ? kb + kSt - 1 : last;
    xs[sn] = g.load_scale(kn);
    g.compute(stage(c), acc, kn, stage(std::integral_constant<int, sn>{}));
    if (kb + 1 <= last) {
      g.store_scale(stage(std::integral_constant<int, s1>{}), xs[s1]);
      publish();
    }
  };
#pragma clang loop unroll(disable)
  for (uint32_t kb = 0; kb < g.nkb; kb += kSt) {
    step(std::integral_constant<int, 0>{}, kb);
    if (kb + 1 > last) break;
    step(std::integral_constant<int, 1>{}, kb + 1);
    if constexpr (kSt == 4) {
      if (kb + 2 > last) break;
      step(std::integral_constant<int, 2>{}, kb + 2);
      if (kb + 3 > last) break;
      step(std::integral_constant<int, 3>{}, kb + 3);
    }
  }
  // the clamped loads of the last blocks may still be landing in stages the
  // epilogue reuses
  wait_vmem();
  __syncthreads();

  if constexpr (kOut != kOutBf16) {
    // a K-split share writes its own fp32 partial: slice blockIdx.y of [splits][M][N]
    const rsrc_t rc = make_rsrc(static_cast<float*>(Cv) + (size_t)blockIdx.y * M * N, M * N * 4u);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t r = g.row0 + g.wm * 64 + 16 * i + g.lr, c = g.col0 + g.wn * 64 + 16 * j + 4 * g.lk;
        store_f32<kOut>(rc, (r * N + c) * 4u, acc[i][j]);
      }
    return;
  }
  uint16_t* C = static_cast<uint16_t*>(Cv);
  // epilogue: bf16 tile staged in LDS (rows 0..63 in stage 0, 64..127 in
  // stage 1, pitch 256 + 16 bytes), then 16-byte buffer stores
  constexpr int kPitch = kMBN * 2 + 16;
  static_assert(64 * kPitch <= (int)sizeof(MStage), "epilogue staging must fit one stage");
  const rsrc_t rc = make_rsrc(C, M * N * 2u);
  auto crow = [&](int r) -> uint8_t* {
    return (r < 64 ? reinterpret_cast<uint8_t*>(&st0) : reinterpret_cast<uint8_t*>(&st1)) + (r & 63) * kPitch;
  };
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = g.wm * 64 + 16 * i + g.lr, c = g.wn * 64 + 16 * j + 4 * g.lk;
      const uint32_t lo = f32_to_bf16_rne(acc[i][j][0]) | (f32_to_bf16_rne(acc[i][j][1]) << 16);
      const uint32_t hi = f32_to_bf16_rne(acc[i][j][2]) | (f32_to_bf16_rne(acc[i][j][3]) << 16);
      *reinterpret_cast<uint2*>(crow(r) + 2 * c) = make_uint2(lo, hi);
    }
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int id16 = g.t + kMThreads * p;  // 16-byte chunk id: 16 per row
    const int r = id16 >> 4, c16 = id16 & 15;
    const uint4 v = *reinterpret_cast<const uint4*>(crow(r) + 16 * c16);
    const v4i_t d = {(int)v.x, (int)v.y, (int)v.z, (int)v.w};
    __builtin_amdgcn_raw_buffer_store_b128(d, rc, ((g.row0 + r) * N + g.col0 + 8 * c16) * 2u, 0, 0);
  }
}

// ---------------------------------------------------------------------------
// Decode FProp (M <= 64 tokens, rollout): parallel weight streaming with the
// sequential accumulation order kept.
//
// One workgroup per kS strips of 16 output columns (a wave's X fragments
// serve all kS strips).  Its kW waves compute the 128-deep block partials
// P_kb = MFMA(W slice, X slice) of different K-blocks at once (wave w takes
// K-block c * kW + w of chunk c, with kD K-blocks of operands and scales in
// flight per wave, loaded straight into registers), and park them in LDS with
// their factors fl32(sx * sw).  After each chunk, wave i (one
// per 16 tokens) folds the chunk's partials in ascending K order:
// acc = fma(P_kb, fl32(sx * sw), acc) -- exactly the per-element operation
// sequence of the 128 x 128 and 256 x 256 FProp kernels, so a token's output
// is bit-identical whichever of these kernels and batch sizes compute it.
// kS and kW are chosen at launch from the strip count; with kW = 1 the lone
// wave folds each partial as soon as it is computed, with no LDS.
//
// Every prefetch load is issued on every path (clamped to the last block past
// the end), so the compiler's wait before a slot's use covers that slot's
// loads only, and the chunk barrier waits for LDS traffic only: a
// __syncthreads() fence would drain the prefetched global loads every chunk.
template <int kMT, int kW, int kS>  // token sub-tiles (M <= 16 kMT), K-phases, strips per wave
struct DecodeCfg {
  // K-blocks of operands in flight per wave: about 128 registers of slots
  // (56 with 16 waves per workgroup, which leaves 128 registers per lane)
  static constexpr int kSlotRegs = 8 * (kS + kMT);
  static constexpr int kFit = (kW == 16 ? 56 : 128) / kSlotRegs;
  static constexpr int kMax = kW == 1 ? 8 : 4;
  static constexpr int kD = kFit > kMax ? kMax : (kFit < 1 ? 1 : kFit);
  static_assert(kW == 1 || kW >= kMT, "one folding wave per 16-token sub-tile");
  static_assert(kW == 1 || kW * kMT * kS <= 64, "parked partials must fit in LDS");
  static_assert(16 * kS <= kBN, "a wave's strips lie in one 128-column weight block");
};

// Prefetched scale loads use the buffer-load intrinsic, as the operands do:
// the compiler keeps these where they are issued, while a plain load would be
// sunk to its use (and then waited for at once).  The offset is held in a
// vector register even when it is uniform, so that the load takes the vector
// memory path: a scalar-cache load can return out of order, and every use of
// one waits for all of them, including the prefetches issued after it.
__device__ __forceinline__ float ld_scale(rsrc_t r, uint32_t byte_off) {
  __asm__("" : "+v"(byte_off));
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0));
}


// kPk: W is in the rollout-packed order of pack_weight_rollout_kernel (each
// 16-row strip's K-block a contiguous 2 KB chunk holding every lane's operand
// bytes in lane order) instead of row-major [N][K]; the loads then cover 1 KB
// of consecutive bytes each and a wave walks one contiguous range of memory.
template <int kMT, int kW, int kS, bool kPk>
__global__ __launch_bounds__(64 * kW) void gemm_fp8_decode_kernel(
    const uint8_t* __restrict__ X, const float* __restrict__ sx, const uint8_t* __restrict__ W,
    const float* __restrict__ sw, uint32_t M, uint32_t N, uint32_t K, uint16_t* __restrict__ Y) {
  constexpr int kD = DecodeCfg<kMT, kW, kS>::kD;
  constexpr uint32_t kWHalf = kPk ? 1024u : 16u;  // byte offset of a lane's second 16 operand bytes
  const int t = threadIdx.x, l = t & 63, lr = l & 15, lk = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const uint32_t n0 = blockIdx.x * (16u * kS);  // the workgroup's kS strips of 16 columns
  const uint32_t mb = blockIdx.y * (16u * kMT);  // its first token (a grid row per 16 kMT tokens)
  const uint32_t nkb = K / kBK;
  const uint32_t nch = (nkb + kW - 1) / kW;
  const rsrc_t rw = make_rsrc(W, N * K);
  const rsrc_t rx = make_rsrc(X, M * K);
  uint32_t w_off[kS], x_off[kMT], xm[kMT];
#pragma unroll
  for (int s = 0; s < kS; ++s)
    w_off[s] = kPk ? (n0 / 16u + s) * nkb * kPackChunk + 16u * l : (n0 + 16u * s + lr) * K + 32u * lk;
#pragma unroll
  for (int i = 0; i < kMT; ++i) {
    xm[i] = (mb + 16u * i + lr) < M ? (mb + 16u * i + lr) : (M - 1);  // ragged tail: repeat the last token
    x_off[i] = xm[i] * K + 32u * lk;
  }
  const rsrc_t rsx = make_rsrc(sx, nkb * M * 4u);
  const rsrc_t rsw = make_rsrc(sw + (n0 / kBN) * nkb, nkb * 4u);

  v8i_t wr[kD][kS], xr[kD][kMT];
  float sxr[kD][kMT], swr[kD];
  auto load = [&](int slot, uint32_t c) {
    uint32_t kb = c * kW + (uint32_t)w;
    kb = kb < nkb ? kb : nkb - 1;  // past the end: a valid block whose product is not used
    const uint32_t kofs = kb * kBK, wofs = kPk ? kb * kPackChunk : kofs;
#pragma unroll
    for (int s = 0; s < kS; ++s) {
      const v4i_t w0 = __builtin_amdgcn_raw_buffer_load_b128(rw, w_off[s], wofs, 0);
      const v4i_t w1 = __builtin_amdgcn_raw_buffer_load_b128(rw, w_off[s] + kWHalf, wofs, 0);
      wr[slot][s] = v8i_t{w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    }
#pragma unroll
    for (int i = 0; i < kMT; ++i) {
      const v4i_t x0 = __builtin_amdgcn_raw_buffer_load_b128(rx, x_off[i], kofs, 0);
      const v4i_t x1 = __builtin_amdgcn_raw_buffer_load_b128(rx, x_off[i] + 16u, kofs, 0);
      xr[slot][i] = v8i_t{x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      sxr[slot][i] = ld_scale(rsx, (kb * M + xm[i]) * 4u);
    }
    swr[slot] = ld_scale(rsw, kb * 4u);
  };
#pragma unroll
  for (int j = 0; j < kD; ++j) {
    load(j, (uint32_t)j);
    __builtin_amdgcn_sched_barrier(0);
  }

  if constexpr (kW == 1) {
    // a lone wave per strip group: fold each partial as soon as it is computed
    v4f_t acc1[kMT][kS];
#pragma unroll
    for (int i = 0; i < kMT; ++i)
#pragma unroll
      for (int s = 0; s < kS; ++s) acc1[i][s] = v4f_t{0.0f, 0.0f, 0.0f, 0.0f};
    uint32_t c0 = 0;
#pragma clang loop unroll(disable)
    do {
#pragma unroll
      for (int j = 0; j < kD; ++j) {
        // Branch-free: a step past the end (a clamped, valid block) gets the
        // factor 0 and leaves acc unchanged bit for bit (acc is never -0).
        const uint32_t kb = c0 + j;
#pragma unroll
        for (int i = 0; i < kMT; ++i) {
          const float sc = kb < nkb ? sxr[j][i] * swr[j] : 0.0f;
#pragma unroll
          for (int s = 0; s < kS; ++s) {
            const v4f_t p = mfma_fp8(wr[j][s], xr[j][i]);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc1[i][s][e] = fmaf(p[e], sc, acc1[i][s][e]);
          }
        }
        load(j, kb + kD);
        __builtin_amdgcn_sched_barrier(0);
      }
      c0 += kD;
    } while (c0 < nch);
#pragma unroll
    for (int i = 0; i < kMT; ++i) {
      const uint32_t m = mb + 16u * i + lr;
      if (m < M) {
#pragma unroll
        for (int s = 0; s < kS; ++s) {
          const uint32_t lo = f32_to_bf16_rne(acc1[i][s][0]) | (f32_to_bf16_rne(acc1[i][s][1]) << 16);
          const uint32_t hi = f32_to_bf16_rne(acc1[i][s][2]) | (f32_to_bf16_rne(acc1[i][s][3]) << 16);
          *reinterpret_cast<uint2*>(Y + (size_t)m * N + n0 + 16 * s + 4 * lk) = make_uint2(lo, hi);
        }
      }
    }
  } else {
    __shared__ v4f_t part[2][kW][kMT][kS][64];
    __shared__ float fac[2][kW][kMT][16];  // fl32(sx * sw) of each parked partial's tokens
    // the folding wave (w < kMT) owns token 16 w + lr, columns n0 + 16 s + 4 lk .. + 3
    v4f_t acc[kS];
#pragma unroll
    for (int s = 0; s < kS; ++s) acc[s] = v4f_t{0.0f, 0.0f, 0.0f, 0.0f};
    uint32_t c0 = 0;
#pragma clang loop unroll(disable)
    do {
#pragma unroll
      for (int j = 0; j < kD; ++j) {
        // Branch-free partials (past the end they are parked but never folded),
        // so the prefetched loads stay ahead of their uses.
        const uint32_t c = c0 + j;
        const int buf = (int)(c & 1);
#pragma unroll
        for (int i = 0; i < kMT; ++i) {
#pragma unroll
          for (int s = 0; s < kS; ++s) part[buf][w][i][s][l] = mfma_fp8(wr[j][s], xr[j][i]);
          if (lk == 0) fac[buf][w][i][lr] = sxr[j][i] * swr[j];
        }
        lds_barrier();
        if (w < kMT) {
#pragma unroll
          for (int k = 0; k < kW; ++k) {
            if (c * kW + k < nkb) {
              const float sc = fac[buf][k][w][lr];
#pragma unroll
              for (int s = 0; s < kS; ++s) {
                const v4f_t p = part[buf][k][w][s][l];
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[s][e] = fmaf(p[e], sc, acc[s][e]);
              }
            }
          }
        }
        load(j, c + kD);
        __builtin_amdgcn_sched_barrier(0);
      }
      c0 += kD;
    } while (c0 < nch);
    if (w < kMT && mb + 16u * (uint32_t)w + lr < M) {
      const uint32_t m = mb + 16u * (uint32_t)w + lr;
#pragma unroll
      for (int s = 0; s < kS; ++s) {
        const uint32_t lo = f32_to_bf16_rne(acc[s][0]) | (f32_to_bf16_rne(acc[s][1]) << 16);
        const uint32_t hi = f32_to_bf16_rne(acc[s][2]) | (f32_to_bf16_rne(acc[s][3]) << 16);
        *reinterpret_cast<uint2*>(Y + (size_t)m * N + n0 + 16 * s + 4 * lk) = make_uint2(lo, hi);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// FProp for rollout batches of 33 .. 256 tokens, weight shared through LDS.
// Once each weight byte feeds more than a few dozen tokens, a wave can no
// longer stream its own strips: the MFMA work per weight byte grows with the
// batch while one wave per SIMD keeps few bytes in flight.  Here a workgroup
// of kNW waves owns kS strips of 16 columns and 16 kR kNW tokens; every
// K-block it stages the kS weight chunks once with direct-to-LDS loads, and all
// its waves read them, each for its own kR sub-tiles of 16 tokens, whose X
// fragments (and the block's sx values) the wave stages into its own part of
// the same LDS stage.  Packed weight (kPk): a strip's K-block is one 2 KB
// chunk in fragment order (lane l's 16 bytes at 16 l of each 1 KB piece).
// Row-major weight, and always X: each 1 KB piece is 8 whole 128-byte rows
// whose 16-byte chunks land at the large kernel's swizzled positions (chunk c
// of row r at c ^ f(r)), so that whole cache lines are fetched and the
// fragment reads are conflict-free 16-byte LDS reads.  kD stages hold the
// next kD K-blocks; a block's fragments are read into registers while the
// block before it computes, and its steps are software-pipelined (see below).
// The weight-block scales of the workgroup's (at most two) 128-column blocks are
// copied to LDS once.  The grid walks (strip group, token group) pairs with
// the token groups of a strip group adjacent on one XCD, so a weight chunk
// read from HBM by one of them is found in that XCD's L2 by the others.  The
// fold is the sequential one of the other FProp kernels, acc = fma(P_kb,
// fl32(sx * sw), acc) in ascending K order: the output is bitwise gemm_fprop's
// on the same rows in any batch.
constexpr int kWsMaxKb = 512;  // K <= 65536: the copied weight-block scales fit 4 KB
template <int kR, int kS, int kNW, int kOcc = 1>  // kOcc: workgroups per CU (LDS split between them)
struct DecodeWsCfg {
  static constexpr int kTM = 16 * kR * kNW;               // tokens of a workgroup
  static constexpr int kWPieces = 2 * kS;                 // 1 KB weight pieces per K-block
  static constexpr int kPW = (kWPieces + kNW - 1) / kNW;  // weight pieces each wave loads (a few twice)
  static constexpr int kG = kPW + 2 * kR + 1;             // loads of one wave per K-block (+ its sx)
  static constexpr int kWBytes = 2048 * kS;
  static constexpr int kXBytes = 2048 * kR;               // one wave's X fragments
  static constexpr int kStage = kWBytes + kNW * kXBytes + 256 * kNW;
  static constexpr int kFit = (kOcc == 1 ? 155 * 1024 : 75 * 1024) / kStage;  // with the scale copy, within the LDS share
  static constexpr int kCnt = 63 / kG + 1;                // (kD - 1) kG loads may stay in flight
  static constexpr int kD0 = kFit < kCnt ? kFit : kCnt;
  static constexpr int kD = kD0 > 8 ? 8 : kD0;
  static_assert(kD >= 2, "at least two K-blocks in flight");
  static_assert((kD - 1) * kG <= 63, "wait count fits vmcnt");
  static_assert(kS <= 8, "a workgroup's strips span at most two weight blocks");
};

template <int kR, int kS, int kNW, bool kPk, int kOcc>
__global__ __launch_bounds__(64 * kNW, kOcc) void gemm_fp8_decode_ws_kernel(
    const uint8_t* __restrict__ X, const float* __restrict__ sx, const uint8_t* __restrict__ Wp,
    const float* __restrict__ sw, uint32_t M, uint32_t N, uint32_t K, uint16_t* __restrict__ Y) {
  using C = DecodeWsCfg<kR, kS, kNW, kOcc>;
  constexpr int kD = C::kD;
  __shared__ __attribute__((aligned(16))) uint8_t ws0[C::kStage], ws1[C::kStage];
  __shared__ __attribute__((aligned(16))) uint8_t ws2[kD > 2 ? C::kStage : 16], ws3[kD > 3 ? C::kStage : 16];
  __shared__ __attribute__((aligned(16))) uint8_t ws4[kD > 4 ? C::kStage : 16], ws5[kD > 5 ? C::kStage : 16];
  __shared__ __attribute__((aligned(16))) uint8_t ws6[kD > 6 ? C::kStage : 16], ws7[kD > 7 ? C::kStage : 16];
  __shared__ float swl[2 * kWsMaxKb];
  auto stage = [&](auto c) -> uint8_t* {
    constexpr int i = decltype(c)::value;
    if constexpr (i == 0) return ws0;
    else if constexpr (i == 1) return ws1;
    else if constexpr (i == 2) return ws2;
    else if constexpr (i == 3) return ws3;
    else if constexpr (i == 4) return ws4;
    else if constexpr (i == 5) return ws5;
    else if constexpr (i == 6) return ws6;
    else return ws7;
  };
  const int t = threadIdx.x, l = t & 63, lr = l & 15, lk = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const uint32_t nkb = K / kBK, last = nkb - 1;
  // (strip group, token group) of this workgroup: with a grid of 8 n
  // workgroups, XCD x (blockIdx mod 8) takes pairs x n .. x n + n - 1, token
  // group fastest
  const uint32_t ntg = (M + C::kTM - 1) / C::kTM, total = (N / (16u * kS)) * ntg;
  uint32_t pair = blockIdx.x;
  if ((total & 7) == 0) pair = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  const uint32_t sg = pair / ntg, tg = pair - sg * ntg;
  const uint32_t strip0 = sg * kS, n0 = 16u * strip0;
  const uint32_t mw = tg * C::kTM + (uint32_t)w * (16u * kR);  // this wave's first token

  // the weight-block scales sw[b0 + h][kb] of the (one or two) 128-column
  // blocks holding the strips, h = 0, 1
  const uint32_t b0 = n0 / kBN, nb = (n0 + 16u * kS - 1u) / kBN - b0 + 1u;
  for (uint32_t i = (uint32_t)t; i < nb * nkb; i += 64u * kNW) swl[i] = sw[b0 * nkb + i];
  __syncthreads();

  const rsrc_t rw = make_rsrc(Wp, N * K);
  const rsrc_t rx = make_rsrc(X, M * K);
  const rsrc_t rsx = make_rsrc(sx, nkb * M * 4u);
  uint32_t w_off[C::kPW], w_lds[C::kPW], x_off[kR][2];
#pragma unroll
  for (int q = 0; q < C::kPW; ++q) {
    const int pc = ((int)w + kNW * q) % C::kWPieces;  // piece pc: strip pc / 2, half pc % 2
    const uint32_t strip = strip0 + (uint32_t)(pc >> 1);
    if constexpr (kPk) {
      w_off[q] = strip * nkb * kPackChunk + 1024u * (pc & 1) + 16u * l;
    } else {
      // row-major weight: as the X pieces below, 8 whole rows with swizzled chunks
      const int r = 8 * (pc & 1) + (l >> 3);
      w_off[q] = (16u * strip + (uint32_t)r) * K + 16u * (uint32_t)((l & 7) ^ lf(r));
    }
    w_lds[q] = 2048u * (pc >> 1) + 1024u * (pc & 1);
  }
  // X piece h of sub-tile i: 8 whole 128-byte token rows 8 h .. 8 h + 7 (lane l:
  // row 8 h + l / 8), each row's 16-byte chunks stored at the swizzled
  // positions of the large kernel (chunk c of row r at c ^ f(r)), so that the
  // fragment reads below are conflict-free
#pragma unroll
  for (int i = 0; i < kR; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = 8 * h + (l >> 3);
      const uint32_t m = mw + 16u * i + (uint32_t)r;
      x_off[i][h] = (m < M ? m : M - 1) * K + 16u * (uint32_t)((l & 7) ^ lf(r));  // ragged tail: the last token
    }
  const uint32_t xr0 = 128u * lr + 16u * (uint32_t)((2 * lk) ^ lf(lr));
  const uint32_t xr1 = 128u * lr + 16u * (uint32_t)((2 * lk + 1) ^ lf(lr));
  const uint32_t x_lds = C::kWBytes + C::kXBytes * (uint32_t)w;
  const uint32_t sx_lds = C::kWBytes + C::kXBytes * kNW + 256u * (uint32_t)w;
  const uint32_t sx_tok = mw + (uint32_t)(l < 16 * kR ? l : 16 * kR - 1);
  const uint32_t sx_lane = (sx_tok < M ? sx_tok : M - 1) * 4u;
  // strip s lies in weight block b0 + sel(s)
  const uint32_t sub = strip0 & 7u;

  auto issue = [&](uint8_t* st, uint32_t kb) {
#pragma unroll
    for (int q = 0; q < C::kPW; ++q) buf_to_lds16(rw, st + w_lds[q], w_off[q], kb * (kPk ? kPackChunk : kBK));
#pragma unroll
    for (int i = 0; i < kR; ++i) {
      buf_to_lds16(rx, st + x_lds + 2048 * i, x_off[i][0], kb * kBK);
      buf_to_lds16(rx, st + x_lds + 2048 * i + 1024, x_off[i][1], kb * kBK);
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsx, (__attribute__((address_space(3))) void*)(st + sx_lds), 4,
                                             sx_lane, kb * M * 4u, 0, 0);
  };
  auto clampb = [&](uint32_t kb) { return kb < last ? kb : last; };  // past the end: a valid block, not folded

  // Every fragment a block's steps use, read from its stage into registers
  // one block ahead: the wave's X fragments, their sx factors (0 for a block
  // past the end: it then leaves acc unchanged bit for bit, as acc is never
  // -0; multiplying by 1 changes no scale), the block's weight-block scales and
  // the weight fragments of all kS strips.
  struct Frags {
    v8i_t xf[kR];
    float sxv[kR];
    float sw0, sw1;
    v8i_t wf[kS];
  };
  auto frag = [&](const uint8_t* p0, const uint8_t* p1) {
    const uint4 lo = *reinterpret_cast<const uint4*>(p0);
    const uint4 hi = *reinterpret_cast<const uint4*>(p1);
    return v8i_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  };
  auto read_frags = [&](const uint8_t* st, uint32_t kb, Frags& f) {
    const float live = kb < nkb ? 1.0f : 0.0f;
#pragma unroll
    for (int i = 0; i < kR; ++i) {
      f.xf[i] = frag(st + x_lds + 2048 * i + xr0, st + x_lds + 2048 * i + xr1);
      f.sxv[i] = reinterpret_cast<const float*>(st + sx_lds)[16 * i + lr] * live;
    }
    const uint32_t kc = clampb(kb);
    f.sw0 = swl[kc];
    f.sw1 = swl[(nb - 1u) * nkb + kc];
#pragma unroll
    for (int s = 0; s < kS; ++s) {
      const uint8_t* sp = st + 2048 * s;
      f.wf[s] = kPk ? frag(sp + 16 * l, sp + 1024 + 16 * l) : frag(sp + xr0, sp + xr1);
    }
  };

  // prologue: every stage filled (block j into stage j), block 0 published
  static_for<kD>([&](auto c) {
    issue(stage(c), clampb(decltype(c)::value));
    __builtin_amdgcn_sched_barrier(0);
  });
  wait_vmem_le<(kD - 1) * C::kG>();
  lds_barrier();
  Frags nxt;
  read_frags(ws0, 0, nxt);

  v4f_t acc[kR][kS];
#pragma unroll
  for (int i = 0; i < kR; ++i)
#pragma unroll
    for (int s = 0; s < kS; ++s) acc[i][s] = v4f_t{0.0f, 0.0f, 0.0f, 0.0f};
  // Steps q = kR s + i of a block (strip s, token sub-tile i) run from
  // registers: step q issues the MFMA of q and rescales the partial of q - 2
  // into acc, so two MFMAs separate every partial from its use.  At the block's
  // second step (at its only one when it has one MFMA) the wave waits for its
  // loads of the next block; the barrier publishes that block and, since every
  // wave's reads of this block's stage completed before it (the barrier waits
  // for the wave's LDS reads), frees this stage, which is refilled at once with
  // block kb + kD; then the next block's fragments are read into registers
  // while this block's remaining MFMAs run.  Scheduling barriers pin the order.
  constexpr int kQ = kR * kS;
  constexpr int kB = kQ >= 2 ? 1 : 0;  // the step that holds the barrier
  uint32_t c0 = 0;
#pragma clang loop unroll(disable)
  do {
    static_for<kD>([&](auto c) {
      constexpr int j = decltype(c)::value;
      const uint32_t kb = c0 + j;
      uint8_t* st = stage(c);
      const Frags cur = nxt;
      float swv[kS];
#pragma unroll
      for (int s = 0; s < kS; ++s) swv[s] = sub + (uint32_t)s >= 8u ? cur.sw1 : cur.sw0;
      v4f_t part[3];
      static_for<kQ + 2>([&](auto qc) {
        constexpr int q = decltype(qc)::value;
        constexpr int s = q / kR, i = q % kR;
        if constexpr (q < kQ) part[q % 3] = mfma_fp8(cur.wf[s], cur.xf[i]);
        if constexpr (q == kB) {
          // this wave's loads of block kb + 1 were issued before the kD - 2 later groups
          wait_vmem_le<(kD - 2) * C::kG>();
          lds_barrier();
          issue(st, clampb(kb + kD));
          read_frags(stage(std::integral_constant<int, (j + 1) % kD>{}), kb + 1, nxt);
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (q >= 2) {
          constexpr int qp = q - 2, ps = qp / kR, pi = qp % kR;
          const float sc = cur.sxv[pi] * swv[ps];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[pi][ps][e] = fmaf(part[qp % 3][e], sc, acc[pi][ps][e]);
        }
        __builtin_amdgcn_sched_barrier(0);
      });
    });
    c0 += kD;
  } while (c0 < nkb);
#pragma unroll
  for (int i = 0; i < kR; ++i) {
    const uint32_t m = mw + 16u * i + lr;
    if (m < M) {
#pragma unroll
      for (int s = 0; s < kS; ++s) {
        const uint32_t lo = f32_to_bf16_rne(acc[i][s][0]) | (f32_to_bf16_rne(acc[i][s][1]) << 16);
        const uint32_t hi = f32_to_bf16_rne(acc[i][s][2]) | (f32_to_bf16_rne(acc[i][s][3]) << 16);
        *reinterpret_cast<uint2*>(Y + (size_t)m * N + n0 + 16 * s + 4 * lk) = make_uint2(lo, hi);
      }
    }
  }
  // no direct-to-LDS load may still be in flight when the workgroup ends
  wait_vmem();
}

__global__ void fill_zero_u16(uint16_t* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

static hipError_t launch_zero(uint16_t* p, int64_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(fill_zero_u16, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

// grid rows: one per 16 kMT tokens (kMT = 1 with several rows runs each
// 16-token slice in waves of its own)
template <int kMT, int kW, int kS, bool kPk>
static void launch_decode_t(const uint8_t* A, const float* sa, const uint8_t* B, const float* sb,
                            uint32_t m, uint32_t n, uint32_t k, uint16_t* C, hipStream_t stream) {
  const dim3 grid(n / (16 * kS), (m + 16 * kMT - 1) / (16 * kMT));
  hipLaunchKernelGGL((gemm_fp8_decode_kernel<kMT, kW, kS, kPk>), grid, dim3(64 * kW), 0, stream, A, sa, B, sb, m,
                     n, k, C);
}

// kw is rounded to an instantiated value: at least kMT (one folding wave per
// token sub-tile) and with the parked partials within LDS.
template <int kMT, int kS, bool kPk>
static void launch_decode_ms(int kw, const uint8_t* A, const float* sa, const uint8_t* B, const float* sb,
                             uint32_t m, uint32_t n, uint32_t k, uint16_t* C, hipStream_t stream) {
  constexpr int kW2 = kMT > 2 ? kMT : 2;
  constexpr int kW8 = 8 * kMT * kS <= 64 ? 8 : (4 * kMT * kS <= 64 ? 4 : kW2);
  constexpr int kW16 = 16 * kMT * kS <= 64 ? 16 : kW8;
  constexpr int kW4 = 4 * kMT * kS <= 64 ? 4 : kW2;
  switch (kw) {
    case 1: launch_decode_t<kMT, 1, kS, kPk>(A, sa, B, sb, m, n, k, C, stream); break;
    case 2: launch_decode_t<kMT, kW2, kS, kPk>(A, sa, B, sb, m, n, k, C, stream); break;
    case 4: launch_decode_t<kMT, kW4, kS, kPk>(A, sa, B, sb, m, n, k, C, stream); break;
    case 8: launch_decode_t<kMT, kW8, kS, kPk>(A, sa, B, sb, m, n, k, C, stream); break;
    default: launch_decode_t<kMT, kW16, kS, kPk>(A, sa, B, sb, m, n, k, C, stream); break;
  }
}

template <int kMT, bool kPk>
static void launch_decode_m(int kw, int ks, const uint8_t* A, const float* sa, const uint8_t* B,
                            const float* sb, uint32_t m, uint32_t n, uint32_t k, uint16_t* C,
                            hipStream_t stream) {
  if (ks == 2) launch_decode_ms<kMT, 2, kPk>(kw, A, sa, B, sb, m, n, k, C, stream);
  else launch_decode_ms<kMT, 1, kPk>(kw, A, sa, B, sb, m, n, k, C, stream);
}

template <bool kPk>
static void launch_decode_p(int mt, int kw, int ks, const uint8_t* A, const float* sa, const uint8_t* B,
                            const float* sb, uint32_t m, uint32_t n, uint32_t k, uint16_t* C,
                            hipStream_t stream) {
  if (mt == 1) launch_decode_m<1, kPk>(kw, ks, A, sa, B, sb, m, n, k, C, stream);
  else if (mt == 2) launch_decode_m<2, kPk>(kw, ks, A, sa, B, sb, m, n, k, C, stream);
  else launch_decode_m<4, kPk>(kw, ks, A, sa, B, sb, m, n, k, C, stream);
}

// Decode FProp (M <= 64) with the launch shape chosen from the problem size.
// Strips per wave: 2 when there are at least 384 strips of 16 columns (each X
// fragment then serves two strips), else 1.  Waves per strip group (K-phases):
//   row-major weight: enough for about 1024 / mt streaming waves (a wave with
//     mt token sub-tiles does mt times the MFMA and X-load work per K-block),
//     or 2048 for long K, where a group's sequential chain is long;
//   packed weight: one (a lone wave streaming its strips' contiguous range
//     with no LDS fold was fastest at every 8B decode shape and M = 16 .. 64),
//     more only while there are fewer than 192 waves; over 16 rows the tokens
//     are split into grid rows of 16 or 32 (see below);
// at most 16, and at most one per two K-blocks.  Measured on the 8B decode
// shapes (K = 4096 and 12288, N = 4096 .. 24576, M = 1 .. 64).
static void launch_decode(bool packed, int64_t Mr, int64_t Nc, int64_t Kc, const uint8_t* A, const float* sa,
                          const uint8_t* B, const float* sb, uint16_t* C, hipStream_t stream) {
  const int64_t nkb = Kc / kBK, strips = Nc / 16;
  int mt = Mr <= 16 ? 1 : (Mr <= 32 ? 2 : 4);
  int ks = strips >= 384 ? 2 : 1;
  int kw = 16;
  if (packed) {
    // over 16 rows: two strips per wave from 256 strips, and the tokens in
    // slices of 16 (17 .. 32 rows with long K) or 32 that run in waves of their
    // own (grid rows), each slice's waves streaming the same weight range
    if (Mr > 16) {
      ks = strips >= 256 ? 2 : 1;
      mt = (Mr > 32 || nkb < 64) ? 2 : 1;
    }
    const int64_t waves = (strips / ks) * ((Mr + 16 * mt - 1) / (16 * mt));
    kw = 1;
    while (kw < 16 && waves * kw < 192 && 2 * kw <= (nkb + 1) / 2) kw *= 2;
  } else {
    const int64_t groups = strips / ks;
    const int64_t target = nkb >= 64 ? 2048 : 1024 / mt;
    while (kw > 1 && (groups * kw > target || kw > (nkb + 1) / 2)) kw /= 2;
  }
  if (kw > 1 && kw < mt) kw = mt;  // wave i folds token sub-tile i
  if (packed)
    launch_decode_p<true>(mt, kw, ks, A, sa, B, sb, (uint32_t)Mr, (uint32_t)Nc, (uint32_t)Kc, C, stream);
  else
    launch_decode_p<false>(mt, kw, ks, A, sa, B, sb, (uint32_t)Mr, (uint32_t)Nc, (uint32_t)Kc, C, stream);
}

template <bool kPk>
static bool launch_decode_ws(int r, int s, int nw, int occ, const uint8_t* A, const float* sa, const uint8_t* B,
                             const float* sb, uint32_t m, uint32_t n, uint32_t k, uint16_t* C, hipStream_t stream);
template <bool kPk>
static bool launch_fprop_ws(int64_t M, int64_t N, int64_t K, const uint8_t* A, const float* sa, const uint8_t* B,
                            const float* sb, uint16_t* C, hipStream_t stream);

// Rows Mr of A (rows of Kc bytes), their scales sa[kb * lds + row] (lds: the
// row count of the whole scale tensor, of which this launch may cover a row
// range), B and the output C [Mr][Nc]; every operand and the output within
// 32-bit byte offsets (launch_gemm splits larger problems into such ranges).
template <int kMode, int kOut>
static hipError_t launch_gemm_rows(const uint8_t* A, const float* sa, const uint8_t* B, const float* sb,
                                   int64_t Mr, int64_t Nc, int64_t Kc, int64_t lds, void* Cv, hipStream_t stream) {
  uint16_t* C = static_cast<uint16_t*>(Cv);
  // rollout batches (FProp, up to 256 tokens): the weight-sharing kernel where
  // launch_fprop_ws chooses it, else the weight-streaming decode kernel (up to
  // 64 tokens)
  if (kMode == kFprop && kOut == kOutBf16 && Mr <= 256 && lds == Mr && Nc * Kc < (int64_t(1) << 31) &&
      Mr * Kc < (int64_t(1) << 31)) {
    if (launch_fprop_ws<false>(Mr, Nc, Kc, A, sa, B, sb, C, stream)) return hipGetLastError();
    if (Mr <= 64) {
      launch_decode(false, Mr, Nc, Kc, A, sa, B, sb, C, stream);
      return hipGetLastError();
    }
  }
  const int64_t nkb = Kc / kBK;
  // the large-tile kernel works with 32-bit byte offsets; it needs >= 256
  // tiles to fill the chip
  const bool fits32 = (Mr + kLBM) * Kc < (int64_t(1) << 31) && Nc * Kc < (int64_t(1) << 31) &&
                      (Mr + kLBM) * Nc * (kOut == kOutBf16 ? 2 : 4) < (int64_t(1) << 31);
  const int64_t large_tiles = ((Mr + kLBM - 1) / kLBM) * (Nc / kLBN);
  if (Nc % kLBN == 0 && fits32 && large_tiles >= 256) {
    // A last round of at most half the CUs' tiles: when the full rounds are
    // whole rows of tiles, they run here and the remaining rows as a launch of
    // their own on the 128 x 128 kernel (two workgroups per CU, a quarter of
    // the work per tile); both kernels fold identically, so the output is
    // bitwise the single launch's (the 8B-layer QKV WGrad, 384 tiles: 486 ->
    // 430 us).
    const int64_t cus = device_cu_count() & ~7, per_row = Nc / kLBN;
    if (cus >= 8 && large_tiles > cus) {
      const int64_t tail = large_tiles % cus, full = large_tiles - tail;
      if (tail != 0 && 2 * tail <= cus && full % per_row == 0) {
        const int64_t main_rows = full / per_row * kLBM;
        const int64_t ob = kOut == kOutBf16 ? 2 : 4;
        const hipError_t e = launch_gemm_rows<kMode, kOut>(A, sa, B, sb, main_rows, Nc, Kc, lds, Cv, stream);
        if (e != hipSuccess) return e;
        return launch_gemm_rows<kMode, kOut>(A + main_rows * Kc, sa + main_rows, B, sb, Mr - main_rows, Nc, Kc, lds,
                                             static_cast<char*>(Cv) + main_rows * Nc * ob, stream);
      }
    }
    // FProp and DGrad: one workgroup per CU looping over tiles when the block
    // count is even (the next tile's first block then lands in stage 0, where
    // a tile starts); otherwise one workgroup per tile.
    int64_t grid = large_tiles;
    if (kMode != kWgrad && nkb % 2 == 0) {
      const int64_t cus = device_cu_count() & ~7;
      if (cus >= 8 && cus < grid) grid = cus;
    }
    hipLaunchKernelGGL((gemm_fp8_large_kernel<kMode, kOut>), dim3((unsigned)grid), dim3(kLThreads), 0, stream,
                       A, sa, B, sb, (uint32_t)Mr, (uint32_t)Nc, (uint32_t)Kc, (uint32_t)lds, Cv, (float*)nullptr);
    return hipGetLastError();
  }
  // the medium-tile kernel (the caller guarantees 32-bit byte offsets): four
  // stages when there is at most one tile per CU (measured at M = 256: the
  // 8B QKV projection, 96 tiles, 36 -> 29 us), two stages and two workgroups
  // per CU otherwise (with 384 tiles, two rounds of the four-stage kernel
  // took 60 us against 45 us for one round of two per CU: a CU's loads in
  // flight are capped, so more CUs pulling data beats deeper prefetch)
  const int64_t tiles = ((Mr + kMBM - 1) / kMBM) * (Nc / kMBN);
  if (tiles <= (int64_t)device_cu_count())
    hipLaunchKernelGGL((gemm_fp8_med_kernel<kMode, kOut, 4>), dim3((unsigned)tiles), dim3(kMThreads), 0, stream,
                       A, sa, B, sb, (uint32_t)Mr, (uint32_t)Nc, (uint32_t)Kc, (uint32_t)lds, Cv);
  else
    hipLaunchKernelGGL((gemm_fp8_med_kernel<kMode, kOut, 2>), dim3((unsigned)tiles), dim3(kMThreads), 0, stream,
                       A, sa, B, sb, (uint32_t)Mr, (uint32_t)Nc, (uint32_t)Kc, (uint32_t)lds, Cv);
  return hipGetLastError();
}

// Row ranges of an Mr-row problem whose A rows (rb bytes each) and output rows
// (ob bytes each) must stay below 2^31 bytes per launch, with one 256-row tile
// of ragged rows: nearly equal ranges of a multiple of 256 rows (each above
// 256 rows whenever the problem is split, so all take the tile kernels).
struct RowChunks {
  int64_t chunk, count;
};
static RowChunks row_chunks(int64_t Mr, int64_t rb, int64_t ob) {
  const int64_t lim = int64_t(1) << 31;
  int64_t cap = (lim - 1) / (rb > ob ? rb : ob) - kLBM;
  cap -= cap % kLBM;
  if (Mr <= cap) return {Mr, 1};
  const int64_t n = (Mr + cap - 1) / cap;
  int64_t chunk = (Mr + n - 1) / n;
  chunk = (chunk + kLBM - 1) / kLBM * kLBM;
  if (chunk > cap) chunk = cap;
  return {chunk, (Mr + chunk - 1) / chunk};
}

// C [Mr][Nc] = the block-scaled product of A [Mr][Kc] and B: beyond 32-bit
// byte offsets, one launch per row range (rows are independent, and every
// range runs a kernel with the sequential K fold, so the result is the one a
// single launch would give).  The caller guarantees that B, and a range of
// 512 rows of A and of C, fit 32-bit offsets.
template <int kMode, int kOut = kOutBf16>
static hipError_t launch_gemm(const uint8_t* A, const float* sa, const uint8_t* B, const float* sb,
                              int64_t Mr, int64_t Nc, int64_t Kc, void* Cv,
                              hipStream_t stream) {
  if (Mr == 0 || Nc == 0) return hipSuccess;
  // an empty contraction: the product is zero (nothing to add for kOutF32Add)
  if (Kc == 0) {
    if (kOut == kOutF32Add) return hipSuccess;
    return launch_zero(static_cast<uint16_t*>(Cv), Mr * Nc * (kOut == kOutF32 ? 2 : 1), stream);
  }
  const int64_t ob = kOut == kOutBf16 ? 2 : 4;
  const RowChunks rc = row_chunks(Mr, Kc, Nc * ob);
  for (int64_t i = 0; i < rc.count; ++i) {
    const int64_t m0 = i * rc.chunk, mc = (Mr - m0 < rc.chunk) ? Mr - m0 : rc.chunk;
    const hipError_t e = launch_gemm_rows<kMode, kOut>(A + m0 * Kc, sa + m0, B, sb, mc, Nc, Kc, Mr,
                                                       static_cast<char*>(Cv) + m0 * Nc * ob, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// K == 0: the gate+up output is zero, so h = silu(0) * 0 = 0: codes 0, scales 1
__global__ void fill_swiglu_empty(uint8_t* __restrict__ q, int64_t nq, float* __restrict__ s, int64_t ns) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nq; i += (int64_t)gridDim.x * blockDim.x)
    q[i] = 0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < ns; i += (int64_t)gridDim.x * blockDim.x)
    s[i] = 1.0f;
}

hipError_t launch_gemm_fprop_swiglu_quant(const uint8_t* qx, const float* sx, const uint8_t* qw, const float* sw,
                                          int64_t M, int64_t N, int64_t K, uint8_t* q, float* s,
                                          hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  if (K == 0) {
    const int64_t nq = M * (N / 2);
    int64_t blocks = (nq + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(fill_swiglu_empty, dim3((unsigned)blocks), dim3(256), 0, stream, q, nq, s, nq / kGroup);
    return hipGetLastError();
  }
  // 256 x 256 tiles of (rows, gate block + up block); one workgroup per CU
  // looping over the tiles when the block count is even, as FProp; one launch
  // per row range beyond 32-bit offsets (as launch_gemm)
  const int64_t nkb = K / kBK, I = N / 2;
  const RowChunks rc = row_chunks(M, K, I);
  for (int64_t i = 0; i < rc.count; ++i) {
    const int64_t m0 = i * rc.chunk, mc = (M - m0 < rc.chunk) ? M - m0 : rc.chunk;
    const int64_t tiles = ((mc + kLBM - 1) / kLBM) * (N / kLBN);
    int64_t grid = tiles;
    if (nkb % 2 == 0) {
      const int64_t cus = device_cu_count() & ~7;
      if (cus >= 8 && cus < grid) grid = cus;
    }
    hipLaunchKernelGGL((gemm_fp8_large_kernel<kFprop, kOutSwiglu>), dim3((unsigned)grid), dim3(kLThreads), 0,
                       stream, qx + m0 * K, sx + m0, qw, sw, (uint32_t)mc, (uint32_t)N, (uint32_t)K, (uint32_t)M,
                       (void*)(q + m0 * I), s + m0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
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

hipError_t launch_gemm_wgrad_f32(const uint8_t* qdyt, const float* sdyt, const uint8_t* qxt,
                                 const float* sxt, int64_t M, int64_t N, int64_t K, float* dw,
                                 bool accumulate, hipStream_t stream) {
  if (accumulate) return launch_gemm<kWgrad, kOutF32Add>(qdyt, sdyt, qxt, sxt, N, K, M, dw, stream);
  return launch_gemm<kWgrad, kOutF32>(qdyt, sdyt, qxt, sxt, N, K, M, dw, stream);
}

// ---------------------------------------------------------------------------
// FProp with K split across workgroups (rollout batches of 17 .. 256 rows),
// through a workspace the caller provides.  Below one 128 x 128 tile per CU
// (the 8B QKV and down projections of a 256-token rollout batch: 96 and 64
// tiles) most CUs idle and each tile's sequential chain of K-blocks waits on
// memory; splitting K into S equal contiguous ranges gives S workgroups per
// tile.  For 17 .. 64 rows it also reads X once per 128 columns instead of
// once per 16 (the decode kernel's strips).  Share s folds its
// blocks in ascending order, acc = fma(P_kb, fl32(sx * sw), acc) from zero,
// and writes the fp32 partial to slice s of the workspace; the reduction adds
// the S partials of each output in share order, ((p0 + p1) + p2) + ..., and
// rounds to bf16.  Deterministic, and the same for a row whatever batch of
// this size range holds it when S is the same, but not the single sequential
// fold of gemm_fprop.
constexpr int kSplitTargetCUs = 256;  // MI355X; fixed so the workspace size needs no device query

int fprop_split_count(int64_t M, int64_t N, int64_t K) {
  if (M > 256 || N % kMBN != 0 || K % kBK != 0) return 1;
  const int64_t tiles = ((M + kMBM - 1) / kMBM) * (N / kMBN);
  const int64_t nkb = K / kBK;
  if (tiles >= kSplitTargetCUs) return 1;
  // Up to 16 rows the weight-streaming decode kernel is faster; from 17 to 32
  // rows only long contractions gain (its waves re-read X, M x K bytes, once
  // per 16-column strip).  Measured at the 8B decode shapes, split against the
  // decode kernel: M = 16: QKV 13.6 / 11.1 us, gate+up 30.0 / 28.2, down 18.1 /
  // 18.2; M = 32: down (K = 12288) 19.3 / 25.0, the others 5-10 % slower;
  // M = 64: QKV 16.6 / 22.8, gate+up 34.0 / 39.3, down 21.6 / 37.8.
  if (M <= 16 || (M <= 32 && nkb < 64)) return 1;
  // the most shares that keep at most two workgroups per CU and at least four
  // K-blocks per share, and divide the block count
  int best = 1;
  for (int64_t s = 2; s <= nkb / 4 && tiles * s <= 2 * kSplitTargetCUs; ++s)
    if (nkb % s == 0) best = (int)s;
  return best;
}

// y[i] = bf16(((p0[i] + p1[i]) + p2[i]) + ...), eight outputs per thread
__global__ __launch_bounds__(256) void splitk_reduce_bf16_kernel(const float* __restrict__ ws, int splits,
                                                                 int64_t n, uint16_t* __restrict__ y) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i >= n) return;
  float4 a = *reinterpret_cast<const float4*>(ws + i);
  float4 b = *reinterpret_cast<const float4*>(ws + i + 4);
  for (int sp = 1; sp < splits; ++sp) {
    const float4 c = *reinterpret_cast<const float4*>(ws + sp * n + i);
    const float4 d = *reinterpret_cast<const float4*>(ws + sp * n + i + 4);
    a.x += c.x; a.y += c.y; a.z += c.z; a.w += c.w;
    b.x += d.x; b.y += d.y; b.z += d.z; b.w += d.w;
  }
  uint4 o;
  o.x = f32_to_bf16_rne(a.x) | (f32_to_bf16_rne(a.y) << 16);
  o.y = f32_to_bf16_rne(a.z) | (f32_to_bf16_rne(a.w) << 16);
  o.z = f32_to_bf16_rne(b.x) | (f32_to_bf16_rne(b.y) << 16);
  o.w = f32_to_bf16_rne(b.z) | (f32_to_bf16_rne(b.w) << 16);
  *reinterpret_cast<uint4*>(y + i) = o;
}

int64_t fprop_splitk_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  const int s = fprop_split_count(M, N, K);
  return s > 1 ? (int64_t)s * M * N * 4 : 0;
}

hipError_t launch_gemm_fprop_splitk(const uint8_t* qx, const float* sx, const uint8_t* qw, const float* sw,
                                    int64_t M, int64_t N, int64_t K, uint16_t* y, float* ws,
                                    hipStream_t stream) {
  const int s = fprop_split_count(M, N, K);
  if (s <= 1) return launch_gemm_fprop(qx, sx, qw, sw, M, N, K, y, stream);
  const int64_t tiles = ((M + kMBM - 1) / kMBM) * (N / kMBN);
  const dim3 grid((unsigned)tiles, (unsigned)s);
  if (tiles * s <= kSplitTargetCUs)
    hipLaunchKernelGGL((gemm_fp8_med_kernel<kFprop, kOutF32, 4>), grid, dim3(kMThreads), 0, stream, qx, sx, qw,
                       sw, (uint32_t)M, (uint32_t)N, (uint32_t)K, (uint32_t)M, (void*)ws);
  else
    hipLaunchKernelGGL((gemm_fp8_med_kernel<kFprop, kOutF32, 2>), grid, dim3(kMThreads), 0, stream, qx, sx, qw,
                       sw, (uint32_t)M, (uint32_t)N, (uint32_t)K, (uint32_t)M, (void*)ws);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = M * N;  // a multiple of 128
  hipLaunchKernelGGL(splitk_reduce_bf16_kernel, dim3((unsigned)((n / 8 + 255) / 256)), dim3(256), 0, stream, ws, s,
                     n, y);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Library-owned split-K workspace of gemm_fprop_splitk_noalloc, the variant of
// gemm_fprop_splitk for callers that cannot allocate device memory (code under
// HIP graph capture, serving loops).  Every device the library runs on holds
// its own copy of this array until the process ends, and every call on that
// device shares it: calls that overlap on one device race.  The K-share kernels
// write every partial the reduction reads, so nothing needs clearing between
// calls.  In host code `scratch` names a host-side stand-in, never the device
// memory: kernels get the address from scratch_address() only.
constexpr int64_t kNoAllocScratchBytes = int64_t(32) << 20;
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / 4];

// This device's copy of `scratch`: looked up with hipGetSymbolAddress on the
// first call on each device (with that device current) and kept per device.
static hipError_t scratch_address(float** out) {
  static std::mutex mu;
  static void* ptrs[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    ptrs[dev] = p;
  }
  *out = static_cast<float*>(ptrs[dev]);
  return hipSuccess;
}

int64_t fprop_noalloc_scratch_bytes() { return kNoAllocScratchBytes; }

hipError_t launch_gemm_fprop_splitk_noalloc(const uint8_t* qx, const float* sx, const uint8_t* qw,
                                            const float* sw, int64_t M, int64_t N, int64_t K, uint16_t* y,
                                            hipStream_t stream) {
  float* ws = nullptr;
  if (fprop_splitk_workspace_bytes(M, N, K) > 0) {
    const hipError_t e = scratch_address(&ws);
    if (e != hipSuccess) return e;
  }
  return launch_gemm_fprop_splitk(qx, sx, qw, sw, M, N, K, y, ws, stream);
}

// ---------------------------------------------------------------------------
// Rollout-packed weight codes.  A rollout batch re-reads the whole FP8 weight
// at every decode step, and at that step the weight stream is the kernel's
// whole cost.  Row-major [N][K] codes make each wave pull 128 bytes from each of
// 16 rows 4 KB apart per K-block, which keeps HBM at about 4.3 TB/s however the
// loads are grouped (measured: 16 to 1024 consecutive bytes per row and load,
// 1 to 8 K-blocks per step); the same bytes stored so that each wave reads one
// contiguous range reach about 5.5 TB/s.  The packed copy holds the same
// codes in the order the decode kernel's lanes consume them:
//   qwp[((t * nkb + kb) * 2 + h) * 1024 + 16 l + b] = qw[16 t + (l & 15)][128 kb + 32 (l >> 4) + 16 h + b]
// (strip t of 16 rows, K-block kb, half h, lane l, byte b): lane l's two
// 16-byte loads at 16 l and 1024 + 16 l of a chunk are the 32 consecutive
// codes of row l & 15, K-slice l >> 4 that the 16x16x128 MFMA takes from it.
// A permutation of bytes only: the packed FProp's products, scales and fold
// are those of the row-major decode kernel, bit for bit.
__global__ __launch_bounds__(256) void pack_weight_rollout_kernel(const uint8_t* __restrict__ qw, uint64_t N,
                                                                  uint64_t K, uint8_t* __restrict__ qwp) {
  const uint64_t nkb = K / kBK, units = N * K / 16;  // 16-byte units of the packed copy
  for (uint64_t u = (uint64_t)blockIdx.x * 256 + threadIdx.x; u < units; u += (uint64_t)gridDim.x * 256) {
    const uint64_t l = u & 63, h = (u >> 6) & 1, c = u >> 7;
    const uint64_t kb = c % nkb, t = c / nkb;
    const uint64_t src = (16 * t + (l & 15)) * K + kBK * kb + 32 * (l >> 4) + 16 * h;
    *reinterpret_cast<uint4*>(qwp + 16 * u) = *reinterpret_cast<const uint4*>(qw + src);
  }
}

hipError_t launch_pack_weight_rollout(const uint8_t* qw, int64_t N, int64_t K, uint8_t* qwp, hipStream_t stream) {
  const int64_t units = N * K / 16;
  if (units == 0) return hipSuccess;
  int64_t blocks = (units + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(pack_weight_rollout_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, qw, (uint64_t)N,
                     (uint64_t)K, qwp);
  return hipGetLastError();
}

template <int kR, int kS, int kNW, bool kPk, int kOcc = 1>
static void launch_decode_ws_t(const uint8_t* A, const float* sa, const uint8_t* B, const float* sb, uint32_t m,
                               uint32_t n, uint32_t k, uint16_t* C, hipStream_t stream) {
  constexpr uint32_t tm = DecodeWsCfg<kR, kS, kNW, kOcc>::kTM;
  const uint32_t grid = (n / (16u * kS)) * ((m + tm - 1) / tm);
  hipLaunchKernelGGL((gemm_fp8_decode_ws_kernel<kR, kS, kNW, kPk, kOcc>), dim3(grid), dim3(64 * kNW), 0, stream, A,
                     sa, B, sb, m, n, k, C);
}

// The weight-sharing kernel's instantiated shapes (tokens per wave / 16,
// strips, waves, workgroups per CU); false for any other.
template <bool kPk>
static bool launch_decode_ws(int r, int s, int nw, int occ, const uint8_t* A, const float* sa, const uint8_t* B,
                             const float* sb, uint32_t m, uint32_t n, uint32_t k, uint16_t* C, hipStream_t stream) {
#define JETFP8_WS(R, S, NW, OCC)                                              \
  if (r == R && s == S && nw == NW && occ == OCC) {                           \
    launch_decode_ws_t<R, S, NW, kPk, OCC>(A, sa, B, sb, m, n, k, C, stream); \
    return true;                                                              \
  }
  JETFP8_WS(1, 6, 4, 2) JETFP8_WS(2, 6, 4, 1) JETFP8_WS(2, 6, 4, 2) JETFP8_WS(1, 2, 4, 1) JETFP8_WS(1, 1, 4, 1)
  JETFP8_WS(1, 4, 4, 2) JETFP8_WS(1, 3, 4, 2) JETFP8_WS(1, 2, 4, 2) JETFP8_WS(1, 1, 4, 2)
  JETFP8_WS(2, 4, 4, 2) JETFP8_WS(2, 3, 4, 2) JETFP8_WS(2, 2, 4, 2) JETFP8_WS(2, 1, 4, 2)
#undef JETFP8_WS
  return false;
}

// The weight-sharing kernel's launch shape for 33 .. 256 rows, or false where
// it is not the choice (up to 32 rows, and for the packed weight 33 .. 64 rows
// with more than 64 K-blocks: the streaming decode kernel).  The shape:
//   at least 1536 strips of 16 columns, a multiple of 6: 6 strips per
//     workgroup of 4 waves; up to 64 rows one token group of 16 tokens per
//     wave, two workgroups per CU; 65 .. 128 rows one group of 32 per wave,
//     one workgroup per CU; over 128 rows groups of 128 rows, two per CU
//     (512 workgroups for the 8B gate+up projection at 256 tokens);
//   otherwise, 33 .. 64 rows: 4 waves of 16 tokens on 2 strips (1 for long
//     contractions); over 64 rows: token groups of 64 rows (128 over 128 rows
//     when K is at most 64 K-blocks) with the most strips per workgroup
//     (6, 4, 3, 2, 1) that still give 256 workgroups, two workgroups per CU.
// Two workgroups per CU split the LDS, so each holds fewer K-blocks in flight
// (2 - 4 instead of 3 - 8), and one computes while the other waits at its
// block barrier.  Measured on the 8B rollout shapes (QKV, gate+up, down at
// 32 .. 256 rows, HIP-graph replays over 4 rotated weights): from 65 rows
// 1.0-2.0x faster than the 128 x 128 kernel and the split-K FProp at every
// shape; two workgroups per CU gained 4-12 % at 256 tokens and 10 % for
// gate+up at 64, and lost 9 % for gate+up at 128.
template <bool kPk>
static bool launch_fprop_ws(int64_t M, int64_t N, int64_t K, const uint8_t* A, const float* sa, const uint8_t* B,
                            const float* sb, uint16_t* C, hipStream_t stream) {
  const int64_t strips = N / 16, nkb = K / kBK;
  if (M <= 32 || M > 256 || nkb > kWsMaxKb) return false;
  int r = 1, s = 1, occ = 1;
  if (strips % 6 == 0 && strips / 6 >= 256) {
    s = 6;
    r = M <= 64 ? 1 : 2;
    occ = (M <= 64 || M > 128) ? 2 : 1;
  } else if (M <= 64) {
    // long contractions: the packed weight streams fastest through the decode
    // kernel, the row-major one through this kernel with one strip per workgroup
    if (nkb > 64) {
      if (kPk) return false;
    } else {
      s = 2;
    }
  } else {
    occ = 2;
    r = (M > 128 && nkb <= 64) ? 2 : 1;
    const int64_t tg = (M + 64 * r - 1) / (64 * r);
    for (int c : {6, 4, 3, 2}) {
      if (strips % c == 0 && (strips / c) * tg >= 256) {
        s = c;
        break;
      }
    }
  }
  return launch_decode_ws<kPk>(r, s, 4, occ, A, sa, B, sb, (uint32_t)M, (uint32_t)N, (uint32_t)K, C, stream);
}

// Packed FProp (up to 256 rows), sequential fold: the weight-sharing kernel
// where launch_fprop_ws chooses it, else the decode kernel (launch_decode's
// packed rule; it also takes contractions of more than 512 K-blocks, whose
// weight-block scales would not fit the weight-sharing kernel's LDS copy).
hipError_t launch_gemm_fprop_packed(const uint8_t* qx, const float* sx, const uint8_t* qwp, const float* sw,
                                    int64_t M, int64_t N, int64_t K, uint16_t* y, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  if (K == 0) return launch_zero(y, M * N, stream);
  if (launch_fprop_ws<true>(M, N, K, qx, sx, qwp, sw, y, stream)) return hipGetLastError();
  launch_decode(true, M, N, K, qx, sx, qwp, sw, y, stream);
  return hipGetLastError();
}

}  // namespace jetfp8
