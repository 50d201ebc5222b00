/*
 * jetfp8.h -- C ABI of the MI355X (gfx950) FP8 linear-layer library.
 *
 * The operations are those of the mixed-granularity FP8 linear layer of
 * Jet-RL ("Jet-RL: Enabling On-Policy FP8 Reinforcement Learning with Unified
 * Training and Rollout Precision Flow", arXiv 2601.14243).  Citations name the
 * page and its section:
 *   [P3-FP8]   paper.rainbus.top summary, section "FP8 量化 (E4M3 格式)"
 *              (E4M3, largest value 448, S = max|X| / 448, X_hat = [X / S]);
 *   [P3-GRAN]  same page, section "Per-group / Per-block 量化粒度"
 *              (1x128 groups for activations and gradients, 128x128 blocks
 *              for weights);
 *   [P3-LAYOUT] same page, section "GEMM 量化布局（Row-wise 与 Column-wise）"
 *              (FProp Y = X W^T, WGrad dW = dY^T X, DGrad dX = dY W);
 *   [P3-CORE]  same page, section "核心方法" (all three GEMMs in FP8;
 *              FProp (1x128)x(128x128), DGrad the same, WGrad
 *              (1x128)x(128x1));
 *   [P3-STEPS] same page, section "方法步骤详情" (steps 1-5: quantisation
 *              granularity, forward GEMM, FP8 activation saving, backward with
 *              BF16 dY and the 1x128 -> 128x1 requantisation, fused RMSNorm);
 *   [P3-NOVEL] same page, section "技术新颖性" (forward saves 1x128, backward
 *              needs 128x1);
 *   [P3-RESULTS] same page, section "实验结果" (the rollout speed-up of FP8,
 *              1.33x on the 32B model);
 *   [P3-WEAK]  same page, section "独立分析的弱点" (8B rollout is bound by
 *              memory traffic rather than arithmetic).
 *
 * Conventions common to every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers to contiguous row-major arrays.
 *   bf16 values are passed as uint16_t bit patterns; FP8 values as uint8_t
 *   OCP E4M3FN bit patterns (0x7E = 448; 0x7F/0xFF are NaN and never
 *   produced); scales are IEEE fp32.
 * - A 1x128-grouped tensor Q[R][C] carries scales S[C/128][R]: S[g][r] scales
 *   elements r*C + 128*g ... r*C + 128*g + 127 ("group-major").  A 128x128
 *   blocked weight Q[N][K] carries S[N/128][K/128].
 * - The cast is round-to-nearest-even to the nearest E4M3 value, saturating
 *   at +-448, sign of zero kept.  S = amax / 448 is an IEEE fp32 division;
 *   S = 1 when that quotient is 0 (amax == 0, or a nonzero amax of at most
 *   448 * 2^-150, which only the fp32 values inside rmsnorm_quant and
 *   requant_transpose_128x1 can reach; the group's codes are then signed
 *   zeros).  q = cast(fl32(x / S)).  Quantiser outputs are bit-exact
 *   functions of their inputs.
 * - GEMMs form each 128-deep block product as one fp32 partial, multiply it
 *   by the product of the two operands' fp32 scales for that block, add it to
 *   an fp32 accumulator, and round the result to bf16 (nearest even);
 *   gemm_wgrad_f32 returns the fp32 accumulator itself.  The block partial is
 *   not the exact sum of its 128 products: the gfx950 FP8 matrix instruction
 *   adds each 32-product slice with reduced internal precision, so products
 *   below about 2^-14 of the largest in their slice can be lost.  Accuracy
 *   contract, with Yref the fp64 product of the dequantised operands:
 *   ||Y - bf16(Yref)||_F <= 1e-3 ||Yref||_F and, elementwise,
 *   |Y - bf16(Yref)| <= ulp_bf16(Yref) + 1e-3 rms(Yref), for codes that
 *   quantise bell-shaped data (activations, weights, gradients: what the
 *   quantisers produce).  For arbitrary codes (every finite code equally
 *   likely) the normwise bound holds and the elementwise one widens by the
 *   slice truncation, 2^-9 sum_k |a_k b_k| (where large products cancel, the
 *   lost small products can exceed 1e-3 rms).
 * - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *   enqueues work on it and returns; the caller keeps the buffers alive until
 *   the stream has reached them.
 * - Ownership: the caller allocates and frees every buffer.  The library never
 *   allocates, frees or retains device memory and keeps no pointer after a call
 *   returns.
 * - Errors: shapes and pointers are checked on the host before anything is
 *   enqueued; an invalid call returns a nonzero status and writes nothing.
 *   Requirements: every pointer 16-byte aligned (except when its tensor is
 *   empty); outputs must not overlap inputs or each other; sizes >= 0 and at
 *   most 2^31 - 1 per dimension; the divisibility rules stated per function.
 *   A status of JETFP8_ELAUNCH reports a HIP error from the enqueue itself.
 * - GEMMs address operands with 32-bit byte offsets per launch.  A GEMM whose
 *   row operand or output does not fit runs as several launches over row
 *   ranges (the rows of X, dY and the output for FProp and DGrad, the output
 *   features of dY^T and dW for WGrad), with the same result as one launch:
 *   the rows are independent and each range folds K in the same order.  What
 *   must fit is the column operand (the weight [N][K] for FProp and DGrad, the
 *   128x1-requantised X^T [K][M] for WGrad: below 2^31 bytes) and 512 rows of
 *   the row operand and of the output; a call beyond that returns
 *   JETFP8_EUNSUPPORTED and writes nothing.
 * - Inputs must be finite (NaN/Inf are outside the contract; the kernels do
 *   not hang on them, but the result is unspecified).
 * - Identical inputs give bitwise identical outputs (no atomics, no split-K
 *   races).  Entry points are reentrant and thread-safe.
 */
#ifndef JETFP8_H
#define JETFP8_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  JETFP8_OK = 0,
  JETFP8_EINVAL = 1,       /* bad shape (negative, not a multiple of 128, too large) */
  JETFP8_EALIGN = 2,       /* a pointer is not 16-byte aligned */
  JETFP8_ENULL = 3,        /* a required pointer is NULL */
  JETFP8_EALIAS = 4,       /* an output overlaps an input or another output */
  JETFP8_EUNSUPPORTED = 5, /* valid request this build does not implement */
  JETFP8_ELAUNCH = 6       /* HIP reported an error when enqueuing */
};

/* Human-readable name of a status code (static storage; never NULL). */
const char* jetfp8_status_string(int status);

/*
 * quantize_act_1x128 -- 1x128 per-group E4M3 quantisation of an activation or
 * a gradient [P3-FP8], [P3-GRAN], [P3-STEPS] steps 1, 2 and 4.
 *   x : bf16 [M][K] input.
 *   q : u8   [M][K] output codes.
 *   s : f32  [K/128][M] output scales (group-major).
 * K % 128 == 0; M >= 0 (any M).  M == 0 or K == 0 is a no-op.
 */
int quantize_act_1x128(const uint16_t* x, int64_t M, int64_t K, uint8_t* q, float* s,
                       void* stream);

/*
 * quantize_weight_128x128 -- 128x128 per-block E4M3 quantisation of a weight
 * [P3-FP8], [P3-GRAN], [P3-STEPS] step 1.  One output object serves FProp,
 * DGrad (read transposed, [P3-STEPS] step 4) and rollout.
 *   w : bf16 [N][K] input (BF16 master weight, [P3-CORE]).
 *   q : u8   [N][K] output codes.
 *   s : f32  [N/128][K/128] output block scales.
 * N % 128 == 0 and K % 128 == 0.
 */
int quantize_weight_128x128(const uint16_t* w, int64_t N, int64_t K, uint8_t* q, float* s,
                            void* stream);

/*
 * rmsnorm_quant -- fused RMSNorm + 1x128 quantisation ([P3-STEPS] step 5
 * names a fused RMSNorm kernel; the formula is the standard RMSNorm in fp32):
 *   ss  = fp32 pairwise-tree sum over the row of x*x (adjacent pairs, level by
 *         level; equivalently the row zero-padded to a power of two);
 *   inv = fl32(1 / fl32(sqrt(fl32(fl32(ss / K) + eps))));
 *   y   = fl32(fl32(x * inv) * gamma);  y is then quantised as in
 *         quantize_act_1x128, with no intermediate bf16 rounding.
 *   x : bf16 [M][K]; gamma : bf16 [K]; eps : fp32.
 *   q : u8 [M][K]; s : f32 [K/128][M].
 * K % 128 == 0 and 0 < K <= 65536; M >= 0.
 */
int rmsnorm_quant(const uint16_t* x, const uint16_t* gamma, int64_t M, int64_t K, float eps,
                  uint8_t* q, float* s, void* stream);

/*
 * rmsnorm_quant_rstd -- rmsnorm_quant that also saves, for the backward, the
 * per-row factor it multiplied by:
 *   rstd[m] = inv = fl32(1 / fl32(sqrt(fl32(fl32(ss / K) + eps))))
 *   rstd : f32 [M] output.  q and s are bitwise those of rmsnorm_quant.
 * Same shape rules as rmsnorm_quant.
 */
int rmsnorm_quant_rstd(const uint16_t* x, const uint16_t* gamma, int64_t M, int64_t K, float eps,
                       uint8_t* q, float* s, float* rstd, void* stream);

/*
 * rmsnorm_backward -- gradients of the RMSNorm of rmsnorm_quant for an
 * upstream gradient dy (the FP8 linear's DGrad output).  The pages train
 * through the fused RMSNorm ([P3-STEPS] step 5) without stating its formula;
 * these are the derivatives of the standard RMSNorm y = x * gamma * rstd:
 *   c[m]      = (1/K) sum_k gamma[k] * dy[m][k] * x[m][k]
 *   dx[m][k]  = rstd[m] * (gamma[k] * dy[m][k] - x[m][k] * rstd[m]^2 * c[m])
 *   dgamma[k] = sum_m dy[m][k] * x[m][k] * rstd[m]
 * evaluated in fp32 (dx rounded to bf16, nearest even; dgamma fp32), with a
 * fixed summation order: identical inputs give identical bits.
 *   x, dy : bf16 [M][K]; gamma : bf16 [K]; rstd : f32 [M] (from
 *           rmsnorm_quant_rstd on the same x, gamma, eps).
 *   dx : bf16 [M][K] output; dgamma : f32 [K] output (zeros when M == 0).
 *   workspace : f32 scratch of rmsnorm_backward_workspace_bytes(M, K) bytes,
 *           owned by the caller (its contents on entry are ignored).
 * K % 128 == 0 and 0 < K <= 24576; M >= 0.
 */
int64_t rmsnorm_backward_workspace_bytes(int64_t M, int64_t K); /* -1 for an invalid shape */
int rmsnorm_backward(const uint16_t* x, const uint16_t* gamma, const float* rstd, const uint16_t* dy,
                     int64_t M, int64_t K, uint16_t* dx, float* dgamma, float* workspace, void* stream);

/*
 * swiglu_quant -- SwiGLU of the gate+up projection's output fused with the
 * 1x128 quantisation of the down projection's input ([P3-CORE] on fusing the
 * quantisation into the neighbouring kernels, [P3-FP8], [P3-GRAN]).  The pages
 * give no formula for SiLU; it is read as the standard one with an exactly
 * specified fp32 evaluation:
 *   gate = y[m][i], up = y[m][I + i]   (y = [gate | up], bf16 [M][2I])
 *   E = the fp32 value nearest to e^-gate (+inf past the fp32 range)
 *   silu = fl32(gate / fl32(1 + E));  h = fl32(silu * up)
 *   (q, s) = the 1x128 quantisation of h, as quantize_act_1x128 does on these
 *            fp32 values (no bf16 rounding of h).
 *   y : bf16 [M][2I] input.  q : u8 [M][I]; s : f32 [I/128][M] outputs.
 * I % 128 == 0; M >= 0.  M == 0 or I == 0 is a no-op.  Bit-exact.  As with
 * non-finite inputs, an h that overflows fp32 (|silu * up| >= 2^128) is
 * outside the contract.
 */
int swiglu_quant(const uint16_t* y, int64_t M, int64_t I, uint8_t* q, float* s, void* stream);

/*
 * requant_transpose_128x1 -- requantise a saved 1x128 FP8 tensor into 128x1
 * groups along its rows (the token dimension) and store it transposed
 * ([P3-STEPS] steps 3-4, [P3-NOVEL]).  Used on the saved (QX, SX) and on
 * (QdY, SdY) to feed gemm_wgrad.
 *   v[m][k] = fl32(decode(q[m][k]) * s[k/128][m]);
 *   for each column k and 128-row block mb: S' = amax / 448 (1 if that is 0),
 *   qt[k][m] = cast(fl32(v[m][k] / S')), st[mb][k] = S'.
 *   q : u8 [M][K]; s : f32 [K/128][M].
 *   qt : u8 [K][M]; st : f32 [M/128][K].
 * M % 128 == 0 and K % 128 == 0.
 */
int requant_transpose_128x1(const uint8_t* q, const float* s, int64_t M, int64_t K, uint8_t* qt,
                            float* st, void* stream);

/*
 * gemm_fprop -- forward GEMM Y = X W^T with (1x128) x (128x128) scaling
 * ([P3-LAYOUT], [P3-CORE], [P3-STEPS] step 2):
 *   Y[m][n] = sum_kb sx[kb][m] * sw[n/128][kb] * sum_{k in kb} qx[m][k] * qw[n][k].
 *   qx : u8 [M][K], sx : f32 [K/128][M]   (quantize_act_1x128 / rmsnorm_quant output)
 *   qw : u8 [N][K], sw : f32 [N/128][K/128] (quantize_weight_128x128 output)
 *   y  : bf16 [M][N].
 * K % 128 == 0, N % 128 == 0, M >= 0 (any M).  K == 0 writes zeros.
 * Batch invariance: a row's output depends only on that row of (qx, sx) and on
 * the weight.  Every kernel folds the K-blocks in ascending order with
 * acc = fma(P_kb, fl32(sx * sw), acc), so the row is bitwise the same whatever
 * M is (a rollout batch or a training batch).
 */
int gemm_fprop(const uint8_t* qx, const float* sx, const uint8_t* qw, const float* sw, int64_t M,
               int64_t N, int64_t K, uint16_t* y, void* stream);

/*
 * gemm_fprop_splitk -- gemm_fprop for rollout batches, with the contraction
 * split across workgroups through a caller-provided fp32 workspace
 * ([P3-LAYOUT], [P3-CORE], [P3-STEPS] step 2; the rollout runs the training
 * forward's FP8 path, [P3-CORE]).  Same operands, layouts and requirements as
 * gemm_fprop.  When the output has fewer 128 x 128 tiles than the chip has
 * CUs (256) and 33 <= M <= 256 (or 17 <= M <= 32 with K >= 8192; smaller
 * batches stream the weights faster unsplit), K's 128-deep blocks are split into S equal
 * contiguous ranges (S divides K/128, at most two workgroups per CU, at least
 * four blocks per range); range s is folded in ascending order as in
 * gemm_fprop, from zero, into an fp32 partial, and
 *   y[m][n] = bf16(((P_0 + P_1) + P_2) + ... + P_{S-1}),
 * deterministic, but not bitwise the sequential fold of gemm_fprop.  Other
 * shapes need no workspace and run gemm_fprop itself.
 *   workspace       : f32 device buffer of at least
 *                     gemm_fprop_splitk_workspace_bytes(M, N, K) bytes (16-byte
 *                     aligned, overlapping no operand); its contents on entry
 *                     are ignored and on return unspecified.  May be NULL when
 *                     that size is 0.
 *   workspace_bytes : its size; smaller than required -> JETFP8_EINVAL.
 */
int gemm_fprop_splitk(const uint8_t* qx, const float* sx, const uint8_t* qw, const float* sw, int64_t M,
                      int64_t N, int64_t K, uint16_t* y, float* workspace, int64_t workspace_bytes,
                      void* stream);

/* Workspace bytes gemm_fprop_splitk needs for this shape (S * M * N * 4, or 0
 * when it runs gemm_fprop); -1 for an invalid shape.  Needs no GPU. */
int64_t gemm_fprop_splitk_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * gemm_fprop_splitk_noalloc -- gemm_fprop_splitk with a workspace the library
 * owns, for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): same
 * operands, results (bit for bit) and requirements, no workspace argument.
 * The workspace is a static device array of JETFP8_NOALLOC_SCRATCH_BYTES
 * (32 MiB) that every device the library runs on holds until the process
 * ends; its address is looked up on the first call on each device.  The call
 * allocates and frees nothing.  The split rule keeps every workspace within
 * that size (at most 512 K-shares of 128 x 128 fp32 partials), so every shape
 * gemm_fprop_splitk takes is accepted; a shape needing more would return
 * JETFP8_EUNSUPPORTED and write nothing.  All calls on one device share the
 * array, so calls that overlap on one device (different streams or threads)
 * race; serialise them.
 */
#define JETFP8_NOALLOC_SCRATCH_BYTES (32ll << 20)
int gemm_fprop_splitk_noalloc(const uint8_t* qx, const float* sx, const uint8_t* qw, const float* sw,
                              int64_t M, int64_t N, int64_t K, uint16_t* y, void* stream);

/*
 * pack_weight_rollout -- the rollout engine's copy of a quantised weight: the
 * codes of quantize_weight_128x128 in the order gemm_fprop_packed streams them
 * (the rollout runs the training forward's FP8 GEMM, [P3-CORE], [P3-STEPS]
 * step 2; at rollout batch sizes that GEMM is bound by reading the weight,
 * [P3-WEAK], and the rollout speed-up is the method's headline result,
 * [P3-RESULTS]).  A byte permutation, no arithmetic:
 *   qwp[((t * (K/128) + kb) * 2 + h) * 1024 + 16 l + b]
 *     = qw[16 t + (l mod 16)][128 kb + 32 floor(l / 16) + 16 h + b]
 *   for t < N/16, kb < K/128, h < 2, l < 64, b < 16:
 * each 16-row strip's 128-deep K-block is one contiguous 2 KB chunk.
 *   qw  : u8 [N][K] input;  qwp : u8, N * K bytes, output.
 * The weight's scales sw [N/128][K/128] are used unchanged.
 * N % 128 == 0, K % 128 == 0; N * K < 2^31 (gemm_fprop_packed's bound;
 * JETFP8_EUNSUPPORTED otherwise).
 */
int pack_weight_rollout(const uint8_t* qw, int64_t N, int64_t K, uint8_t* qwp, void* stream);

/*
 * gemm_fprop_packed -- gemm_fprop for rollout batches of up to 256 rows over
 * the packed weight ([P3-LAYOUT], [P3-CORE], [P3-STEPS] step 2):
 *   y = gemm_fprop(qx, sx, qw, sw) bit for bit, with qwp = pack_weight_rollout(qw).
 *   qx : u8 [M][K], sx : f32 [K/128][M]; qwp : u8, N * K bytes;
 *   sw : f32 [N/128][K/128]; y : bf16 [M][N].
 * 0 <= M <= 256 (JETFP8_EUNSUPPORTED above), N % 128 == 0, K % 128 == 0,
 * N * K < 2^31 and M * K < 2^31 (JETFP8_EUNSUPPORTED otherwise).  K == 0
 * writes zeros.  A row's output is the sequential K fold of gemm_fprop, so it
 * is bitwise the same as in a training batch or a rollout batch of any size.
 */
int gemm_fprop_packed(const uint8_t* qx, const float* sx, const uint8_t* qwp, const float* sw, int64_t M,
                      int64_t N, int64_t K, uint16_t* y, void* stream);

/*
 * gemm_fprop_swiglu_quant -- the gate+up projection's FProp fused with SwiGLU
 * and the 1x128 quantisation of its result: the FP8 input of the down
 * projection, with no bf16 gate+up output written at all ([P3-CORE] on fusing
 * the quantisation into the producing kernels; [P3-STEPS] step 2):
 *   (qh, sh) = swiglu_quant(gemm_fprop(qx, sx, qw, sw)), bit for bit: the GEMM
 *   epilogue rounds each output to bf16 exactly as gemm_fprop does and then
 *   applies swiglu_quant's arithmetic.
 *   qx : u8 [M][K], sx : f32 [K/128][M]
 *   qw : u8 [N][K], sw : f32 [N/128][K/128]: the gate+up weight, N = 2I rows,
 *        gate in rows 0 .. I-1 and up in rows I .. 2I-1 (swiglu_quant's layout)
 *   qh : u8 [M][I], sh : f32 [I/128][M] outputs.
 * N % 256 == 0 (I % 128 == 0), K % 128 == 0, M >= 0.  K == 0 gives h = 0
 * (codes 0, scales 1).  Runs the 256 x 256 tile kernel at every size: for
 * rollout batches (M of a few hundred or less) gemm_fprop or gemm_fprop_packed
 * followed by swiglu_quant is faster (same bits).
 */
int gemm_fprop_swiglu_quant(const uint8_t* qx, const float* sx, const uint8_t* qw, const float* sw, int64_t M,
                            int64_t N, int64_t K, uint8_t* qh, float* sh, void* stream);

/*
 * gemm_fprop_quant -- gemm_fprop, plus the 1x128 quantisation of its output for
 * the next layer's GEMM (the fused quantisation that removes a separate pass
 * over Y: [P3-CORE] on fusing quantisation into the producing kernels, [P3-STEPS]
 * step 2):
 *   y = gemm_fprop(qx, sx, qw, sw)   (bf16 [M][N], as gemm_fprop)
 *   (qy, sy) = quantize_act_1x128(y) (qy u8 [M][N], sy f32 [N/128][M]),
 * bit for bit: the quantisation reads the bf16 values of y.  The 1x128
 * quantiser runs right after the GEMM on the same stream (measured faster on
 * gfx950 than quantising in the GEMM epilogue).  Same shape rules as
 * gemm_fprop; y, qy and sy are all outputs (no overlap with each other or the
 * inputs).
 */
int gemm_fprop_quant(const uint8_t* qx, const float* sx, const uint8_t* qw, const float* sw,
                     int64_t M, int64_t N, int64_t K, uint16_t* y, uint8_t* qy, float* sy,
                     void* stream);

/*
 * gemm_dgrad -- input-gradient GEMM dX = dY W, same (1x128) x (128x128)
 * configuration as FProp with the weight blocks used transposed ([P3-LAYOUT],
 * [P3-CORE], [P3-STEPS] step 4):
 *   dX[m][k] = sum_nb sdy[nb][m] * sw[nb][k/128] * sum_{n in nb} qdy[m][n] * qw[n][k].
 *   qdy : u8 [M][N], sdy : f32 [N/128][M]  (quantize_act_1x128 of the bf16 dY)
 *   qw  : u8 [N][K], sw : f32 [N/128][K/128] (the same object FProp reads)
 *   dx  : bf16 [M][K].
 * N % 128 == 0, K % 128 == 0, M >= 0 (any M).  N == 0 writes zeros.
 */
int gemm_dgrad(const uint8_t* qdy, const float* sdy, const uint8_t* qw, const float* sw, int64_t M,
               int64_t N, int64_t K, uint16_t* dx, void* stream);

/*
 * gemm_wgrad -- weight-gradient GEMM dW = dY^T X with (1x128) x (128x1)
 * scaling, contracting over the M tokens ([P3-LAYOUT], [P3-CORE],
 * [P3-STEPS] step 4).  Both operands come from requant_transpose_128x1:
 *   dW[n][k] = sum_mb sdyt[mb][n] * sxt[mb][k] * sum_{m in mb} qdyt[n][m] * qxt[k][m].
 *   qdyt : u8 [N][M], sdyt : f32 [M/128][N]
 *   qxt  : u8 [K][M], sxt  : f32 [M/128][K]
 *   dw   : bf16 [N][K].
 * M % 128 == 0, N % 128 == 0, K % 128 == 0.  M == 0 writes zeros.
 */
int gemm_wgrad(const uint8_t* qdyt, const float* sdyt, const uint8_t* qxt, const float* sxt,
               int64_t M, int64_t N, int64_t K, uint16_t* dw, void* stream);

/*
 * gemm_wgrad_f32 -- gemm_wgrad with an fp32 output that is written or added
 * to.  The pages fix the weight gradient's operands and scaling ([P3-CORE],
 * [P3-STEPS] step 4) but not the precision the gradient is kept in; with an
 * fp32 output the gradients of several micro-batches (or of several token
 * shards on different GPUs) are summed before a single final rounding,
 * where bf16 partial gradients would each be rounded.
 *   accumulate == 0:  dw[n][k] = G[n][k]
 *   accumulate == 1:  dw[n][k] = fl32(dw[n][k] + G[n][k])
 * G is the fp32 accumulator that gemm_wgrad rounds: gemm_wgrad's output is
 * exactly the bf16 (nearest-even) rounding of G.
 *   dw : f32 [N][K], read as well as written when accumulate == 1.
 * Shape rules as gemm_wgrad, with 4-byte output elements in the size limit
 * (512 rows of dw below 2^31 bytes); accumulate must be 0 or 1 (else
 * JETFP8_EINVAL).  M == 0 writes zeros
 * (accumulate == 0) or leaves dw unchanged (accumulate == 1).
 */
int gemm_wgrad_f32(const uint8_t* qdyt, const float* sdyt, const uint8_t* qxt, const float* sxt,
                   int64_t M, int64_t N, int64_t K, float* dw, int accumulate, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* JETFP8_H */
