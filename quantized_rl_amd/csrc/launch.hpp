// Kernel launchers of the FP8 linear layer (internal; shapes already validated).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace jetfp8 {

// Compute units of the current device (cached per device; 0 if unknown).
int device_cu_count();

hipError_t launch_quant_act(const uint16_t* x, int64_t M, int64_t K, uint8_t* q, float* s,
                            hipStream_t stream);
hipError_t launch_quant_weight(const uint16_t* w, int64_t N, int64_t K, uint8_t* q, float* s,
                               hipStream_t stream);
hipError_t launch_rmsnorm_quant(const uint16_t* x, const uint16_t* gamma, int64_t M, int64_t K,
                                float eps, uint8_t* q, float* s, float* rstd, hipStream_t stream);
// Workgroups (and rows of K floats in the workspace) of the RMSNorm backward for M rows.
int64_t rmsnorm_backward_parts(int64_t M);
hipError_t launch_rmsnorm_backward(const uint16_t* x, const uint16_t* gamma, const float* rstd,
                                   const uint16_t* dy, int64_t M, int64_t K, uint16_t* dx,
                                   float* dgamma, float* workspace, hipStream_t stream);
hipError_t launch_swiglu_quant(const uint16_t* y, int64_t M, int64_t I, uint8_t* q, float* s,
                               hipStream_t stream);
hipError_t launch_requant(const uint8_t* q, const float* s, int64_t M, int64_t K, uint8_t* qt,
                          float* st, hipStream_t stream);
hipError_t launch_gemm_fprop(const uint8_t* qx, const float* sx, const uint8_t* qw, const float* sw,
                             int64_t M, int64_t N, int64_t K, uint16_t* y, hipStream_t stream);
// FProp with K split across workgroups through a caller workspace (65 .. 256
// rows with fewer 128 x 128 tiles than CUs); 0 bytes: plain FProp.
int64_t fprop_splitk_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_fprop_splitk(const uint8_t* qx, const float* sx, const uint8_t* qw, const float* sw,
                                    int64_t M, int64_t N, int64_t K, uint16_t* y, float* ws,
                                    hipStream_t stream);
// The same with the library's own workspace (at most fprop_noalloc_scratch_bytes()).
int64_t fprop_noalloc_scratch_bytes();
hipError_t launch_gemm_fprop_splitk_noalloc(const uint8_t* qx, const float* sx, const uint8_t* qw,
                                            const float* sw, int64_t M, int64_t N, int64_t K, uint16_t* y,
                                            hipStream_t stream);
// FProp of a gate+up projection (N = 2I weight rows: gate then up) fused with
// SwiGLU and the 1x128 quantisation of its result (q [M][I], s [I/128][M]).
hipError_t launch_gemm_fprop_swiglu_quant(const uint8_t* qx, const float* sx, const uint8_t* qw, const float* sw,
                                          int64_t M, int64_t N, int64_t K, uint8_t* q, float* s,
                                          hipStream_t stream);
// Rollout-packed copy of quantised weight codes (a byte permutation) and the
// FProp of up to 256 rows that streams it.
hipError_t launch_pack_weight_rollout(const uint8_t* qw, int64_t N, int64_t K, uint8_t* qwp, hipStream_t stream);
hipError_t launch_gemm_fprop_packed(const uint8_t* qx, const float* sx, const uint8_t* qwp, const float* sw,
                                    int64_t M, int64_t N, int64_t K, uint16_t* y, hipStream_t stream);
hipError_t launch_gemm_dgrad(const uint8_t* qdy, const float* sdy, const uint8_t* qw,
                             const float* sw, int64_t M, int64_t N, int64_t K, uint16_t* dx,
                             hipStream_t stream);
hipError_t launch_gemm_wgrad(const uint8_t* qdyt, const float* sdyt, const uint8_t* qxt,
                             const float* sxt, int64_t M, int64_t N, int64_t K, uint16_t* dw,
                             hipStream_t stream);
hipError_t launch_gemm_wgrad_f32(const uint8_t* qdyt, const float* sdyt, const uint8_t* qxt,
                                 const float* sxt, int64_t M, int64_t N, int64_t K, float* dw,
                                 bool accumulate, hipStream_t stream);

}  // namespace jetfp8
