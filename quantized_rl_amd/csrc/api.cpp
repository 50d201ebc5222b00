// C ABI of the FP8 linear-layer library: host-side validation, then launch.
//
// Every argument is checked before anything is enqueued, so an invalid call
// writes nothing.  The checks need no GPU, so they are exercised on the CPU.
#include <stdint.h>

#include <initializer_list>

#include "../../include/jetfp8.h"
#include "launch.hpp"

namespace {

constexpr int64_t kMaxDim = 2147483647;  // 2^31 - 1

struct Buf {
  const void* p;
  int64_t bytes;  // 0 for an empty tensor
};

bool dim_ok(int64_t d) { return d >= 0 && d <= kMaxDim; }

int check_ptrs(std::initializer_list<Buf> ins, std::initializer_list<Buf> outs) {
  auto check_one = [](const Buf& b) -> int {
    if (b.bytes == 0) return JETFP8_OK;
    if (b.p == nullptr) return JETFP8_ENULL;
    if (reinterpret_cast<uintptr_t>(b.p) & 15u) return JETFP8_EALIGN;
    return JETFP8_OK;
  };
  for (const Buf& b : ins)
    if (int st = check_one(b)) return st;
  for (const Buf& b : outs)
    if (int st = check_one(b)) return st;
  auto overlap = [](const Buf& a, const Buf& b) {
    if (a.bytes == 0 || b.bytes == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + static_cast<uintptr_t>(b.bytes) && b0 < a0 + static_cast<uintptr_t>(a.bytes);
  };
  for (const Buf* o = outs.begin(); o != outs.end(); ++o) {
    for (const Buf& i : ins)
      if (overlap(*o, i)) return JETFP8_EALIAS;
    for (const Buf* o2 = o + 1; o2 != outs.end(); ++o2)
      if (overlap(*o, *o2)) return JETFP8_EALIAS;
  }
  return JETFP8_OK;
}

int launched(hipError_t e) { return e == hipSuccess ? JETFP8_OK : JETFP8_ELAUNCH; }

// The GEMM kernels address their operands with 32-bit byte offsets (buffer
// resources).  The library launches a problem whose rows do not fit as
// several row ranges, so what must fit is the B operand (cols x kc bytes) and
// a range of 512 rows of A (kc bytes each) and of the output (cols elements of
// out_bytes each).
bool gemm_fits(int64_t cols, int64_t kc, int64_t out_bytes = 2) {
  const int64_t lim = int64_t(1) << 31;
  return cols * kc < lim && 512 * kc < lim && 512 * cols * out_bytes < lim;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

const char* jetfp8_status_string(int status) {
  switch (status) {
    case JETFP8_OK: return "ok";
    case JETFP8_EINVAL: return "invalid shape";
    case JETFP8_EALIGN: return "pointer not 16-byte aligned";
    case JETFP8_ENULL: return "null pointer";
    case JETFP8_EALIAS: return "output overlaps an input or another output";
    case JETFP8_EUNSUPPORTED: return "unsupported";
    case JETFP8_ELAUNCH: return "HIP launch error";
    default: return "unknown status";
  }
}

int quantize_act_1x128(const uint16_t* x, int64_t M, int64_t K, uint8_t* q, float* s,
                       void* stream) {
  if (!dim_ok(M) || !dim_ok(K) || K % 128) return JETFP8_EINVAL;
  const int64_t n = M * K;
  if (int st = check_ptrs({{x, 2 * n}}, {{q, n}, {s, 4 * (n / 128)}})) return st;
  return launched(jetfp8::launch_quant_act(x, M, K, q, s, as_stream(stream)));
}

int quantize_weight_128x128(const uint16_t* w, int64_t N, int64_t K, uint8_t* q, float* s,
                            void* stream) {
  if (!dim_ok(N) || !dim_ok(K) || N % 128 || K % 128) return JETFP8_EINVAL;
  const int64_t n = N * K;
  if (int st = check_ptrs({{w, 2 * n}}, {{q, n}, {s, 4 * (n / (128 * 128))}})) return st;
  return launched(jetfp8::launch_quant_weight(w, N, K, q, s, as_stream(stream)));
}

int rmsnorm_quant(const uint16_t* x, const uint16_t* gamma, int64_t M, int64_t K, float eps,
                  uint8_t* q, float* s, void* stream) {
  if (!dim_ok(M) || K <= 0 || K > 65536 || K % 128) return JETFP8_EINVAL;
  const int64_t n = M * K;
  if (int st = check_ptrs({{x, 2 * n}, {gamma, 2 * K}}, {{q, n}, {s, 4 * (n / 128)}})) return st;
  return launched(jetfp8::launch_rmsnorm_quant(x, gamma, M, K, eps, q, s, nullptr, as_stream(stream)));
}

int rmsnorm_quant_rstd(const uint16_t* x, const uint16_t* gamma, int64_t M, int64_t K, float eps,
                       uint8_t* q, float* s, float* rstd, void* stream) {
  if (!dim_ok(M) || K <= 0 || K > 65536 || K % 128) return JETFP8_EINVAL;
  const int64_t n = M * K;
  if (int st = check_ptrs({{x, 2 * n}, {gamma, 2 * K}}, {{q, n}, {s, 4 * (n / 128)}, {rstd, 4 * M}}))
    return st;
  return launched(jetfp8::launch_rmsnorm_quant(x, gamma, M, K, eps, q, s, rstd, as_stream(stream)));
}

int64_t rmsnorm_backward_workspace_bytes(int64_t M, int64_t K) {
  if (!dim_ok(M) || K <= 0 || K > 24576 || K % 128) return -1;
  return 4 * jetfp8::rmsnorm_backward_parts(M) * K;
}

int rmsnorm_backward(const uint16_t* x, const uint16_t* gamma, const float* rstd, const uint16_t* dy,
                     int64_t M, int64_t K, uint16_t* dx, float* dgamma, float* workspace, void* stream) {
  const int64_t ws = rmsnorm_backward_workspace_bytes(M, K);
  if (ws < 0) return JETFP8_EINVAL;
  const int64_t n = M * K;
  if (int st = check_ptrs({{x, 2 * n}, {gamma, 2 * K}, {rstd, 4 * M}, {dy, 2 * n}},
                          {{dx, 2 * n}, {dgamma, 4 * K}, {workspace, ws}}))
    return st;
  return launched(jetfp8::launch_rmsnorm_backward(x, gamma, rstd, dy, M, K, dx, dgamma, workspace,
                                                  as_stream(stream)));
}

int swiglu_quant(const uint16_t* y, int64_t M, int64_t I, uint8_t* q, float* s, void* stream) {
  if (!dim_ok(M) || !dim_ok(I) || I % 128 || I > kMaxDim / 2) return JETFP8_EINVAL;
  const int64_t n = M * I;
  if (int st = check_ptrs({{y, 4 * n}}, {{q, n}, {s, 4 * (n / 128)}})) return st;
  return launched(jetfp8::launch_swiglu_quant(y, M, I, q, s, as_stream(stream)));
}

int requant_transpose_128x1(const uint8_t* q, const float* s, int64_t M, int64_t K, uint8_t* qt,
                            float* st, void* stream) {
  if (!dim_ok(M) || !dim_ok(K) || M % 128 || K % 128) return JETFP8_EINVAL;
  const int64_t n = M * K;
  if (int e = check_ptrs({{q, n}, {s, 4 * (n / 128)}}, {{qt, n}, {st, 4 * (n / 128)}})) return e;
  return launched(jetfp8::launch_requant(q, s, M, K, qt, st, as_stream(stream)));
}

int gemm_fprop(const uint8_t* qx, const float* sx, const uint8_t* qw, const float* sw, int64_t M,
               int64_t N, int64_t K, uint16_t* y, void* stream) {
  if (!dim_ok(M) || !dim_ok(N) || !dim_ok(K) || N % 128 || K % 128) return JETFP8_EINVAL;
  if (int st = check_ptrs({{qx, M * K}, {sx, 4 * (M * K / 128)}, {qw, N * K},
                           {sw, 4 * (N * K / (128 * 128))}},
                          {{y, 2 * M * N}}))
    return st;
  if (!gemm_fits(N, K)) return JETFP8_EUNSUPPORTED;
  return launched(jetfp8::launch_gemm_fprop(qx, sx, qw, sw, M, N, K, y, as_stream(stream)));
}

int64_t gemm_fprop_splitk_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (!dim_ok(M) || !dim_ok(N) || !dim_ok(K) || N % 128 || K % 128) return -1;
  return jetfp8::fprop_splitk_workspace_bytes(M, N, K);
}

int gemm_fprop_splitk(const uint8_t* qx, const float* sx, const uint8_t* qw, const float* sw, int64_t M,
                      int64_t N, int64_t K, uint16_t* y, float* workspace, int64_t workspace_bytes,
                      void* stream) {
  const int64_t ws = gemm_fprop_splitk_workspace_bytes(M, N, K);
  if (ws < 0 || workspace_bytes < ws) return JETFP8_EINVAL;
  if (int st = check_ptrs({{qx, M * K}, {sx, 4 * (M * K / 128)}, {qw, N * K},
                           {sw, 4 * (N * K / (128 * 128))}},
                          {{y, 2 * M * N}, {workspace, ws}}))
    return st;
  if (!gemm_fits(N, K)) return JETFP8_EUNSUPPORTED;
  return launched(jetfp8::launch_gemm_fprop_splitk(qx, sx, qw, sw, M, N, K, y, workspace, as_stream(stream)));
}

int gemm_fprop_splitk_noalloc(const uint8_t* qx, const float* sx, const uint8_t* qw, const float* sw,
                              int64_t M, int64_t N, int64_t K, uint16_t* y, void* stream) {
  static_assert(JETFP8_NOALLOC_SCRATCH_BYTES == (int64_t(32) << 20), "header and library agree on the size");
  const int64_t ws = gemm_fprop_splitk_workspace_bytes(M, N, K);
  if (ws < 0) return JETFP8_EINVAL;
  if (int st = check_ptrs({{qx, M * K}, {sx, 4 * (M * K / 128)}, {qw, N * K},
                           {sw, 4 * (N * K / (128 * 128))}},
                          {{y, 2 * M * N}}))
    return st;
  if (!gemm_fits(N, K) || ws > jetfp8::fprop_noalloc_scratch_bytes()) return JETFP8_EUNSUPPORTED;
  return launched(jetfp8::launch_gemm_fprop_splitk_noalloc(qx, sx, qw, sw, M, N, K, y, as_stream(stream)));
}

int pack_weight_rollout(const uint8_t* qw, int64_t N, int64_t K, uint8_t* qwp, void* stream) {
  if (!dim_ok(N) || !dim_ok(K) || N % 128 || K % 128) return JETFP8_EINVAL;
  const int64_t n = N * K;
  if (int st = check_ptrs({{qw, n}}, {{qwp, n}})) return st;
  if (n >= (int64_t(1) << 31)) return JETFP8_EUNSUPPORTED;
  return launched(jetfp8::launch_pack_weight_rollout(qw, N, K, qwp, as_stream(stream)));
}

int gemm_fprop_packed(const uint8_t* qx, const float* sx, const uint8_t* qwp, const float* sw, int64_t M,
                      int64_t N, int64_t K, uint16_t* y, void* stream) {
  if (!dim_ok(M) || !dim_ok(N) || !dim_ok(K) || N % 128 || K % 128) return JETFP8_EINVAL;
  if (int st = check_ptrs({{qx, M * K}, {sx, 4 * (M * K / 128)}, {qwp, N * K},
                           {sw, 4 * (N * K / (128 * 128))}},
                          {{y, 2 * M * N}}))
    return st;
  const int64_t lim = int64_t(1) << 31;
  if (M > 256 || N * K >= lim || M * K >= lim) return JETFP8_EUNSUPPORTED;
  return launched(jetfp8::launch_gemm_fprop_packed(qx, sx, qwp, sw, M, N, K, y, as_stream(stream)));
}

int gemm_fprop_swiglu_quant(const uint8_t* qx, const float* sx, const uint8_t* qw, const float* sw, int64_t M,
                            int64_t N, int64_t K, uint8_t* qh, float* sh, void* stream) {
  if (!dim_ok(M) || !dim_ok(N) || !dim_ok(K) || N % 256 || K % 128) return JETFP8_EINVAL;
  const int64_t nh = M * (N / 2);
  if (int st = check_ptrs({{qx, M * K}, {sx, 4 * (M * K / 128)}, {qw, N * K},
                           {sw, 4 * (N * K / (128 * 128))}},
                          {{qh, nh}, {sh, 4 * (nh / 128)}}))
    return st;
  const int64_t lim = int64_t(1) << 31;
  if (N * K >= lim || 512 * K >= lim || 512 * (N / 2) >= lim) return JETFP8_EUNSUPPORTED;
  return launched(jetfp8::launch_gemm_fprop_swiglu_quant(qx, sx, qw, sw, M, N, K, qh, sh, as_stream(stream)));
}

int gemm_fprop_quant(const uint8_t* qx, const float* sx, const uint8_t* qw, const float* sw,
                     int64_t M, int64_t N, int64_t K, uint16_t* y, uint8_t* qy, float* sy,
                     void* stream) {
  if (!dim_ok(M) || !dim_ok(N) || !dim_ok(K) || N % 128 || K % 128) return JETFP8_EINVAL;
  if (int st = check_ptrs({{qx, M * K}, {sx, 4 * (M * K / 128)}, {qw, N * K},
                           {sw, 4 * (N * K / (128 * 128))}},
                          {{y, 2 * M * N}, {qy, M * N}, {sy, 4 * (M * N / 128)}}))
    return st;
  if (!gemm_fits(N, K)) return JETFP8_EUNSUPPORTED;
  // FProp, then the 1x128 quantiser on y, back to back on the stream.  (Doing the
  // quantisation in the 256 x 256 kernel's epilogue was measured slower: there it
  // runs after the main loop at two waves per SIMD with nothing to overlap, while
  // the separate kernel hides the same ALU work under its memory traffic.)
  const hipError_t e = jetfp8::launch_gemm_fprop(qx, sx, qw, sw, M, N, K, y, as_stream(stream));
  if (e != hipSuccess) return launched(e);
  return launched(jetfp8::launch_quant_act(y, M, N, qy, sy, as_stream(stream)));
}

int gemm_dgrad(const uint8_t* qdy, const float* sdy, const uint8_t* qw, const float* sw, int64_t M,
               int64_t N, int64_t K, uint16_t* dx, void* stream) {
  if (!dim_ok(M) || !dim_ok(N) || !dim_ok(K) || N % 128 || K % 128) return JETFP8_EINVAL;
  if (int st = check_ptrs({{qdy, M * N}, {sdy, 4 * (M * N / 128)}, {qw, N * K},
                           {sw, 4 * (N * K / (128 * 128))}},
                          {{dx, 2 * M * K}}))
    return st;
  if (!gemm_fits(K, N)) return JETFP8_EUNSUPPORTED;
  return launched(jetfp8::launch_gemm_dgrad(qdy, sdy, qw, sw, M, N, K, dx, as_stream(stream)));
}

int gemm_wgrad(const uint8_t* qdyt, const float* sdyt, const uint8_t* qxt, const float* sxt,
               int64_t M, int64_t N, int64_t K, uint16_t* dw, void* stream) {
  if (!dim_ok(M) || !dim_ok(N) || !dim_ok(K) || M % 128 || N % 128 || K % 128)
    return JETFP8_EINVAL;
  if (int st = check_ptrs({{qdyt, N * M}, {sdyt, 4 * (N * M / 128)}, {qxt, K * M},
                           {sxt, 4 * (K * M / 128)}},
                          {{dw, 2 * N * K}}))
    return st;
  if (!gemm_fits(K, M)) return JETFP8_EUNSUPPORTED;
  return launched(jetfp8::launch_gemm_wgrad(qdyt, sdyt, qxt, sxt, M, N, K, dw, as_stream(stream)));
}

int gemm_wgrad_f32(const uint8_t* qdyt, const float* sdyt, const uint8_t* qxt, const float* sxt,
                   int64_t M, int64_t N, int64_t K, float* dw, int accumulate, void* stream) {
  if (!dim_ok(M) || !dim_ok(N) || !dim_ok(K) || M % 128 || N % 128 || K % 128) return JETFP8_EINVAL;
  if (accumulate != 0 && accumulate != 1) return JETFP8_EINVAL;
  if (int st = check_ptrs({{qdyt, N * M}, {sdyt, 4 * (N * M / 128)}, {qxt, K * M},
                           {sxt, 4 * (K * M / 128)}},
                          {{dw, 4 * N * K}}))
    return st;
  if (!gemm_fits(K, M, 4)) return JETFP8_EUNSUPPORTED;
  return launched(jetfp8::launch_gemm_wgrad_f32(qdyt, sdyt, qxt, sxt, M, N, K, dw, accumulate != 0,
                                                as_stream(stream)));
}

}  // extern "C"
