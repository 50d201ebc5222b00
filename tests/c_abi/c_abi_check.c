/* Drives libjetfp8.so from plain C through include/jetfp8.h (no Python, no
 * torch): reads X bf16 [M][K] and W bf16 [N][K] from files, runs
 * quantize_act_1x128, quantize_weight_128x128, gemm_fprop and
 * gemm_fprop_splitk (with the workspace it asks for) on the default stream,
 * checks a few invalid calls for their status codes, and writes the outputs
 * to files for the test to compare with the oracle.
 *   usage: c_abi_check M K N x.bin w.bin out_prefix
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "jetfp8.h"

#define CHECK_HIP(x)                                                               \
  do {                                                                             \
    hipError_t e_ = (x);                                                           \
    if (e_ != hipSuccess) {                                                        \
      fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      return 2;                                                                    \
    }                                                                              \
  } while (0)

static int read_file(const char* path, void* dst, size_t bytes) {
  FILE* f = fopen(path, "rb");
  if (!f) return -1;
  size_t n = fread(dst, 1, bytes, f);
  fclose(f);
  return n == bytes ? 0 : -1;
}

static int write_file(const char* prefix, const char* name, const void* src, size_t bytes) {
  char path[1024];
  snprintf(path, sizeof path, "%s%s", prefix, name);
  FILE* f = fopen(path, "wb");
  if (!f) return -1;
  size_t n = fwrite(src, 1, bytes, f);
  fclose(f);
  return n == bytes ? 0 : -1;
}

int main(int argc, char** argv) {
  if (argc != 7) {
    fprintf(stderr, "usage: %s M K N x.bin w.bin out_prefix\n", argv[0]);
    return 2;
  }
  const int64_t M = atoll(argv[1]), K = atoll(argv[2]), N = atoll(argv[3]);
  const size_t xb = (size_t)(M * K) * 2, wb = (size_t)(N * K) * 2;
  uint16_t* hx = malloc(xb);
  uint16_t* hw = malloc(wb);
  uint8_t* hq = malloc((size_t)(M * K));
  float* hs = malloc((size_t)(M * K / 128) * 4);
  uint16_t* hy = malloc((size_t)(M * N) * 2);
  if (!hx || !hw || !hq || !hs || !hy) return 2;
  if (read_file(argv[4], hx, xb) || read_file(argv[5], hw, wb)) {
    fprintf(stderr, "cannot read inputs\n");
    return 2;
  }
  void *x, *w, *qx, *sx, *qw, *sw, *y;
  CHECK_HIP(hipMalloc(&x, xb));
  CHECK_HIP(hipMalloc(&w, wb));
  CHECK_HIP(hipMalloc(&qx, (size_t)(M * K)));
  CHECK_HIP(hipMalloc(&sx, (size_t)(M * K / 128) * 4));
  CHECK_HIP(hipMalloc(&qw, (size_t)(N * K)));
  CHECK_HIP(hipMalloc(&sw, (size_t)(N * K / (128 * 128)) * 4));
  CHECK_HIP(hipMalloc(&y, (size_t)(M * N) * 2));
  CHECK_HIP(hipMemcpy(x, hx, xb, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(w, hw, wb, hipMemcpyHostToDevice));

  int st = quantize_act_1x128(x, M, K, qx, sx, NULL);
  if (st) { fprintf(stderr, "quantize_act_1x128: %s\n", jetfp8_status_string(st)); return 1; }
  st = quantize_weight_128x128(w, N, K, qw, sw, NULL);
  if (st) { fprintf(stderr, "quantize_weight_128x128: %s\n", jetfp8_status_string(st)); return 1; }
  st = gemm_fprop(qx, sx, qw, sw, M, N, K, y, NULL);
  if (st) { fprintf(stderr, "gemm_fprop: %s\n", jetfp8_status_string(st)); return 1; }
  /* the split-K FProp with the workspace it asks for (none for shapes it does not split) */
  const int64_t need = gemm_fprop_splitk_workspace_bytes(M, N, K);
  if (need < 0) return 3;
  void *y2, *ws = NULL;
  CHECK_HIP(hipMalloc(&y2, (size_t)(M * N) * 2));
  if (need > 0) CHECK_HIP(hipMalloc(&ws, (size_t)need));
  st = gemm_fprop_splitk(qx, sx, qw, sw, M, N, K, y2, ws, need, NULL);
  if (st) { fprintf(stderr, "gemm_fprop_splitk: %s\n", jetfp8_status_string(st)); return 1; }
  /* invalid calls: rejected on the host before anything is enqueued */
  if (gemm_fprop_splitk_workspace_bytes(64, 384, 1024) <= 0) return 3;  /* a shape that splits */
  if (gemm_fprop_splitk(qx, sx, qw, sw, 64, 384, 1024, y2, NULL, 0, NULL) != JETFP8_EINVAL) return 3;
  if (gemm_fprop(qx, sx, qw, sw, M, N + 1, K, y, NULL) != JETFP8_EINVAL) return 3;
  if (gemm_fprop(qx, sx, qw, sw, M, N, K, (uint16_t*)qx, NULL) != JETFP8_EALIAS) return 3;
  if (quantize_act_1x128(x, M, K, NULL, sx, NULL) != JETFP8_ENULL) return 3;
  CHECK_HIP(hipDeviceSynchronize());

  CHECK_HIP(hipMemcpy(hq, qx, (size_t)(M * K), hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(hs, sx, (size_t)(M * K / 128) * 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(hy, y, (size_t)(M * N) * 2, hipMemcpyDeviceToHost));
  if (write_file(argv[6], "qx.bin", hq, (size_t)(M * K)) || write_file(argv[6], "sx.bin", hs, (size_t)(M * K / 128) * 4) ||
      write_file(argv[6], "y.bin", hy, (size_t)(M * N) * 2))
    return 2;
  CHECK_HIP(hipMemcpy(hy, y2, (size_t)(M * N) * 2, hipMemcpyDeviceToHost));
  if (write_file(argv[6], "y_splitk.bin", hy, (size_t)(M * N) * 2)) return 2;
  printf("c_abi_check ok\n");
  return 0;
}
