/* bi_gemm and bi_logsoftmax_argmax driven from plain C with HIP-runtime device memory (no
 * C++, no torch): small-integer operands make every partial sum an exact fp32 integer, so
 * the fp32 output must equal the integer product exactly and the bf16 output its one
 * round-to-nearest-even rounding; a one-row call must give the full call's row bit for
 * bit; the argmax of rows with a unique maximum must be its index.  Built by
 * tests/c/build.py, run by tests/test_gpu_c_abi.py; prints "ok" and exits 0, or prints
 * the first failing check and exits 1 (2 without a device). */
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "bi.h"

#define CHECK(cond)                                                  \
  do {                                                               \
    if (!(cond)) {                                                   \
      printf("failed: %s (line %d)\n", #cond, __LINE__);             \
      return 1;                                                      \
    }                                                                \
  } while (0)
#define HIP(call) CHECK((call) == hipSuccess)

static uint32_t lcg(uint32_t* s) { return *s = *s * 1664525u + 1013904223u; }

static uint16_t bf16_of_small_int(int v) {   /* exact: |v| < 256 */
  float f = (float)v;
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

static uint16_t bf16_rne(float f) {   /* finite f */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

int main(void) {
  int n_dev = 0;
  if (hipGetDeviceCount(&n_dev) != hipSuccess || n_dev < 1) {
    printf("no device\n");
    return 2;
  }
  enum { M = 300, N = 257, K = 1000, V = 1000, R = 3 };
  uint16_t* a = malloc(sizeof(uint16_t) * M * K);
  uint16_t* b = malloc(sizeof(uint16_t) * N * K);
  int* ai = malloc(sizeof(int) * M * K);
  int* bi = malloc(sizeof(int) * N * K);
  float* c32 = malloc(sizeof(float) * M * N);
  uint16_t* c16 = malloc(sizeof(uint16_t) * M * N);
  float* row32 = malloc(sizeof(float) * N);
  float* logits = malloc(sizeof(float) * R * V);
  CHECK(a && b && ai && bi && c32 && c16 && row32 && logits);
  uint32_t s = 12345u;
  for (int i = 0; i < M * K; ++i) {
    ai[i] = (int)(lcg(&s) >> 24) % 9 - 4;
    a[i] = bf16_of_small_int(ai[i]);
  }
  for (int i = 0; i < N * K; ++i) {
    bi[i] = (int)(lcg(&s) >> 24) % 9 - 4;
    b[i] = bf16_of_small_int(bi[i]);
  }
  int want_argmax[R];
  for (int r = 0; r < R; ++r) {
    for (int v = 0; v < V; ++v) logits[r * V + v] = (float)((int)(lcg(&s) >> 24) % 100) * 0.01f;
    want_argmax[r] = (int)(lcg(&s) % V);
    logits[r * V + want_argmax[r]] = 5.0f;
  }

  void *dA, *dB, *dC32, *dC16, *dRow, *dL;
  int32_t* dAm;
  HIP(hipMalloc(&dA, sizeof(uint16_t) * M * K));
  HIP(hipMalloc(&dB, sizeof(uint16_t) * N * K));
  HIP(hipMalloc(&dC32, sizeof(float) * M * N));
  HIP(hipMalloc(&dC16, sizeof(uint16_t) * M * N));
  HIP(hipMalloc(&dRow, sizeof(float) * N));
  HIP(hipMalloc(&dL, sizeof(float) * R * V));
  HIP(hipMalloc((void**)&dAm, sizeof(int32_t) * R));
  HIP(hipMemcpy(dA, a, sizeof(uint16_t) * M * K, hipMemcpyHostToDevice));
  HIP(hipMemcpy(dB, b, sizeof(uint16_t) * N * K, hipMemcpyHostToDevice));
  HIP(hipMemcpy(dL, logits, sizeof(float) * R * V, hipMemcpyHostToDevice));

  CHECK(bi_gemm(dA, dB, dC32, M, N, K, K, K, N, BI_B_NK, BI_BF16, BI_F32, NULL) == BI_OK);
  CHECK(bi_gemm(dA, dB, dC16, M, N, K, K, K, N, BI_B_NK, BI_BF16, BI_BF16, NULL) == BI_OK);
  /* row 7 alone (its A row as a one-row matrix) */
  CHECK(bi_gemm((const uint16_t*)dA + 7 * K, dB, dRow, 1, N, K, K, K, N, BI_B_NK, BI_BF16, BI_F32,
                NULL) == BI_OK);
  CHECK(bi_logsoftmax_argmax((const float*)dL, R, V, V, NULL, dAm, NULL) == BI_OK);
  HIP(hipDeviceSynchronize());
  HIP(hipMemcpy(c32, dC32, sizeof(float) * M * N, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(c16, dC16, sizeof(uint16_t) * M * N, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(row32, dRow, sizeof(float) * N, hipMemcpyDeviceToHost));
  int32_t am[R];
  HIP(hipMemcpy(am, dAm, sizeof(int32_t) * R, hipMemcpyDeviceToHost));

  for (int i = 0; i < M; ++i)
    for (int j = 0; j < N; ++j) {
      int acc = 0;
      for (int k = 0; k < K; ++k) acc += ai[i * K + k] * bi[j * K + k];
      CHECK(c32[i * N + j] == (float)acc);
      CHECK(c16[i * N + j] == bf16_rne((float)acc));
    }
  CHECK(memcmp(row32, c32 + 7 * N, sizeof(float) * N) == 0);
  for (int r = 0; r < R; ++r) CHECK(am[r] == want_argmax[r]);

  HIP(hipFree(dA));
  HIP(hipFree(dB));
  HIP(hipFree(dC32));
  HIP(hipFree(dC16));
  HIP(hipFree(dRow));
  HIP(hipFree(dL));
  HIP(hipFree(dAm));
  free(a); free(b); free(ai); free(bi); free(c32); free(c16); free(row32); free(logits);
  printf("ok\n");
  return 0;
}
