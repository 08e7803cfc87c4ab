/* The C ABI used from plain C (no C++, no torch): include/bi.h compiles as C99, libbi.so
 * links, and the calls that need no GPU work behave as the header states -- the
 * compile-time strategy, status strings, and argument validation that returns before
 * anything is launched.  Built and run by tests/test_abi_cpu.py; exits 0 when every check
 * holds, else prints the first failing check and exits 1. */
#include <stdio.h>
#include <string.h>

#include "bi.h"

#define CHECK(cond)                                              \
  do {                                                           \
    if (!(cond)) {                                               \
      printf("failed: %s (line %d)\n", #cond, __LINE__);         \
      return 1;                                                  \
    }                                                            \
  } while (0)

int main(void) {
  bi_config cfg;
  memset(&cfg, 0, sizeof cfg);
  CHECK(bi_get_config(&cfg) == BI_OK);
  CHECK(cfg.tree_max_lanes == 256 && cfg.wave_size == 64 && cfg.attn_chunk == 256);
  CHECK(cfg.gemm_mfma_m == 16 && cfg.gemm_mfma_n == 16 && cfg.gemm_mfma_k == 32);
  CHECK(bi_get_config(NULL) == BI_ERR_NULL);
  CHECK(strcmp(bi_status_string(BI_OK), "BI_OK") == 0);
  CHECK(strcmp(bi_status_string(BI_ERR_WORKSPACE), "BI_ERR_WORKSPACE") == 0);

  /* never dereferenced: every call below fails validation first */
  void* p = (void*)(uintptr_t)16;
  CHECK(bi_rmsnorm(p, p, p, 4, 8, 8, 8, 1e-6f, 7, BI_BF16, NULL) == BI_ERR_DTYPE);
  CHECK(bi_rmsnorm(p, p, p, 4, 8, 4, 8, 1e-6f, BI_BF16, BI_BF16, NULL) == BI_ERR_SHAPE);
  CHECK(bi_rmsnorm(NULL, p, p, 4, 8, 8, 8, 1e-6f, BI_BF16, BI_BF16, NULL) == BI_ERR_NULL);
  CHECK(bi_rmsnorm(NULL, NULL, NULL, 0, 8, 8, 8, 1e-6f, BI_BF16, BI_BF16, NULL) == BI_OK);
  CHECK(bi_gemm(p, p, p, 4, 4, 0, 8, 8, 4, BI_B_NK, BI_BF16, BI_BF16, NULL) == BI_ERR_SHAPE);
  CHECK(bi_gemm((void*)(uintptr_t)18, p, p, 4, 4, 8, 8, 8, 4, BI_B_NK, BI_BF16, BI_BF16, NULL) ==
        BI_ERR_ALIGN);
  CHECK(bi_logsoftmax_argmax((const float*)p, 2, 10, 8, NULL, (int32_t*)p, NULL) == BI_ERR_SHAPE);
  /* attention: head_dim 64 is not supported; a missing workspace is reported */
  const int32_t* ip = (const int32_t*)p;
  CHECK(bi_attention(p, BI_BF16, p, p, p, p, ip, ip, ip, 2, 4, 32, 8, 64, 16, 4, 64, 0.088f, p,
                     BI_BF16, NULL, 0, NULL) == BI_ERR_UNSUPPORTED);
  CHECK(bi_attention(p, BI_BF16, p, p, p, p, ip, ip, ip, 2, 4, 32, 8, 128, 16, 4, 64, 0.088f, p,
                     BI_BF16, NULL, 0, NULL) == BI_ERR_WORKSPACE);
  CHECK(bi_attention_workspace_bytes(4, 32, 128, 64) ==
        (size_t)(4 * 32 * 2 + 4 * 32 * 128) * 4 + 4 * 16);
  CHECK(bi_rope_kv_write(p, 6144, BI_BF16, p, 5, p, p, ip, ip, ip, 2, 4, 32, 8, 128, 16, 4, 10000.0,
                         NULL) == BI_ERR_DTYPE);
  printf("ok\n");
  return 0;
}
