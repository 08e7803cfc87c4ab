// Library-wide entry points of libbi: status strings and the compile-time strategy.
#include "bi_common.h"

extern "C" int bi_get_config(bi_config* out) {
  if (!out) return BI_ERR_NULL;
  out->version = 3;
  out->tree_max_lanes = 256;
  out->wave_size = 64;
  out->gemm_tile_m = 128;
  out->gemm_tile_n = 128;
  out->gemm_tile_k = 64;
  out->gemm_mfma_m = 16;
  out->gemm_mfma_n = 16;
  out->gemm_mfma_k = 32;
  out->attn_chunk = 256;
  out->attn_max_group = 16;
  out->gemm_big_tile_m = 256;
  out->gemm_big_tile_n = 256;
  out->attn_merge_group = 4;
  return BI_OK;
}

extern "C" const char* bi_status_string(int status) {
  switch (status) {
    case BI_OK: return "BI_OK";
    case BI_ERR_NULL: return "BI_ERR_NULL";
    case BI_ERR_SHAPE: return "BI_ERR_SHAPE";
    case BI_ERR_DTYPE: return "BI_ERR_DTYPE";
    case BI_ERR_ALIGN: return "BI_ERR_ALIGN";
    case BI_ERR_WORKSPACE: return "BI_ERR_WORKSPACE";
    case BI_ERR_UNSUPPORTED: return "BI_ERR_UNSUPPORTED";
    case BI_ERR_HIP: return "BI_ERR_HIP";
    default: return "BI_ERR_UNKNOWN";
  }
}
