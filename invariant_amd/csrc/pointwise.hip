// Pointwise glue of a Mistral-shaped decoder layer: embedding gather, RoPE (with the
// q/k/v split of the fused projection), SwiGLU and the residual add.
//
// "Defeating nondeterminism in LLM inference", section on making kernels
// batch-invariant: a pointwise operation is batch-invariant when every element runs
// the same code, whatever the number of rows.  Each kernel below maps one thread to a
// fixed set of elements by index only; the math is fp32 (RoPE angles in fp64) with one
// rounding to the output type.
#include "bi_common.h"

namespace bi {
namespace {

__device__ __forceinline__ float load_as_f32(const void* p, int64_t i, bool f32) {
  return f32 ? static_cast<const float*>(p)[i] : bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
}
__device__ __forceinline__ void store_from_f32(void* p, int64_t i, float v, bool f32) {
  if (f32) static_cast<float*>(p)[i] = v;
  else static_cast<uint16_t*>(p)[i] = f32_to_bf16(v);
}

__global__ void embedding_kernel(const int32_t* __restrict__ ids, const void* __restrict__ table,
                                 int table_f32, void* __restrict__ out, int64_t T, int64_t D,
                                 int64_t vocab, int out_f32) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= T * D) return;
  const int64_t t = i / D, d = i % D;
  const int32_t id = ids[t];
  const float v = (id >= 0 && id < vocab) ? load_as_f32(table, static_cast<int64_t>(id) * D + d, table_f32) : 0.f;
  store_from_f32(out, i, v, out_f32);
}

// One thread per (token, group of hpt heads, i < D/2): the rotation angle depends on the
// token's position and on i only, so the thread computes its cosine and sine once (fp64
// angle, each rounded to fp32) for the pairs (i, i + D/2) of all its q and k heads and copies
// its v heads.  Each element gets the same operations whatever the number of tokens, heads
// or heads per thread (one for a few tokens, where parallelism matters more than the
// repeated cosines; eight for many).
__global__ void rope_qkv_kernel(const void* __restrict__ qkv, int64_t ld, int qkv_f32,
                                const int32_t* __restrict__ positions, void* __restrict__ q, int q_f32,
                                uint16_t* __restrict__ k, uint16_t* __restrict__ v, int64_t T,
                                int hq, int hkv, int hd, double base, int hpt) {
  const int half = hd / 2;
  const int heads = hq + 2 * hkv;
  const int groups = (heads + hpt - 1) / hpt;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= T * groups * half) return;
  const int j = static_cast<int>(i % half);
  const int64_t tg = i / half;
  const int64_t t = tg / groups;
  const int h0 = static_cast<int>(tg % groups) * hpt;
  const int h1 = min(h0 + hpt, heads);
  const int64_t row = t * ld;
  float c = 1.f, s = 0.f;
  if (h0 < hq + hkv) rope_cos_sin(positions[t], j, hd, base, c, s);
  for (int h = h0; h < h1; ++h) {
    const int64_t src = row + static_cast<int64_t>(h) * hd;
    const float x1 = load_as_f32(qkv, src + j, qkv_f32);
    const float x2 = load_as_f32(qkv, src + j + half, qkv_f32);
    if (h >= hq + hkv) {   // v: copied
      uint16_t* dst = v + (t * hkv + (h - hq - hkv)) * hd;
      dst[j] = f32_to_bf16(x1);
      dst[j + half] = f32_to_bf16(x2);
      continue;
    }
    float y1, y2;
    rope_rotate(x1, x2, c, s, y1, y2);
    if (h < hq) {   // q: bf16, or fp32 (the FP32-activation variant)
      const int64_t o = (t * hq + h) * hd;
      store_from_f32(q, o + j, y1, q_f32);
      store_from_f32(q, o + j + half, y2, q_f32);
      continue;
    }
    uint16_t* dst = k + (t * hkv + (h - hq)) * hd;
    dst[j] = f32_to_bf16(y1);
    dst[j + half] = f32_to_bf16(y2);
  }
}

__global__ void swiglu_kernel(const uint16_t* __restrict__ gu, int64_t ld, uint16_t* __restrict__ out,
                              int64_t T, int64_t F) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= T * F) return;
  const int64_t t = i / F, j = i % F;
  out[i] = swiglu_bf16(gu[t * ld + j], gu[t * ld + F + j]);
}

__global__ void residual_add_kernel(const void* __restrict__ a, int af, const void* __restrict__ b,
                                    int bf, void* out, int of, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float v = load_as_f32(a, i, af) + load_as_f32(b, i, bf);
  store_from_f32(out, i, v, of);
}

// bf16 + bf16 -> bf16 with every pointer 16-byte aligned: 8 elements per thread (the same
// add and rounding per element as above).
__global__ void residual_add_bf16x8_kernel(const u16x8* __restrict__ a, const u16x8* __restrict__ b,
                                           u16x8* out, int64_t n8) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const u16x8 x = a[i], y = b[i];
  u16x8 o;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = f32_to_bf16(bf16_to_f32(x[e]) + bf16_to_f32(y[e]));
  out[i] = o;
}

unsigned blocks_for(int64_t n, int per) { return static_cast<unsigned>((n + per - 1) / per); }

}  // namespace
}  // namespace bi

using namespace bi;

extern "C" int bi_embedding(const int32_t* ids, const void* table, int table_dtype, void* out,
                            int64_t T, int64_t D, int64_t vocab, int out_dtype, void* stream) {
  if ((out_dtype != BI_BF16 && out_dtype != BI_F32) || (table_dtype != BI_BF16 && table_dtype != BI_F32))
    return BI_ERR_DTYPE;
  if (T < 0 || D < 0 || vocab < 0) return BI_ERR_SHAPE;
  if (T == 0 || D == 0) return BI_OK;
  if (T * D > (int64_t(1) << 40)) return BI_ERR_SHAPE;
  if (!ids || !table || !out) return BI_ERR_NULL;
  embedding_kernel<<<blocks_for(T * D, 256), 256, 0, as_stream(stream)>>>(
      ids, table, table_dtype == BI_F32, out, T, D, vocab, out_dtype == BI_F32);
  return launch_status();
}

extern "C" int bi_rope_qkv(const void* qkv, int64_t ldqkv, int qkv_dtype, const int32_t* positions,
                           void* q, int q_dtype, void* k, void* v, int64_t T, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, double base, void* stream) {
  if ((qkv_dtype != BI_BF16 && qkv_dtype != BI_F32) || (q_dtype != BI_BF16 && q_dtype != BI_F32))
    return BI_ERR_DTYPE;
  if (T < 0 || num_q_heads < 1 || num_kv_heads < 1 || head_dim < 2 || (head_dim & 1))
    return BI_ERR_SHAPE;
  if (ldqkv < static_cast<int64_t>(num_q_heads + 2 * num_kv_heads) * head_dim) return BI_ERR_SHAPE;
  if (T == 0) return BI_OK;
  if (!qkv || !positions || !q || !k || !v) return BI_ERR_NULL;
  const int hpt = T >= 256 ? 8 : 1;
  const int64_t groups = (num_q_heads + 2 * num_kv_heads + hpt - 1) / hpt;
  const int64_t n = T * groups * (head_dim / 2);
  rope_qkv_kernel<<<blocks_for(n, 256), 256, 0, as_stream(stream)>>>(
      qkv, ldqkv, qkv_dtype == BI_F32, positions, q, q_dtype == BI_F32,
      static_cast<uint16_t*>(k), static_cast<uint16_t*>(v), T, num_q_heads, num_kv_heads, head_dim,
      base, hpt);
  return launch_status();
}

extern "C" int bi_swiglu(const void* gu, int64_t ldgu, void* out, int64_t T, int64_t F,
                         void* stream) {
  if (T < 0 || F < 0 || ldgu < 2 * F) return BI_ERR_SHAPE;
  if (T == 0 || F == 0) return BI_OK;
  if (!gu || !out) return BI_ERR_NULL;
  swiglu_kernel<<<blocks_for(T * F, 256), 256, 0, as_stream(stream)>>>(
      static_cast<const uint16_t*>(gu), ldgu, static_cast<uint16_t*>(out), T, F);
  return launch_status();
}

extern "C" int bi_residual_add(const void* a, int a_dtype, const void* b, int b_dtype, void* out,
                               int out_dtype, int64_t n, void* stream) {
  for (int d : {a_dtype, b_dtype, out_dtype})
    if (d != BI_BF16 && d != BI_F32) return BI_ERR_DTYPE;
  if (n < 0) return BI_ERR_SHAPE;
  if (n == 0) return BI_OK;
  if (!a || !b || !out) return BI_ERR_NULL;
  if (a_dtype == BI_BF16 && b_dtype == BI_BF16 && out_dtype == BI_BF16 && n % 8 == 0 && aligned16(a) &&
      aligned16(b) && aligned16(out)) {
    residual_add_bf16x8_kernel<<<blocks_for(n / 8, 256), 256, 0, as_stream(stream)>>>(
        static_cast<const u16x8*>(a), static_cast<const u16x8*>(b), static_cast<u16x8*>(out), n / 8);
    return launch_status();
  }
  residual_add_kernel<<<blocks_for(n, 256), 256, 0, as_stream(stream)>>>(
      a, a_dtype == BI_F32, b, b_dtype == BI_F32, out, out_dtype == BI_F32, n);
  return launch_status();
}
