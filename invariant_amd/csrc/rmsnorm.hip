// bi_rmsnorm: one row per workgroup, fixed fp32 reduction tree (a function of D only).
//
// "Defeating nondeterminism in LLM inference", section on batch-invariant RMSNorm:
// y = x * rsqrt(mean(x^2)) * weight with a reduction order per row that no batch size
// can change.  Each row is reduced entirely inside one workgroup of 256 lanes; nothing
// is split across workgroups and there are no atomics.
//
// Tree (w = 8 bf16 or 4 fp32 elements per 16-byte vector, T = min(256, ceil(D/w))):
//   lane t owns vectors t, t+T, ...; adds its squares in ascending order from +0;
//   wave64 butterfly with offsets 1..32; waves combined as (w0 + w1) + (w2 + w3).
// Lanes t >= T hold +0.  Because every partial sum is >= +0, adding those +0 lanes or
// waves leaves each partial unchanged bit for bit, so one 256-lane shape serves every D.
#include "contract_fp.h"

namespace bi {
namespace {

constexpr int kThreads = 256;

template <bool F32>
struct Vec;
template <>
struct Vec<false> {  // 8 bf16
  static constexpr int W = 8;
  // NT: the row is read once (it fits in the registers), so the load does not allocate in
  // the caches
  template <bool NT = false>
  __device__ static void load(const void* row, int v, int D, bool vec_ok, float (&e)[8]) {
    const uint16_t* p = static_cast<const uint16_t*>(row) + static_cast<int64_t>(v) * 8;
    if (vec_ok && v * 8 + 8 <= D) {
      u16x8 q = NT ? __builtin_nontemporal_load(reinterpret_cast<const u16x8*>(p))
                   : *reinterpret_cast<const u16x8*>(p);
#pragma unroll
      for (int i = 0; i < 8; ++i) e[i] = bf16_to_f32(q[i]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) e[i] = (v * 8 + i < D) ? bf16_to_f32(p[i]) : 0.f;
    }
  }
};
template <>
struct Vec<true> {  // 4 fp32
  static constexpr int W = 4;
  template <bool NT = false>
  __device__ static void load(const void* row, int v, int D, bool vec_ok, float (&e)[4]) {
    const float* p = static_cast<const float*>(row) + static_cast<int64_t>(v) * 4;
    if (vec_ok && v * 4 + 4 <= D) {
      floatx4 q = *reinterpret_cast<const floatx4*>(p);
#pragma unroll
      for (int i = 0; i < 4; ++i) e[i] = q[i];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) e[i] = (v * 4 + i < D) ? p[i] : 0.f;
    }
  }
};

template <bool YF32, int W, bool FULL>
__device__ __forceinline__ void store_out(void* yrow, int v, int D, bool vec_ok, const float (&o)[W]) {
  if (YF32) {
    float* p = static_cast<float*>(yrow) + static_cast<int64_t>(v) * W;
    if (vec_ok && (FULL || v * W + W <= D) && W == 4) {
      floatx4 q;
#pragma unroll
      for (int i = 0; i < 4; ++i) q[i] = o[i];
      *reinterpret_cast<floatx4*>(p) = q;
    } else {
#pragma unroll
      for (int i = 0; i < W; ++i)
        if (v * W + i < D) p[i] = o[i];
    }
  } else {
    uint16_t* p = static_cast<uint16_t*>(yrow) + static_cast<int64_t>(v) * W;
    if (vec_ok && (FULL || v * W + W <= D) && W == 8) {
      u16x8 q;
#pragma unroll
      for (int i = 0; i < 8; ++i) q[i] = f32_to_bf16(o[i]);
      if (FULL) __builtin_nontemporal_store(q, reinterpret_cast<u16x8*>(p));   // written once
      else *reinterpret_cast<u16x8*>(p) = q;
    } else {
#pragma unroll
      for (int i = 0; i < W; ++i)
        if (v * W + i < D) p[i] = f32_to_bf16(o[i]);
    }
  }
}

// NV vectors per lane stay in registers between the two passes; longer rows re-read.
// FULL (bf16 in and out): D is a multiple of the vector width, at most NV vectors per
// lane (D <= 8192) and every row is 16-byte aligned, so no element needs a bounds check
// and x and y are each touched once: their loads and stores bypass the caches.
template <bool XF32, bool YF32, bool FULL>
__global__ __launch_bounds__(kThreads) void rmsnorm_kernel(const void* __restrict__ x,
                                                           const uint16_t* __restrict__ gamma,
                                                           void* __restrict__ y, int D,
                                                           int64_t ldx, int64_t ldy, float eps,
                                                           int vec_x, int vec_y, int vec_g) {
  using V = Vec<XF32>;
  constexpr int W = V::W;
  constexpr int NV = XF32 ? 8 : 4;
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int nvec = (D + W - 1) / W;
  const int T = nvec < kThreads ? nvec : kThreads;
  const char* xrow = static_cast<const char*>(x) + row * ldx * (XF32 ? 4 : 2);
  char* yrow = static_cast<char*>(y) + row * ldy * (YF32 ? 4 : 2);

  float cache[NV][W];
  float acc = 0.f;
  if (tid < T) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int v = tid + j * T;
      if (v < nvec) {
        V::template load<FULL>(xrow, v, D, FULL || vec_x, cache[j]);
#pragma unroll
        for (int i = 0; i < W; ++i)
          if (FULL || v * W + i < D) acc = acc + cache[j][i] * cache[j][i];
      }
    }
    for (int v = tid + NV * T; v < nvec; v += T) {
      float e[W];
      V::load(xrow, v, D, FULL || vec_x, e);
#pragma unroll
      for (int i = 0; i < W; ++i)
        if (FULL || v * W + i < D) acc = acc + e[i] * e[i];
    }
  }

  __shared__ float wave_part[kThreads / kWave];
  const float wsum = wave_tree_sum(acc);
  if ((tid & (kWave - 1)) == 0) wave_part[tid / kWave] = wsum;
  __syncthreads();
  const float ssum = (wave_part[0] + wave_part[1]) + (wave_part[2] + wave_part[3]);
  const float r = rms_scale(ssum, D, eps);

  if (tid >= T) return;
  for (int j = 0, v = tid; v < nvec; ++j, v += T) {
    float e[W];
    if (j < NV) {
#pragma unroll
      for (int jj = 0; jj < NV; ++jj)
        if (jj == j) {
#pragma unroll
          for (int i = 0; i < W; ++i) e[i] = cache[jj][i];
        }
    } else {
      V::load(xrow, v, D, FULL || vec_x, e);
    }
    float g[W];
    const uint16_t* gp = gamma + static_cast<int64_t>(v) * W;
    if ((FULL || (vec_g && v * W + W <= D)) && W == 8) {
      u16x8 q = *reinterpret_cast<const u16x8*>(gp);
#pragma unroll
      for (int i = 0; i < W; ++i) g[i] = bf16_to_f32(q[i]);
    } else {
#pragma unroll
      for (int i = 0; i < W; ++i) g[i] = (v * W + i < D) ? bf16_to_f32(gp[i]) : 0.f;
    }
    float o[W];
#pragma unroll
    for (int i = 0; i < W; ++i) o[i] = (e[i] * r) * g[i];
    store_out<YF32, W, FULL>(yrow, v, D, vec_y, o);
  }
}

// Residual add fused with the RMSNorm that follows it: s = a + b (fp32 add, rounded to the
// dtype of s, as bi_residual_add), written out, and y = rmsnorm(s) from those rounded values
// with the tree above (w = the vector width of s's dtype).  Both outputs equal the two calls'
// bits.  Rows are contiguous, 16-byte aligned, D a multiple of 8 and at most 8192: each lane
// holds its vectors in registers.  Every lane loads all of its a and b elements before it
// stores any element of s, and touches only its own elements, so s may be a or b itself.
template <bool F32, bool YF32>
__global__ __launch_bounds__(kThreads) void add_rmsnorm_kernel(const void* a, const void* b, void* sum,
                                                               const uint16_t* __restrict__ gamma,
                                                               void* __restrict__ y, int D, float eps) {
  constexpr int W = F32 ? 4 : 8;              // elements per 16-byte vector of a, b and s
  constexpr int NV = F32 ? 8 : 4;             // vectors per lane: D <= 8192
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int nvec = D / W;
  const int T = nvec < kThreads ? nvec : kThreads;
  float x[NV][W];
  float acc = 0.f;
  if (tid < T) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int v = tid + j * T;
      if (v >= nvec) continue;
      const int64_t e0 = row * D + static_cast<int64_t>(v) * W;
      if constexpr (F32) {
        const floatx4 qa = *reinterpret_cast<const floatx4*>(static_cast<const float*>(a) + e0);
        const floatx4 qb = *reinterpret_cast<const floatx4*>(static_cast<const float*>(b) + e0);
#pragma unroll
        for (int i = 0; i < 4; ++i) x[j][i] = qa[i] + qb[i];
      } else {
        const u16x8 qa = *reinterpret_cast<const u16x8*>(static_cast<const uint16_t*>(a) + e0);
        const u16x8 qb = *reinterpret_cast<const u16x8*>(static_cast<const uint16_t*>(b) + e0);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[j][i] = bf16_to_f32(f32_to_bf16(bf16_to_f32(qa[i]) + bf16_to_f32(qb[i])));
      }
#pragma unroll
      for (int i = 0; i < W; ++i) acc = acc + x[j][i] * x[j][i];
    }
#pragma unroll
    for (int j = 0; j < NV; ++j) {             // s: x holds it exactly in either dtype
      const int v = tid + j * T;
      if (v >= nvec) continue;
      const int64_t e0 = row * D + static_cast<int64_t>(v) * W;
      if constexpr (F32) {
        floatx4 q;
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = x[j][i];
        *reinterpret_cast<floatx4*>(static_cast<float*>(sum) + e0) = q;
      } else {
        u16x8 q;
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = f32_to_bf16(x[j][i]);
        *reinterpret_cast<u16x8*>(static_cast<uint16_t*>(sum) + e0) = q;
      }
    }
  }
  __shared__ float wave_part[kThreads / kWave];
  const float wsum = wave_tree_sum(acc);
  if ((tid & (kWave - 1)) == 0) wave_part[tid / kWave] = wsum;
  __syncthreads();
  const float ssum = (wave_part[0] + wave_part[1]) + (wave_part[2] + wave_part[3]);
  const float r = rms_scale(ssum, D, eps);
  if (tid >= T) return;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int v = tid + j * T;
    if (v >= nvec) continue;
    const int64_t e0 = row * D + static_cast<int64_t>(v) * W;
    float g[W];
#pragma unroll
    for (int i = 0; i < W; i += 4) {            // gamma is 16-byte aligned: W elements from v*W
      const u16x4 q = *reinterpret_cast<const u16x4*>(gamma + static_cast<int64_t>(v) * W + i);
#pragma unroll
      for (int e = 0; e < 4; ++e) g[i + e] = bf16_to_f32(q[e]);
    }
    float o[W];
#pragma unroll
    for (int i = 0; i < W; ++i) o[i] = (x[j][i] * r) * g[i];
    if constexpr (YF32) {
#pragma unroll
      for (int i = 0; i < W; i += 4) {
        floatx4 q;
#pragma unroll
        for (int e = 0; e < 4; ++e) q[e] = o[i + e];
        *reinterpret_cast<floatx4*>(static_cast<float*>(y) + e0 + i) = q;
      }
    } else if constexpr (W == 8) {
      u16x8 q;
#pragma unroll
      for (int i = 0; i < 8; ++i) q[i] = f32_to_bf16(o[i]);
      *reinterpret_cast<u16x8*>(static_cast<uint16_t*>(y) + e0) = q;
    } else {
      u16x4 q;
#pragma unroll
      for (int i = 0; i < 4; ++i) q[i] = f32_to_bf16(o[i]);
      *reinterpret_cast<u16x4*>(static_cast<uint16_t*>(y) + e0) = q;
    }
  }
}

}  // namespace
}  // namespace bi

using namespace bi;

extern "C" int bi_rmsnorm(const void* x, const void* gamma, void* y, int64_t M, int64_t D,
                          int64_t ldx, int64_t ldy, float eps, int x_dtype, int y_dtype,
                          void* stream) {
  if ((x_dtype != BI_BF16 && x_dtype != BI_F32) || (y_dtype != BI_BF16 && y_dtype != BI_F32))
    return BI_ERR_DTYPE;
  if (M < 0 || D < 0) return BI_ERR_SHAPE;
  if (M == 0) return BI_OK;
  if (D < 1 || ldx < D || ldy < D || D > (int64_t(1) << 24) || M > 0x7fffffffLL)
    return BI_ERR_SHAPE;
  if (!x || !gamma || !y) return BI_ERR_NULL;
  const bool xf = x_dtype == BI_F32, yf = y_dtype == BI_F32;
  const int wx = xf ? 4 : 8;
  const int vec_x = aligned16(x) && (ldx % wx == 0);
  const int vec_y = aligned16(y) && (ldy % (yf ? 4 : 8) == 0) && (yf ? wx == 4 : wx == 8);
  const int vec_g = aligned16(gamma);
  dim3 grid(static_cast<unsigned>(M)), block(kThreads);
  hipStream_t s = as_stream(stream);
  // bf16 rows that fit in the registers of one workgroup (D <= 8192), aligned: one read and
  // one write per element, streamed past the caches
  const bool full_bf16 = !xf && !yf && vec_x && vec_y && vec_g && (D % 8) == 0 && D <= 4 * kThreads * 8;
  if (full_bf16)
    rmsnorm_kernel<false, false, true><<<grid, block, 0, s>>>(x, static_cast<const uint16_t*>(gamma), y, int(D), ldx, ldy, eps, vec_x, vec_y, vec_g);
  else if (!xf && !yf)
    rmsnorm_kernel<false, false, false><<<grid, block, 0, s>>>(x, static_cast<const uint16_t*>(gamma), y, int(D), ldx, ldy, eps, vec_x, vec_y, vec_g);
  else if (!xf && yf)
    rmsnorm_kernel<false, true, false><<<grid, block, 0, s>>>(x, static_cast<const uint16_t*>(gamma), y, int(D), ldx, ldy, eps, vec_x, 0, vec_g);
  else if (xf && !yf)
    rmsnorm_kernel<true, false, false><<<grid, block, 0, s>>>(x, static_cast<const uint16_t*>(gamma), y, int(D), ldx, ldy, eps, vec_x, 0, vec_g);
  else
    rmsnorm_kernel<true, true, false><<<grid, block, 0, s>>>(x, static_cast<const uint16_t*>(gamma), y, int(D), ldx, ldy, eps, vec_x, vec_y, vec_g);
  return launch_status();
}

extern "C" int bi_add_rmsnorm(const void* a, const void* b, void* sum, int dtype, const void* gamma,
                              void* y, int y_dtype, int64_t M, int64_t D, float eps, void* stream) {
  if ((dtype != BI_BF16 && dtype != BI_F32) || (y_dtype != BI_BF16 && y_dtype != BI_F32))
    return BI_ERR_DTYPE;
  if (M < 0 || D < 0) return BI_ERR_SHAPE;
  if (M == 0) return BI_OK;
  if (D < 1 || M > 0x7fffffffLL) return BI_ERR_SHAPE;
  if (!a || !b || !sum || !gamma || !y) return BI_ERR_NULL;
  if (D % 8 != 0 || D > 4 * kThreads * 8) return BI_ERR_UNSUPPORTED;
  if (!aligned16(a) || !aligned16(b) || !aligned16(sum) || !aligned16(y) || !aligned16(gamma))
    return BI_ERR_ALIGN;
  const dim3 grid(static_cast<unsigned>(M)), block(kThreads);
  hipStream_t s = as_stream(stream);
  const uint16_t* g = static_cast<const uint16_t*>(gamma);
  const int di = static_cast<int>(D);
  if (dtype == BI_BF16 && y_dtype == BI_BF16)
    add_rmsnorm_kernel<false, false><<<grid, block, 0, s>>>(a, b, sum, g, y, di, eps);
  else if (dtype == BI_BF16)
    add_rmsnorm_kernel<false, true><<<grid, block, 0, s>>>(a, b, sum, g, y, di, eps);
  else if (y_dtype == BI_BF16)
    add_rmsnorm_kernel<true, false><<<grid, block, 0, s>>>(a, b, sum, g, y, di, eps);
  else
    add_rmsnorm_kernel<true, true><<<grid, block, 0, s>>>(a, b, sum, g, y, di, eps);
  return launch_status();
}
