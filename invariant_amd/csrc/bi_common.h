// Device helpers shared by the HIP kernels of libbi (gfx950, wave64).
// Every file of the library is compiled with -ffp-contract=off: each fp32 multiply and
// add is rounded on its own unless a kernel asks for a fused multiply-add by name.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "../../include/bi.h"

namespace bi {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round to nearest even; a NaN keeps its sign and payload top bits and gets the
// quiet bit.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// fp32 v split exactly into three bf16 terms, v = hi + mid + lo for every normal v (24
// significand bits = 3 x 8): each term is the truncation to bf16 of what the previous terms
// leave.  A product of an fp32 operand with a bf16 one is then three exact bf16 products,
// accumulated hi, mid, lo (the "FP32 upcast" of the cross-vendor mismatch abstract).
__device__ __forceinline__ void split_bf16x3(float v, uint16_t& hi, uint16_t& mid, uint16_t& lo) {
  hi = static_cast<uint16_t>(__float_as_uint(v) >> 16);
  const float r1 = v - bf16_to_f32(hi);
  mid = static_cast<uint16_t>(__float_as_uint(r1) >> 16);
  const float r2 = r1 - bf16_to_f32(mid);
  lo = static_cast<uint16_t>(__float_as_uint(r2) >> 16);
}

// SwiGLU of one bf16 (gate, up) pair: silu(g) u in fp32 (silu(g) = g / (1 + 2^(-g log2 e)),
// hardware exp2, correctly rounded division), one RNE rounding.  The stand-alone kernel and
// the GEMM epilogue both call this, so fused and unfused outputs share every bit.
__device__ __forceinline__ uint16_t swiglu_bf16(uint16_t gb, uint16_t ub) {
  const float g = bf16_to_f32(gb);
  const float u = bf16_to_f32(ub);
  const float e = __builtin_amdgcn_exp2f(-g * 1.44269502f);
  const float silu = g / (1.0f + e);
  return f32_to_bf16(silu * u);
}

// RoPE of the rotate-half pair (j, j + D/2) at position pos: the angle pos * base^(-2j/D)
// in fp64, its cosine and sine each rounded to fp32, then y1 = x1 c - x2 s and
// y2 = x2 c + x1 s from separately rounded fp32 products.  bi_rope_qkv and the fused
// RoPE + cache write both call these, so their q and k share every bit.
__device__ __forceinline__ void rope_cos_sin(int pos, int j, int hd, double base, float& c, float& s) {
  const double inv = pow(base, -2.0 * j / hd);
  const double ang = static_cast<double>(pos) * inv;
  c = static_cast<float>(cos(ang));
  s = static_cast<float>(sin(ang));
}
__device__ __forceinline__ void rope_rotate(float x1, float x2, float c, float s, float& y1, float& y2) {
  y1 = x1 * c - x2 * s;
  y2 = x2 * c + x1 * s;
}

__device__ __forceinline__ float wave_xor(float v, int off) { return __shfl_xor(v, off, kWave); }

// Butterfly over the 64 lanes with offsets 1, 2, 4, 8, 16, 32.  fp32 addition is
// commutative, so every lane ends with the index-order pairwise tree sum.
__device__ __forceinline__ float wave_tree_sum(float v) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) v = v + wave_xor(v, off);
  return v;
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Compute units of the current device, read once per device (256 when unknown).
inline int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cached[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v < 1)
    v = 256;
  cached[dev].store(v, std::memory_order_relaxed);
  return v;
}

inline int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? BI_OK : BI_ERR_HIP;
}

}  // namespace bi
