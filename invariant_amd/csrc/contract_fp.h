// The fp32 functions whose results are part of the library's contract, bit for bit: the
// EXP and LOG of the log-softmax head and the scale of RMSNorm.  Every operation is a
// separately rounded IEEE fp32 operation (the library is built with -ffp-contract=off and
// correctly rounded division and square root), so any IEEE machine can replay them.
// Included by the kernels that use them and by the test library that sweeps them.
#pragma once

#include "bi_common.h"

namespace bi {

// EXP(d), d <= 0 or NaN: Cody & Waite (1980) reduction d = k ln2 + r with ln2 split into a
// 16-significant-bit head (k * head is exact) and a rounded tail; exp(r) by the Taylor
// polynomial of degree 7 (coefficients 1/n! rounded to binary32) in Horner form; result
// p * 2^k from exponent bits; k < -125 gives +0.
// LOG(s), s >= 1: s = 2^e f, f moved into [sqrt(1/2), sqrt(2)); log f =
// z (2 + 2/3 z^2 + ... + 2/15 z^14), z = (f - 1)/(f + 1) (J.-M. Muller, Elementary
// Functions, range reduction and the atanh series); e ln2 added head then tail.
// Constants (binary32 bit patterns): 1/ln2 = 0x3fb8aa3b; ln2 head = 0x3f317200 (ln 2
// rounded to 16 significant bits), ln2 tail = 0x35bfbe8e; sqrt 2 = 0x3fb504f3;
// 1/n! for n = 0..7 and 2/(2i+1) for i = 0..7 rounded to nearest.
__device__ __forceinline__ float f32c(uint32_t b) { return __uint_as_float(b); }

__device__ __forceinline__ float exp_cw(float d) {
  // branch-free form of the same steps: k outside [-125, 0] and NaN are selected away at
  // the end, after computing with a clamped k
  const float t = d * f32c(0x3fb8aa3bu);
  const float k = __builtin_rintf(t);
  const float kc = fmaxf(k, -126.0f);
  float r = d - kc * f32c(0x3f317200u);
  r = r - kc * f32c(0x35bfbe8eu);
  float p = f32c(0x39500d01u);       // 1/5040
  p = p * r + f32c(0x3ab60b61u);     // 1/720
  p = p * r + f32c(0x3c088889u);     // 1/120
  p = p * r + f32c(0x3d2aaaabu);     // 1/24
  p = p * r + f32c(0x3e2aaaabu);     // 1/6
  p = p * r + f32c(0x3f000000u);     // 1/2
  p = p * r + f32c(0x3f800000u);     // 1
  p = p * r + f32c(0x3f800000u);     // 1
  const int ki = static_cast<int>(kc);
  const float res = p * __int_as_float((ki + 127) << 23);
  const float live = (k >= -125.0f) ? res : 0.0f;
  return (d != d) ? d : live;
}

__device__ __forceinline__ float log_at(float s) {
  if (!__builtin_isfinite(s)) return s;
  const uint32_t b = __float_as_uint(s);
  int e = static_cast<int>(b >> 23) - 127;
  float f = __uint_as_float((b & 0x7fffffu) | 0x3f800000u);
  if (f > f32c(0x3fb504f3u)) {
    f = f * 0.5f;
    e += 1;
  }
  const float z = (f - 1.0f) / (f + 1.0f);
  const float w = z * z;
  float q = f32c(0x3e088889u);       // 2/15
  q = q * w + f32c(0x3e1d89d9u);     // 2/13
  q = q * w + f32c(0x3e3a2e8cu);     // 2/11
  q = q * w + f32c(0x3e638e39u);     // 2/9
  q = q * w + f32c(0x3e924925u);     // 2/7
  q = q * w + f32c(0x3ecccccdu);     // 2/5
  q = q * w + f32c(0x3f2aaaabu);     // 2/3
  q = q * w + f32c(0x40000000u);     // 2
  const float lf = z * q;
  const float ef = static_cast<float>(e);
  return ef * f32c(0x3f317200u) + (ef * f32c(0x35bfbe8eu) + lf);
}

// RMSNorm's scale of a row whose squares sum to ssum over D elements:
// r = 1 / sqrt(ssum / D + eps), each of the four operations rounded on its own (the divide
// and the square root correctly rounded).
__device__ __forceinline__ float rms_scale(float ssum, int D, float eps) {
  const float mean = ssum / static_cast<float>(D);
  const float var = mean + eps;
  return 1.0f / __builtin_sqrtf(var);
}

}  // namespace bi
