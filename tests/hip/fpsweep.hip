// Test-only HIP library: the fp32 functions of the library's contract (contract_fp.h, the
// same source the kernels include) evaluated on every float of a bit-pattern range, for
// exhaustive comparison with the oracle's replay on the host.  Not part of the product
// ABI; built with the product's flags (correctly rounded divide and square root, no
// contraction, denormals kept).
#include "../../invariant_amd/csrc/contract_fp.h"

namespace {

enum { kExp = 0, kLog = 1, kSqrt = 2, kRcp = 3, kDiv14336 = 4 };

__global__ void sweep_kernel(uint32_t first, int64_t n, int fn, float* __restrict__ out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float x = __uint_as_float(first + static_cast<uint32_t>(i));
  float y;
  switch (fn) {
    case kExp: y = bi::exp_cw(x); break;
    case kLog: y = bi::log_at(x); break;
    case kSqrt: y = __builtin_sqrtf(x); break;        // the operations rms_scale is made of
    case kRcp: y = 1.0f / x; break;
    default: y = x / static_cast<float>(14336); break;
  }
  out[i] = y;
}

// rms_scale itself on given (ssum, D, eps) triples.
__global__ void rms_scale_kernel(const float* __restrict__ ssum, const int* __restrict__ d,
                                 float eps, int64_t n, float* __restrict__ out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) out[i] = bi::rms_scale(ssum[i], d[i], eps);
}

}  // namespace

// out[i] = fn(float with bits first + i), i < n; fn: 0 EXP, 1 LOG, 2 sqrt, 3 1/x, 4 x/14336.
// Returns 0, or -1 for a bad argument, -7 when the launch fails.
extern "C" int fps_sweep(uint32_t first, int64_t n, int fn, float* out, void* stream) {
  if (n < 0 || fn < 0 || fn > 4 || (n > 0 && !out) || n > (int64_t(1) << 32)) return -1;
  if (n == 0) return 0;
  sweep_kernel<<<dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                 reinterpret_cast<hipStream_t>(stream)>>>(first, n, fn, out);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

extern "C" int fps_rms_scale(const float* ssum, const int* d, float eps, int64_t n, float* out,
                             void* stream) {
  if (n < 0 || (n > 0 && (!ssum || !d || !out))) return -1;
  if (n == 0) return 0;
  rms_scale_kernel<<<dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream)>>>(ssum, d, eps, n, out);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}
