// bi_logsoftmax_argmax: greedy-decoding head, one row per workgroup.
//
// Greedy decoding takes the most likely token ("Does the same LLM give different
// outputs on different GPUs? Why?", experiment set-up; "Defeating nondeterminism in
// LLM inference", introduction: temperature 0); token probabilities come from the
// normalised scores.  A near tie decides the token ("Same model, same input,
// different answer", sampling), so the argmax rule is exact: lowest index of the
// maximum, a NaN counting as the maximum and -0 == +0.  That is a selection under a
// total order, so any combination order gives the same index.
//
// The sum of exponentials uses the fixed tree of bi_rmsnorm over 4-element vectors
// (T = min(256, ceil(V/4)) lanes, ascending per lane, wave64 butterfly 1..32, waves
// (w0 + w1) + (w2 + w3)).  EXP and LOG (contract_fp.h) are evaluated with separately
// rounded fp32 operations from published methods, so every bit is reproducible.
#include "contract_fp.h"

namespace bi {

namespace {

constexpr int kThreads = 256;

// (value, index) selection: larger value wins, NaN beats numbers, equal -> lower index.
__device__ __forceinline__ void pick(float& bv, int& bi, float v, int i) {
  const bool bn = bv != bv, vn = v != v;
  const bool gt = v > bv, lt = v < bv, lower = i < bi;
  const bool take = (vn && !bn) || (!vn && !bn && (gt || (!lt && lower))) || (vn && bn && lower);
  bv = take ? v : bv;
  bi = take ? i : bi;
}

template <bool FULL>
__device__ __forceinline__ void load4(const float* row, int v, int V, bool vec, float (&e)[4]) {
  const float* p = row + static_cast<int64_t>(v) * 4;
  if (FULL || (vec && v * 4 + 4 <= V)) {
    floatx4 q = *reinterpret_cast<const floatx4*>(p);
    e[0] = q[0]; e[1] = q[1]; e[2] = q[2]; e[3] = q[3];
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) e[i] = (v * 4 + i < V) ? p[i] : 0.f;
  }
}

// The first NVC vectors of every lane stay in registers across the three passes (all of
// a 32768-wide row); longer rows re-read the rest.  Only where the values live changes, not
// the order in which they are combined.
constexpr int NVC = 32;

// FULL: every 4-element vector lies inside the row and rows are 16-byte aligned, so no
// element needs a bounds check (V % 4 == 0, aligned pointers and ld).
template <bool FULL>
__global__ __launch_bounds__(kThreads) void logsoftmax_argmax_kernel(
    const float* __restrict__ logits, int V, int64_t ld, float* __restrict__ logprobs,
    int32_t* __restrict__ argmax, int vec_in, int vec_out) {
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int nvec = (V + 3) / 4;
  const int T = nvec < kThreads ? nvec : kThreads;
  const float* x = logits + row * ld;
  __shared__ float sv[kThreads / kWave];
  __shared__ int si[kThreads / kWave];
  __shared__ float ss[kThreads / kWave];

  float cache[NVC][4];
  if (tid < T) {
#pragma unroll
    for (int j = 0; j < NVC; ++j) {
      const int v = tid + j * T;
      if (v < nvec) load4<FULL>(x, v, V, vec_in, cache[j]);
    }
  }

  // pass 1: maximum and lowest index attaining it
  float bv = -__builtin_huge_valf();
  int bidx = 0x7fffffff;
  if (tid < T) {
#pragma unroll
    for (int j = 0; j < NVC; ++j) {
      const int v = tid + j * T;
      if (v < nvec) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (FULL || v * 4 + i < V) pick(bv, bidx, cache[j][i], v * 4 + i);
      }
    }
    for (int v = tid + NVC * T; v < nvec; v += T) {
      float e[4];
      load4<FULL>(x, v, V, vec_in, e);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (FULL || v * 4 + i < V) pick(bv, bidx, e[i], v * 4 + i);
    }
  }
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const float ov = __shfl_xor(bv, off, kWave);
    const int oi = __shfl_xor(bidx, off, kWave);
    pick(bv, bidx, ov, oi);
  }
  if ((tid & (kWave - 1)) == 0) {
    sv[tid / kWave] = bv;
    si[tid / kWave] = bidx;
  }
  __syncthreads();
  float mv = sv[0];
  int mi = si[0];
#pragma unroll
  for (int w = 1; w < kThreads / kWave; ++w) pick(mv, mi, sv[w], si[w]);
  const float m = mv;

  // pass 2: s = tree sum of EXP(x - m), each lane in ascending element order
  float acc = 0.f;
  if (tid < T) {
#pragma unroll
    for (int j = 0; j < NVC; ++j) {
      const int v = tid + j * T;
      if (v < nvec) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (FULL || v * 4 + i < V) acc = acc + exp_cw(cache[j][i] - m);
      }
    }
    for (int v = tid + NVC * T; v < nvec; v += T) {
      float e[4];
      load4<FULL>(x, v, V, vec_in, e);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (FULL || v * 4 + i < V) acc = acc + exp_cw(e[i] - m);
    }
  }
  const float wsum = wave_tree_sum(acc);
  if ((tid & (kWave - 1)) == 0) ss[tid / kWave] = wsum;
  __syncthreads();
  const float s = (ss[0] + ss[1]) + (ss[2] + ss[3]);
  const float L = log_at(s);

  if (tid == 0) argmax[row] = mi;
  if (logprobs == nullptr || tid >= T) return;
  float* out = logprobs + row * ld;
  auto emit = [&](int v, const float (&e)[4]) {
    float o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = (e[i] - m) - L;
    if ((FULL && vec_out) || (vec_out && v * 4 + 4 <= V)) {
      floatx4 q;
      q[0] = o[0]; q[1] = o[1]; q[2] = o[2]; q[3] = o[3];
      *reinterpret_cast<floatx4*>(out + static_cast<int64_t>(v) * 4) = q;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (v * 4 + i < V) out[static_cast<int64_t>(v) * 4 + i] = o[i];
    }
  };
#pragma unroll
  for (int j = 0; j < NVC; ++j) {
    const int v = tid + j * T;
    if (v < nvec) emit(v, cache[j]);
  }
  for (int v = tid + NVC * T; v < nvec; v += T) {
    float e[4];
    load4<FULL>(x, v, V, vec_in, e);
    emit(v, e);
  }
}

// Wide form for rows of 1024 .. 32768 elements (V % 4 == 0, 16-byte aligned rows): the same
// tree with its elementwise work spread over four times the threads.  Thread (g, t),
// g = tid / 256, holds vectors j = 8 g .. 8 g + 7 of tree lane t (vector t + 256 j), takes
// their maximum and their EXP values, and parks the EXP values in LDS; tree lane t (g = 0)
// then adds its own 4 x 32 values in the same ascending order as above.  The maximum is a
// selection under a total order, so splitting it changes nothing either: the bits equal
// the one-row-per-256-threads form.
constexpr int kWideGroups = 4;
constexpr int kWideThreads = kWideGroups * kThreads;
constexpr int kWideJ = NVC / kWideGroups;   // vectors per thread

__global__ __launch_bounds__(kWideThreads) void logsoftmax_argmax_wide_kernel(
    const float* __restrict__ logits, int V, int64_t ld, float* __restrict__ logprobs,
    int32_t* __restrict__ argmax) {
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int t = tid % kThreads, g = tid / kThreads;
  const int nvec = V / 4;                     // kThreads <= nvec <= NVC * kThreads
  const float* x = logits + row * ld;
  __shared__ floatx4 se[NVC * kThreads];     // EXP values, vector j of lane t at j * 256 + t
  __shared__ float sv[kWideThreads / kWave];
  __shared__ int si[kWideThreads / kWave];
  __shared__ float ss[kThreads / kWave];

  float c[kWideJ][4];
#pragma unroll
  for (int jj = 0; jj < kWideJ; ++jj) {
    const int v = t + (g * kWideJ + jj) * kThreads;
    if (v < nvec) {
      const floatx4 q = *reinterpret_cast<const floatx4*>(x + static_cast<int64_t>(v) * 4);
      c[jj][0] = q[0]; c[jj][1] = q[1]; c[jj][2] = q[2]; c[jj][3] = q[3];
    }
  }
  float bv = -__builtin_huge_valf();
  int bidx = 0x7fffffff;
#pragma unroll
  for (int jj = 0; jj < kWideJ; ++jj) {
    const int v = t + (g * kWideJ + jj) * kThreads;
    if (v < nvec) {
#pragma unroll
      for (int i = 0; i < 4; ++i) pick(bv, bidx, c[jj][i], v * 4 + i);
    }
  }
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const float ov = __shfl_xor(bv, off, kWave);
    const int oi = __shfl_xor(bidx, off, kWave);
    pick(bv, bidx, ov, oi);
  }
  if ((tid & (kWave - 1)) == 0) {
    sv[tid / kWave] = bv;
    si[tid / kWave] = bidx;
  }
  __syncthreads();
  float mv = sv[0];
  int mi = si[0];
#pragma unroll
  for (int w = 1; w < kWideThreads / kWave; ++w) pick(mv, mi, sv[w], si[w]);
  const float m = mv;

#pragma unroll
  for (int jj = 0; jj < kWideJ; ++jj) {
    const int j = g * kWideJ + jj;
    if (t + j * kThreads < nvec) {
      floatx4 e;
#pragma unroll
      for (int i = 0; i < 4; ++i) e[i] = exp_cw(c[jj][i] - m);
      se[j * kThreads + t] = e;
    }
  }
  __syncthreads();
  if (g == 0) {
    float acc = 0.f;
    for (int j = 0; j < NVC; ++j) {
      if (t + j * kThreads >= nvec) break;
      const floatx4 e = se[j * kThreads + t];
      acc = acc + e[0];
      acc = acc + e[1];
      acc = acc + e[2];
      acc = acc + e[3];
    }
    const float wsum = wave_tree_sum(acc);
    if ((tid & (kWave - 1)) == 0) ss[tid / kWave] = wsum;
  }
  __syncthreads();
  const float s = (ss[0] + ss[1]) + (ss[2] + ss[3]);
  const float L = log_at(s);

  if (tid == 0) argmax[row] = mi;
  if (logprobs == nullptr) return;
  float* out = logprobs + row * ld;
#pragma unroll
  for (int jj = 0; jj < kWideJ; ++jj) {
    const int v = t + (g * kWideJ + jj) * kThreads;
    if (v < nvec) {
      floatx4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = (c[jj][i] - m) - L;
      *reinterpret_cast<floatx4*>(out + static_cast<int64_t>(v) * 4) = o;
    }
  }
}

// Argmax alone (logprobs NULL) for the rows the wide form takes: no EXP or LOG is needed,
// and the maximum is found in two cheap passes instead of the sequential pick: the largest
// value and whether a NaN is present, then the lowest index holding that value (-0 == +0)
// or the lowest NaN.  Thread t holds vectors t + 256 j.  The index equals the pick's.
__global__ __launch_bounds__(kThreads) void argmax_rows_kernel(const float* __restrict__ logits,
                                                               int V, int64_t ld,
                                                               int32_t* __restrict__ argmax) {
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int u = tid % kWave, g = tid / kWave;
  const int nvec = V / 4;                 // kThreads <= nvec <= NVC * kThreads
  const float* x = logits + row * ld;
  __shared__ float smax[kThreads / kWave];
  __shared__ int sflag[kThreads / kWave];
  __shared__ int sidx[kThreads / kWave];

  float c[NVC][4];
#pragma unroll
  for (int j = 0; j < NVC; ++j) {
    const int v = tid + j * kThreads;
    if (v < nvec) {
      const floatx4 e = *reinterpret_cast<const floatx4*>(x + static_cast<int64_t>(v) * 4);
      c[j][0] = e[0]; c[j][1] = e[1]; c[j][2] = e[2]; c[j][3] = e[3];
    }
  }
  float mx = -__builtin_huge_valf();
  int nan = 0;
#pragma unroll
  for (int j = 0; j < NVC; ++j)
    if (tid + j * kThreads < nvec) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        mx = fmaxf(mx, c[j][i]);
        nan |= c[j][i] != c[j][i];
      }
    }
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    mx = fmaxf(mx, __shfl_xor(mx, off, kWave));
    nan |= __shfl_xor(nan, off, kWave);
  }
  if (u == 0) {
    smax[g] = mx;
    sflag[g] = nan;
  }
  __syncthreads();
  mx = fmaxf(fmaxf(smax[0], smax[1]), fmaxf(smax[2], smax[3]));
  const bool any_nan = (sflag[0] | sflag[1] | sflag[2] | sflag[3]) != 0;

  int best = 0x7fffffff;
#pragma unroll
  for (int j = 0; j < NVC; ++j) {
    const int v = tid + j * kThreads;
    if (v < nvec) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = c[j][i];
        const bool hit = any_nan ? (e != e) : (e == mx);
        best = hit ? min(best, v * 4 + i) : best;
      }
    }
  }
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) best = min(best, __shfl_xor(best, off, kWave));
  if (u == 0) sidx[g] = best;
  __syncthreads();
  if (tid == 0) argmax[row] = min(min(sidx[0], sidx[1]), min(sidx[2], sidx[3]));
}

}  // namespace
}  // namespace bi

using namespace bi;

extern "C" int bi_logsoftmax_argmax(const float* logits, int64_t M, int64_t V, int64_t ld,
                                    float* logprobs, int32_t* argmax, void* stream) {
  if (M < 0 || V < 0) return BI_ERR_SHAPE;
  if (M == 0) return BI_OK;
  if (V < 1 || ld < V || V > 0x7ffffff0LL || M > 0x7fffffffLL) return BI_ERR_SHAPE;
  if (!logits || !argmax) return BI_ERR_NULL;
  // 16-byte vector accesses where rows allow them; element accesses otherwise (same math)
  const int vec_in = aligned16(logits) && (ld % 4) == 0;
  const int vec_out = logprobs && aligned16(logprobs) && (ld % 4) == 0;
  const bool full = vec_in && (V % 4) == 0 && (!logprobs || vec_out);
  if (logprobs) {
    // outputs must not alias inputs (rows past the register cache are read twice)
    const int64_t extent = (M - 1) * ld + V;
    if (logprobs < logits + extent && logits < logprobs + extent) return BI_ERR_SHAPE;
  }
  if (full && !logprobs && V >= 4 * kThreads && V <= 4 * NVC * kThreads)
    argmax_rows_kernel<<<dim3(static_cast<unsigned>(M)), dim3(kThreads), 0, as_stream(stream)>>>(
        logits, static_cast<int>(V), ld, argmax);
  else if (full && V >= 4 * kThreads && V <= 4 * NVC * kThreads)
    logsoftmax_argmax_wide_kernel<<<dim3(static_cast<unsigned>(M)), dim3(kWideThreads), 0,
                                    as_stream(stream)>>>(logits, static_cast<int>(V), ld,
                                                         logprobs, argmax);
  else if (full)
    logsoftmax_argmax_kernel<true><<<dim3(static_cast<unsigned>(M)), dim3(kThreads), 0,
                                     as_stream(stream)>>>(logits, static_cast<int>(V), ld,
                                                          logprobs, argmax, vec_in, vec_out);
  else
    logsoftmax_argmax_kernel<false><<<dim3(static_cast<unsigned>(M)), dim3(kThreads), 0,
                                      as_stream(stream)>>>(logits, static_cast<int>(V), ld,
                                                           logprobs, argmax, vec_in, vec_out);
  return launch_status();
}
