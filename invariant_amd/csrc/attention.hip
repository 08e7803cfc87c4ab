// bi_attention: causal GQA attention over a paged KV cache, batch- and
// prefill/decode-invariant.
//
// "Defeating nondeterminism in LLM inference", section on batch-invariant attention:
//  * the K/V cache and the page table are updated BEFORE the attention kernel, so a
//    query token sees its keys laid out the same way however many tokens are in
//    flight (step 1 below runs first, on the same stream);
//  * the reduction order of a token may not depend on how many other tokens of its
//    sequence are processed with it: here the keys of every query are split into
//    chunks of 256 at ABSOLUTE positions [256c, 256c + 256), each chunk is reduced by
//    one workgroup with one fixed instruction sequence (chunk_partial), and the chunk
//    partials are merged in ascending c (merge_step).  Split-KV decode and the prefill
//    walk call exactly these two routines, so a token's bits never depend on the path,
//    the batch, its neighbours or the physical pages.
//
// Per chunk (one workgroup of 4 waves, 16 query columns; GQA: every column of a
// workgroup reads the same kv head; wave w owns the 64 keys [64w, 64w + 64)):
//   S^T = K . Q^T   4 tiles of v_mfma_f32_16x16x32_bf16 per wave (keys x columns), the
//                   d-sum over 4 instructions in ascending order;
//   t = S * (scale * log2 e), masked to -inf beyond the query position;
//   m_c = max t over the chunk (the 4 wave maxima exchanged through LDS);
//   P = 2^(t - m_c) (v_exp_f32);  per wave: l_w = sum P (per-lane ascending, then lanes
//   (g0 + g1) + (g2 + g3)) and O_w^T = V^T . P^T over its two 32-key slices, P split into
//   bf16 hi + lo (two instructions per slice, hi first, one fp32 accumulation chain);
//   l_c = (l_0 + l_1) + (l_2 + l_3),  o_c = (O_0 + O_1) + (O_2 + O_3).
//   Rounding P itself to bf16 would cost tens of bf16 ulps in the output; hi + lo keeps
//   16 bits.
// Merge, in two fixed levels set by absolute positions only: the chunks of each group of
// GROUP = 4 (keys [1024g, 1024g + 1024)) are merged in ascending c, then the groups in
// ascending g; each level copies its first partial and then applies
//   m' = max(m, m_c); a = 2^(m - m'); b = 2^(m_c - m');  l' = a l + b l_c;  o' = a o + b o_c,
// and out = o / l.  Split-KV decode writes one partial per group (a quarter of the
// per-chunk partials' bytes), or, when that leaves fewer work units than two per CU, one
// per chunk, whose first level the combine kernel then applies; the prefill walk applies
// the same two levels in registers.
//
// Cache layout, chosen so every matrix-operand load of a wave covers whole 128-byte
// lines:
//   k_cache [page][kv head][16 d-groups][slot'][8]: d-group j holds d = 8j .. 8j+7 of
//           every slot; inside each aligned block of 16 slots the slot order is
//           s' = s with bits 2 and 3 swapped (0-3, 8-11, 4-7, 12-15), which puts the 8
//           keys one matrix instruction reads from a page next to each other;
//   v_cache [page][kv head][128 d][slot]  (V transposed, slots in order).
#include <algorithm>

#include "bi_common.h"

namespace bi {
namespace {

constexpr int CHUNK = 256;
constexpr int GROUP = 4;                // chunks per merge group (1024 keys at absolute positions)
constexpr int HD = 128;
constexpr int SPLIT_MAX_TOKENS = 1024;  // calls with more tokens walk chunks in registers

__device__ __forceinline__ bf16x8 as_bf16x8(u16x8 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ floatx4 mfma16(u16x8 a, u16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Largest b < batch with qsl[b] <= t, by a 64-way search (one probe per lane and a
// ballot per step).  Wave-uniform t required; qsl is non-decreasing with qsl[0] = 0.
__device__ __forceinline__ int find_seq_wave(const int32_t* qsl, int batch, int t) {
  const int lane = threadIdx.x & 63;
  int lo = 0, n = batch;
  while (n > 1) {
    const int step = (n + 63) / 64;
    const bool ok = lane * step < n && qsl[lo + lane * step] <= t;
    const unsigned long long m = __ballot(ok);
    const int k = 63 - __clzll(m);
    lo += k * step;
    n = min(step, n - k * step);
  }
  return lo;
}

// Physical slot of logical slot s inside a K page: bits 2 and 3 swapped.
__device__ __forceinline__ int k_slot(int s) {
  return (s & ~12) | ((s & 4) << 1) | ((s & 8) >> 1);
}

__device__ __forceinline__ int find_seq(const int32_t* qsl, int batch, int t) {
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (qsl[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

struct Seq {
  const uint16_t* kc;   // k_cache base
  const uint16_t* vc;   // v_cache base
  const int32_t* bt;    // block-table row of the sequence
  int ps;               // page size (a power of two)
  int hkv, kvh;
  int seq_len;
  int maxp;             // columns of the block table (pages per sequence)
  int ps_shift;         // log2(ps)
};

// Exchange area of one workgroup for one chunk.
struct ChunkLDS {
  float mx[4][16];
  float l[4][16];
  floatx4 o[4][8][64];
};

// The reduction of one 256-key chunk for the workgroup's 16 columns, in phases (all 4
// waves call each phase together): the page ids, the K and V operand loads, the scores
// with the chunk maximum and P, and the values with the workgroup sums.  chunk_partial
// runs them back to back; the split kernel interleaves them with the loads of its next
// chunk.  The operations of a chunk, and so its bits, are the same either way.

// Physical page of chunk page l, held by lane l (0 for lanes past the chunk's pages and
// for pages past the sequence: page 0 always exists, its data is masked out).
__device__ __forceinline__ int chunk_pages(const Seq& sq, int c) {
  const int lane = threadIdx.x & 63;
  const int ppc = CHUNK >> sq.ps_shift;
  const int l = lane < ppc ? lane : 0;
  const int pg = sq.bt[min(max(c * ppc + l, 0), sq.maxp - 1)];
  return (lane < ppc && c * CHUNK + lane * sq.ps < sq.seq_len) ? pg : 0;
}

// 16 bytes of the K/V cache.  Every cache byte is read once per call, so the loads are
// non-temporal: they do not displace the partial results, page table and queries from
// the caches (without the hint, the partials written back under the K/V stream cost
// about a tenth of the call).
__device__ __forceinline__ u16x8 stream_load(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u16x8*>(p));
}

// K operands of this wave's 64 keys (4 tiles of 16 keys x 4 d-steps).  Every address is
// inside the cache: a key past the sequence reads a slot of its page that holds no key yet,
// or page 0; its score is masked to -inf later.
__device__ __forceinline__ void chunk_load_k(const Seq& sq, int pg, u16x8 (&kop)[2][2][4]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int kr0 = 8 * (i >> 2) + (i & 3);           // key of MFMA row i in the first tile of a pair
  const int64_t page_elems = static_cast<int64_t>(sq.ps) * HD;
#pragma unroll
  for (int uu = 0; uu < 2; ++uu) {
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int kk = 32 * (2 * w + uu) + kr0 + 4 * h2;   // chunk-relative key of this lane's row
      const int phys = __shfl(pg, kk >> sq.ps_shift, 64);
      const uint16_t* kp = sq.kc + (static_cast<int64_t>(phys) * sq.hkv + sq.kvh) * page_elems +
                           ((4 * g) * sq.ps + k_slot(kk & (sq.ps - 1))) * 8;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        kop[uu][h2][t] = stream_load(kp + static_cast<int64_t>(t) * sq.ps * 8);
    }
  }
}

// V^T operands of this wave's two 32-key slices (masked later, in chunk_values).
__device__ __forceinline__ void chunk_load_v(const Seq& sq, int pg, u16x8 (&vop)[2][8]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int64_t page_elems = static_cast<int64_t>(sq.ps) * HD;
#pragma unroll
  for (int uu = 0; uu < 2; ++uu) {
    const int kk0 = 32 * (2 * w + uu) + 8 * g;      // first of this lane's 8 keys
    const int phys = __shfl(pg, kk0 >> sq.ps_shift, 64);
    const uint16_t* vbase =
        sq.vc + (static_cast<int64_t>(phys) * sq.hkv + sq.kvh) * page_elems + (kk0 & (sq.ps - 1));
#pragma unroll
    for (int db = 0; db < 8; ++db)
      vop[uu][db] = stream_load(vbase + static_cast<int64_t>(16 * db + i) * sq.ps);
  }
}

// Keep every load issued so far above this point: the scheduler would otherwise sink
// loads next to their uses and leave one or two in flight.
__device__ __forceinline__ void issue_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// S = K Q^T for this wave's keys (q as NQ bf16 terms: 1, or hi, mid, lo of an fp32 q,
// each 32-wide d step accumulating its terms in that order), scaled to log2 units and masked
// beyond the column's position; m = the chunk maximum of column lane % 16 (the 4 wave maxima exchanged
// through LDS); on return s holds P = 2^(t - m) and lsum this wave's sum of P.
template <int NQ>
__device__ __forceinline__ void chunk_scores(int c, const u16x8 (&kop)[2][2][4], const u16x8 (&qop)[NQ][4],
                                             int pcol, float sl2, ChunkLDS& sh, floatx4 (&s)[2][2],
                                             float& m, float& lsum) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int c0 = c * CHUNK;
#pragma unroll
  for (int uu = 0; uu < 2; ++uu) {
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int j = 0; j < NQ; ++j) acc = mfma16(kop[uu][h2][t], qop[j][t], acc);
      s[uu][h2] = acc;
    }
  }
  float mx = -__builtin_huge_valf();
#pragma unroll
  for (int uu = 0; uu < 2; ++uu)
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kp = c0 + 32 * (2 * w + uu) + 8 * g + 4 * h2 + r;
        const float t = s[uu][h2][r] * sl2;
        s[uu][h2][r] = (kp <= pcol) ? t : -__builtin_huge_valf();
        mx = fmaxf(mx, s[uu][h2][r]);
      }
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  if (g == 0) sh.mx[w][i] = mx;
  __syncthreads();
  m = fmaxf(fmaxf(sh.mx[0][i], sh.mx[1][i]), fmaxf(sh.mx[2][i], sh.mx[3][i]));

  lsum = 0.f;
#pragma unroll
  for (int uu = 0; uu < 2; ++uu)
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kp = c0 + 32 * (2 * w + uu) + 8 * g + 4 * h2 + r;
        const float p = (kp <= pcol) ? exp2_hw(s[uu][h2][r] - m) : 0.f;
        s[uu][h2][r] = p;
        lsum = lsum + p;
      }
  lsum = lsum + __shfl_xor(lsum, 16, 64);
  lsum = lsum + __shfl_xor(lsum, 32, 64);
}

// O_w^T = V^T . P^T over this wave's two 32-key slices (V past the sequence zeroed, P
// split into bf16 hi + lo), then l_c = (l_0 + l_1) + (l_2 + l_3) and
// o_c = (O_0 + O_1) + (O_2 + O_3) through LDS.  Returns, in every wave, m_c and l_c of
// column lane % 16 and, in wave w, o_c for d-blocks 2w and 2w + 1 in the MFMA output
// layout (oc[j][r] is d = 16 (2w + j) + 4 (lane / 16) + r).
__device__ __forceinline__ void chunk_values(const Seq& sq, int c, u16x8 (&vop)[2][8],
                                             const floatx4 (&s)[2][2], float m, float lsum,
                                             ChunkLDS& sh, float& m_c, float& l_c, floatx4 (&oc)[2]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int c0 = c * CHUNK;
  if (c0 + 64 * (w + 1) > sq.seq_len) {   // this wave's keys reach past the sequence
#pragma unroll
    for (int uu = 0; uu < 2; ++uu) {
      const int nvalid = sq.seq_len - (c0 + 32 * (2 * w + uu) + 8 * g);   // keys kk0 + e valid for e < nvalid
      u32x4 keep;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        keep[k] = (2 * k < nvalid ? 0x0000ffffu : 0u) | (2 * k + 1 < nvalid ? 0xffff0000u : 0u);
#pragma unroll
      for (int db = 0; db < 8; ++db)
        vop[uu][db] = __builtin_bit_cast(u16x8, __builtin_bit_cast(u32x4, vop[uu][db]) & keep);
    }
  }
  floatx4 o[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) o[db] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int uu = 0; uu < 2; ++uu) {
    // P = hi + lo, both rounded to nearest even (v_cvt_pk_bf16_f32 converts two at a time)
    u32x4 hi, lo;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int r = 0; r < 4; r += 2) {
        const floatx2 p = {s[uu][h2][r], s[uu][h2][r + 1]};
        const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf16x2));
        const floatx2 back = {__uint_as_float(h << 16), __uint_as_float(h & 0xffff0000u)};
        hi[2 * h2 + r / 2] = h;
        lo[2 * h2 + r / 2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(p - back, bf16x2));
      }
    const u16x8 phi = __builtin_bit_cast(u16x8, hi), plo = __builtin_bit_cast(u16x8, lo);
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      o[db] = mfma16(vop[uu][db], phi, o[db]);
      o[db] = mfma16(vop[uu][db], plo, o[db]);
    }
  }
  if (g == 0) sh.l[w][i] = lsum;
#pragma unroll
  for (int db = 0; db < 8; ++db) sh.o[w][db][lane] = o[db];
  __syncthreads();
  l_c = (sh.l[0][i] + sh.l[1][i]) + (sh.l[2][i] + sh.l[3][i]);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int db = 2 * w + j;
    oc[j] = (sh.o[0][db][lane] + sh.o[1][db][lane]) + (sh.o[2][db][lane] + sh.o[3][db][lane]);
  }
  m_c = m;
}

// One 256-key chunk, phases back to back.  pcol: absolute position of this lane's column
// (-1: unused column).  K is loaded first: loads complete in order, so the scores are
// computed while V is still arriving.
template <int NQ>
__device__ __forceinline__ void chunk_partial(const Seq& sq, int c, const u16x8 (&qop)[NQ][4], int pcol,
                                              float sl2, ChunkLDS& sh, float& m_c, float& l_c,
                                              floatx4 (&oc)[2]) {
  const int pg = chunk_pages(sq, c);
  u16x8 kop[2][2][4], vop[2][8];
  chunk_load_k(sq, pg, kop);
  chunk_load_v(sq, pg, vop);
  issue_fence();
  floatx4 s[2][2];
  float m, lsum;
  chunk_scores(c, kop, qop, pcol, sl2, sh, s, m, lsum);
  chunk_values(sq, c, vop, s, m, lsum, sh, m_c, l_c, oc);
}

__device__ __forceinline__ void merge_step(float& m, float& l, float mc, float lc, float& a,
                                           float& b) {
  const float mn = fmaxf(m, mc);
  a = exp2_hw(m - mn);
  b = exp2_hw(mc - mn);
  l = a * l + b * lc;
  m = mn;
}

__device__ __forceinline__ float mix(float o, float oc, float a, float b) { return a * o + b * oc; }

// Q operand of one column: q[token][head][32 g + 8 t .. + 7] for t = 0..3; NQ = 1: q is bf16,
// NQ = 3: q is fp32, split exactly into bf16 hi, mid, lo.
template <int NQ>
__device__ __forceinline__ void load_q_at(const void* q, int64_t token, int head, int hq,
                                          u16x8 (&qop)[NQ][4]) {
  const int g = (threadIdx.x & 63) >> 4;
  const int64_t off = (token * hq + head) * HD + 32 * g;
  if constexpr (NQ == 1) {
    const uint16_t* p = static_cast<const uint16_t*>(q) + off;
#pragma unroll
    for (int t = 0; t < 4; ++t) qop[0][t] = *reinterpret_cast<const u16x8*>(p + 8 * t);
  } else {
    static_assert(NQ == 3, "bf16 or fp32 q");
    const float* p = static_cast<const float*>(q) + off;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const floatx4 x0 = *reinterpret_cast<const floatx4*>(p + 8 * t);
      const floatx4 x1 = *reinterpret_cast<const floatx4*>(p + 8 * t + 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint16_t h, m, l;
        split_bf16x3(e < 4 ? x0[e] : x1[e - 4], h, m, l);
        qop[0][t][e] = h;
        qop[1][t][e] = m;
        qop[2][t][e] = l;
      }
    }
  }
}

template <int NQ>
__device__ __forceinline__ void load_q(const void* q, int64_t token, int head, int hq, bool ok,
                                       u16x8 (&qop)[NQ][4]) {
  if (ok) {
    load_q_at<NQ>(q, token, head, hq, qop);
  } else {
#pragma unroll
    for (int j = 0; j < NQ; ++j)
#pragma unroll
      for (int t = 0; t < 4; ++t) qop[j][t] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
  }
}

// ---------------------------------------------------------------- step 1: cache write
// (not launched when the call's keys and values were written by rope_kv_write_kernel)
__global__ __launch_bounds__(256) void kv_write_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    uint16_t* __restrict__ kc, uint16_t* __restrict__ vc, const int32_t* __restrict__ bt,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ qsl, int batch,
    int max_pages, int hkv, int ps, int4* __restrict__ tok) {
  const int t = blockIdx.x;
  const int b = find_seq_wave(qsl, batch, t);
  const int pos = seq_lens[b] - (qsl[b + 1] - qsl[b]) + (t - qsl[b]);
  if (tok && threadIdx.x == 0) tok[t] = make_int4(b, pos, seq_lens[b], 0);
  const int phys = bt[static_cast<int64_t>(b) * max_pages + pos / ps];
  const int slot = pos % ps;
  const int nvec = hkv * HD / 8;
  for (int v = threadIdx.x; v < 2 * nvec; v += blockDim.x) {
    const bool is_v = v >= nvec;
    const int vv = is_v ? v - nvec : v;
    const int head = vv / (HD / 8), d0 = (vv % (HD / 8)) * 8;
    const int64_t src = (static_cast<int64_t>(t) * hkv + head) * HD + d0;
    const int64_t pg = (static_cast<int64_t>(phys) * hkv + head) * ps * HD;
    if (!is_v) {
      *reinterpret_cast<u16x8*>(kc + pg + (static_cast<int64_t>(d0 / 8) * ps + k_slot(slot)) * 8) =
          *reinterpret_cast<const u16x8*>(k_new + src);
    } else {
      const u16x8 x = *reinterpret_cast<const u16x8*>(v_new + src);
#pragma unroll
      for (int e = 0; e < 8; ++e) vc[pg + static_cast<int64_t>(d0 + e) * ps + slot] = x[e];
    }
  }
}

// ---------------------------------------------------------------- step 1 fused with RoPE
// One workgroup per token: RoPE of its q and k heads, q stored to [T, Hq, D], the rotated k
// and the v of the fused projection written straight into the token's page slot (no
// [T, Hkv, D] k or v tensor is written and read back).  The rotation position is the
// token's cache position (seq_len - new tokens of its sequence + its index among them);
// cosines and sines come from rope_cos_sin, once per pair index, and every element is
// rope_rotate's, so q and the cache hold the bits of bi_rope_qkv followed by the cache
// write.  Item (h, g): head h, elements 8g .. 8g + 7 and D/2 + 8g .. + 7, which are
// d-groups g and g + 8 of the K layout.
__device__ __forceinline__ void load8_f32(const void* p, int64_t i, int f32, int vec, float (&x)[8]) {
  if (f32) {
    const float* f = static_cast<const float*>(p) + i;
    if (vec) {
      const floatx4 a = *reinterpret_cast<const floatx4*>(f), c = *reinterpret_cast<const floatx4*>(f + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) { x[e] = a[e]; x[4 + e] = c[e]; }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = f[e];
    }
  } else {
    const uint16_t* h = static_cast<const uint16_t*>(p) + i;
    if (vec) {
      const u16x8 a = *reinterpret_cast<const u16x8*>(h);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = bf16_to_f32(a[e]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = bf16_to_f32(h[e]);
    }
  }
}

__device__ __forceinline__ void store8_f32(void* p, int64_t i, int f32, int vec, const float (&y)[8]) {
  if (f32) {
    float* f = static_cast<float*>(p) + i;
    if (vec) {
      floatx4 a, c;
#pragma unroll
      for (int e = 0; e < 4; ++e) { a[e] = y[e]; c[e] = y[4 + e]; }
      *reinterpret_cast<floatx4*>(f) = a;
      *reinterpret_cast<floatx4*>(f + 4) = c;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = y[e];
    }
  } else {
    uint16_t* h = static_cast<uint16_t*>(p) + i;
    u16x8 a;
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = f32_to_bf16(y[e]);
    if (vec) {
      *reinterpret_cast<u16x8*>(h) = a;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = a[e];
    }
  }
}

__global__ __launch_bounds__(256) void rope_kv_write_kernel(
    const void* __restrict__ qkv, int64_t ld, int qkv_f32, int qkv_vec, void* __restrict__ q, int q_f32,
    int q_vec, uint16_t* __restrict__ kc, uint16_t* __restrict__ vc, const int32_t* __restrict__ bt,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ qsl, int batch, int max_pages,
    int hq, int hkv, int ps, double base) {
  constexpr int HALF = HD / 2;
  const int t = blockIdx.x;
  const int b = find_seq_wave(qsl, batch, t);
  const int pos = seq_lens[b] - (qsl[b + 1] - qsl[b]) + (t - qsl[b]);
  __shared__ float cs[2][HALF];
  if (threadIdx.x < HALF) rope_cos_sin(pos, threadIdx.x, HD, base, cs[0][threadIdx.x], cs[1][threadIdx.x]);
  __syncthreads();
  const int phys = bt[static_cast<int64_t>(b) * max_pages + pos / ps];
  const int slot = pos % ps;
  const int64_t row = static_cast<int64_t>(t) * ld;
  for (int it = threadIdx.x; it < (hq + 2 * hkv) * 8; it += blockDim.x) {
    const int h = it >> 3, g = it & 7;
    const int64_t src = row + static_cast<int64_t>(h) * HD + 8 * g;
    float x1[8], x2[8];
    load8_f32(qkv, src, qkv_f32, qkv_vec, x1);
    load8_f32(qkv, src + HALF, qkv_f32, qkv_vec, x2);
    if (h >= hq + hkv) {   // v: stored as it is (rounded to bf16), V layout [d][slot]
      uint16_t* pv = vc + (static_cast<int64_t>(phys) * hkv + (h - hq - hkv)) * ps * HD;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pv[static_cast<int64_t>(8 * g + e) * ps + slot] = f32_to_bf16(x1[e]);
        pv[static_cast<int64_t>(HALF + 8 * g + e) * ps + slot] = f32_to_bf16(x2[e]);
      }
      continue;
    }
    float y1[8], y2[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) rope_rotate(x1[e], x2[e], cs[0][8 * g + e], cs[1][8 * g + e], y1[e], y2[e]);
    if (h < hq) {   // q: bf16, or fp32 (the FP32-activation variant)
      const int64_t o = (static_cast<int64_t>(t) * hq + h) * HD + 8 * g;
      store8_f32(q, o, q_f32, q_vec, y1);
      store8_f32(q, o + HALF, q_f32, q_vec, y2);
      continue;
    }
    // k: d-groups g and g + 8 of the token's slot
    uint16_t* pk = kc + (static_cast<int64_t>(phys) * hkv + (h - hq)) * ps * HD;
    u16x8 a, c;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = f32_to_bf16(y1[e]);
      c[e] = f32_to_bf16(y2[e]);
    }
    *reinterpret_cast<u16x8*>(pk + (static_cast<int64_t>(g) * ps + k_slot(slot)) * 8) = a;
    *reinterpret_cast<u16x8*>(pk + (static_cast<int64_t>(g + HALF / 8) * ps + k_slot(slot)) * 8) = c;
  }
}

// ---------------------------------------------------------------- step 2a: split-KV groups
// Work units: group g (chunks 4g .. 4g + 3, those at or before the token's position) of
// token t for kv head h, ordered by (t, g, h); the unit's 16 columns are the token's G q
// heads (the rest unused).  A persistent grid: workgroup w reduces units w, w + gridDim.x,
// ... chunk by chunk, merging each unit's chunks in registers and writing one partial per
// unit.  The token records (sequence, position, length), written by kv_write_kernel or
// derived in the prologue, and the running count of units per token sit in LDS.  Loads are software-pipelined across
// chunks: the next chunk's q and K go out once this chunk's scores are done, the page ids
// of the chunk three ahead and the next chunk's V once its values are done, so a
// workgroup keeps loads in flight while it computes.  Which workgroup reduces a unit, and
// when, changes no bit of it.
struct SplitStep {
  int u, k, nk;      // unit index, chunk offset in the unit, chunks in the unit
  int t, g, c, kvh, pos;
  Seq sq;
};

// First chunk of unit `u` (a 32-bit index: the host bounds the count); `t0` is a token at
// or before the unit's token: a workgroup's units advance, so a short search finds it.
__device__ __forceinline__ SplitStep split_unit(int u, int t0, const int4* s_tok, const int* s_start,
                                                int num_tokens, const uint16_t* kc, const uint16_t* vc,
                                                const int32_t* bt, int max_pages, int ps, int hkv, int uc) {
  SplitStep it;
  const unsigned j = static_cast<unsigned>(u) / static_cast<unsigned>(hkv);
  if (t0 < 0 || t0 >= num_tokens || s_start[t0] > static_cast<int>(j)) t0 = 0;   // hint past the unit
  int t = t0;
  if (s_start[t0 + 1] <= static_cast<int>(j)) {   // past t0: binary search above it
    int lo = t0 + 1, hi = num_tokens - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_start[mid] <= static_cast<int>(j)) lo = mid;
      else hi = mid - 1;
    }
    t = lo;
  }
  // the unit is the same for the whole workgroup: keep its fields in scalar registers
  const int4 r = s_tok[t];
  it.u = u;
  it.k = 0;
  it.kvh = __builtin_amdgcn_readfirstlane(u - static_cast<int>(j) * hkv);
  it.t = __builtin_amdgcn_readfirstlane(t);
  it.g = __builtin_amdgcn_readfirstlane(static_cast<int>(j) - s_start[t]);
  it.pos = __builtin_amdgcn_readfirstlane(r.y);
  it.c = uc * it.g;
  it.nk = min(uc, it.pos / CHUNK - it.c + 1);
  const int b = __builtin_amdgcn_readfirstlane(r.x);
  const int len = __builtin_amdgcn_readfirstlane(r.z);
  it.sq = Seq{kc, vc, bt + static_cast<int64_t>(b) * max_pages, ps, hkv, it.kvh, len, max_pages,
              __builtin_ctz(ps)};
  return it;
}

// Q operands of one column, loaded unconditionally (an unused column loads the group's
// first head; its scores are masked and its output is never stored).
template <int NQ>
__device__ __forceinline__ void load_q_col(const void* q, int64_t token, int head, int hq,
                                           u16x8 (&qop)[NQ][4]) {
  load_q_at<NQ>(q, token, head, hq, qop);
}

// tok NULL (the keys and values were written by rope_kv_write_kernel, which writes no
// records): each workgroup derives the records itself from the batch description, exactly
// as kv_write_kernel does (sequence = the last b with qsl[b] <= t, searched in LDS when the
// offsets fit there).
template <int NQ>
__global__ __launch_bounds__(256) void attn_split_kernel(
    const void* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ bt, const int4* __restrict__ tok,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ qsl, int batch,
    int num_tokens, int max_pages, int hq, int hkv, int ps, int max_groups, float sl2,
    float* __restrict__ ws_ml, float* __restrict__ ws_o, int uc) {
  __shared__ ChunkLDS sh;
  __shared__ int4 s_tok[SPLIT_MAX_TOKENS];
  __shared__ int s_start[SPLIT_MAX_TOKENS + 1];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (tok) {
    for (int t = threadIdx.x; t < num_tokens; t += 256) s_tok[t] = tok[t];
  } else {
    const bool staged = batch <= SPLIT_MAX_TOKENS;   // s_start holds the offsets meanwhile
    if (staged)
      for (int i = threadIdx.x; i <= batch; i += 256) s_start[i] = qsl[i];
    __syncthreads();
    for (int t = threadIdx.x; t < num_tokens; t += 256) {
      int lo = 0, hi = batch - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((staged ? s_start[mid] : qsl[mid]) <= t) lo = mid;
        else hi = mid - 1;
      }
      const int q0 = staged ? s_start[lo] : qsl[lo], q1 = staged ? s_start[lo + 1] : qsl[lo + 1];
      const int len = seq_lens[lo];
      s_tok[t] = make_int4(lo, len - (q1 - q0) + (t - q0), len, 0);
    }
  }
  __syncthreads();
  if (w == 0) {   // s_start[t] = groups of tokens 0 .. t-1 (token t has pos / 1024 + 1)
    int carry = 0;
    for (int base = 0; base < num_tokens; base += 64) {
      const int t = base + lane;
      const int pos = t < num_tokens ? s_tok[t].y : -1;
      int v = pos >= 0 ? pos / (CHUNK * uc) + 1 : 0;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(v, o, 64);
        if (lane >= o) v += u;
      }
      if (t < num_tokens) s_start[t + 1] = carry + v;
      carry += __shfl(v, 63, 64);
    }
    if (lane == 0) s_start[0] = 0;
  }
  __syncthreads();
  const int n_units = s_start[num_tokens] * hkv;
  if (static_cast<int>(blockIdx.x) >= n_units) return;
  const int stride = gridDim.x;
  const int G = hq / hkv;
  const int col = lane & 15;
  const bool used = col < G;
  const int hcol = used ? col : 0;
  // the chunk after `p` in this workgroup's sequence (p itself after the last one: those
  // reloads are never used); the token hint only moves forward
  auto advance = [&](const SplitStep& p) {
    if (p.k + 1 < p.nk) {
      SplitStep n = p;
      n.k = p.k + 1;
      n.c = p.c + 1;
      return n;
    }
    if (p.u + stride < n_units)
      return split_unit(p.u + stride, p.t, s_tok, s_start, num_tokens, kc, vc, bt, max_pages, ps, hkv, uc);
    return p;
  };

  SplitStep cur = split_unit(blockIdx.x, 0, s_tok, s_start, num_tokens, kc, vc, bt, max_pages, ps, hkv, uc);
  int pg = chunk_pages(cur.sq, cur.c);
  u16x8 qop[NQ][4], kop[2][2][4], vop[2][8];
  load_q_col<NQ>(q, cur.t, cur.kvh * G + hcol, hq, qop);
  chunk_load_k(cur.sq, pg, kop);
  SplitStep nxt = advance(cur);
  int pgn = chunk_pages(nxt.sq, nxt.c);
  SplitStep nxt2 = advance(nxt);
  int pgn2 = chunk_pages(nxt2.sq, nxt2.c);
  chunk_load_v(cur.sq, pg, vop);
  issue_fence();
  float mu = 0.f, lu = 0.f;   // the unit's running merge (column lane % 16)
  floatx4 ou[2];
  for (;;) {
    const bool last = cur.k + 1 == cur.nk && cur.u + stride >= n_units;
    const SplitStep nxt3 = advance(nxt2);
    floatx4 s[2][2];
    float m, lsum;
    chunk_scores<NQ>(cur.c, kop, qop, used ? cur.pos : -1, sl2, sh, s, m, lsum);
    load_q_col<NQ>(q, nxt.t, nxt.kvh * G + hcol, hq, qop);
    chunk_load_k(nxt.sq, pgn, kop);
    issue_fence();
    float m_c, l_c;
    floatx4 oc[2];
    chunk_values(cur.sq, cur.c, vop, s, m, lsum, sh, m_c, l_c, oc);
    const int pgn3 = chunk_pages(nxt3.sq, nxt3.c);   // page ids three chunks ahead
    chunk_load_v(nxt.sq, pgn, vop);
    issue_fence();
    if (cur.k == 0) {
      mu = m_c;
      lu = l_c;
      ou[0] = oc[0];
      ou[1] = oc[1];
    } else {
      float a, bb;
      merge_step(mu, lu, m_c, l_c, a, bb);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) ou[j][r] = mix(ou[j][r], oc[j][r], a, bb);
    }
    if (cur.k + 1 == cur.nk && used) {
      const int64_t slot = (static_cast<int64_t>(cur.t) * hq + cur.kvh * G + col) * max_groups + cur.g;
      float* po = ws_o + slot * HD + 4 * (lane >> 4);
#pragma unroll
      for (int j = 0; j < 2; ++j) *reinterpret_cast<floatx4*>(po + 16 * (2 * w + j)) = ou[j];
      if (w == 0 && (lane >> 4) == 0) {
        ws_ml[2 * slot] = mu;
        ws_ml[2 * slot + 1] = lu;
      }
    }
    if (last) break;
    cur = nxt;
    nxt = nxt2;
    pgn = pgn2;
    nxt2 = nxt3;
    pgn2 = pgn3;
  }
}

// ---------------------------------------------------------------- step 3a: merge chunks
// one wave per (token, q head); lane holds d = 2 lane, 2 lane + 1.  Each partial covers
// `group` chunks; with fold = 1 the partials are merged in order, with fold = GROUP (single
// chunks as partials) in the two levels of the split path: the chunks of each group of
// GROUP, then the groups -- the same operations in the same order as the in-register merge
// of a group, so both give the same bits.
__global__ __launch_bounds__(256) void attn_combine_kernel(
    const float* __restrict__ ws_ml, const float* __restrict__ ws_o,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ qsl, int batch, int hq,
    int max_chunks, int64_t n_rows, void* __restrict__ out, int out_f32, int group, int fold) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= n_rows) return;
  const int t = static_cast<int>(row / hq);
  const int lane = threadIdx.x & 63;
  const int b = find_seq_wave(qsl, batch, t);
  const int pos = seq_lens[b] - (qsl[b + 1] - qsl[b]) + (t - qsl[b]);
  const int nc = (pos / CHUNK) / group + 1;   // partials to merge (chunks, or groups of them)
  const float* ml = ws_ml + row * max_chunks * 2;
  const float* po = ws_o + row * max_chunks * HD + 2 * lane;
  float m = 0.f, l = 0.f, o0 = 0.f, o1 = 0.f;
  float mg = 0.f, lg = 0.f, g0 = 0.f, g1 = 0.f;   // the current group of `fold` partials
  // chunks in groups of 64: lane c holds (m_c, l_c) of chunk base + c; 8 o loads in flight
  for (int base = 0; base < nc; base += 64) {
    const int cl = base + lane;
    const float mc_l = cl < nc ? ml[2 * cl] : 0.f;
    const float lc_l = cl < nc ? ml[2 * cl + 1] : 0.f;
    const int n = min(64, nc - base);
    for (int j0 = 0; j0 < n; j0 += 8) {
      float2 ov[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j0 + j < n) ov[j] = *reinterpret_cast<const float2*>(po + static_cast<int64_t>(base + j0 + j) * HD);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j0 + j >= n) break;
        const int c = base + j0 + j;
        const float mc = __shfl(mc_l, j0 + j, 64);
        const float lc = __shfl(lc_l, j0 + j, 64);
        if (c % fold == 0) {
          mg = mc; lg = lc; g0 = ov[j].x; g1 = ov[j].y;
        } else {
          float a, bb;
          merge_step(mg, lg, mc, lc, a, bb);
          g0 = mix(g0, ov[j].x, a, bb);
          g1 = mix(g1, ov[j].y, a, bb);
        }
        if (c % fold != fold - 1 && c != nc - 1) continue;   // group not complete yet
        if (c < fold) {
          m = mg; l = lg; o0 = g0; o1 = g1;
        } else {
          float a, bb;
          merge_step(m, l, mg, lg, a, bb);
          o0 = mix(o0, g0, a, bb);
          o1 = mix(o1, g1, a, bb);
        }
      }
    }
  }
  const float r0 = o0 / l, r1 = o1 / l;
  if (out_f32) {
    float* p = static_cast<float*>(out) + row * HD + 2 * lane;
    p[0] = r0;
    p[1] = r1;
  } else {
    uint16_t* p = static_cast<uint16_t*>(out) + row * HD + 2 * lane;
    p[0] = f32_to_bf16(r0);
    p[1] = f32_to_bf16(r1);
  }
}

// ---------------------------------------------------------------- comparison variant
// NOT batch-invariant: one workgroup per (token, group of `group` consecutive chunks, kv
// head) walks its chunks and merges them in registers, then the groups are merged.  The
// group size is chosen from the whole batch's work, so the association of the merges of
// a token -- and its bits -- change with the batch.
template <int NQ>
__global__ __launch_bounds__(256) void attn_group_kernel(
    const void* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ bt,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ qsl, int batch,
    int max_pages, int hq, int hkv, int ps, int max_groups, int group, float sl2,
    float* __restrict__ ws_ml, float* __restrict__ ws_o) {
  __shared__ ChunkLDS sh;
  const int t = blockIdx.x / max_groups;
  const int gi = blockIdx.x % max_groups;
  const int kvh = blockIdx.y;
  const int b = find_seq_wave(qsl, batch, t);
  const int L = seq_lens[b];
  const int pos = L - (qsl[b + 1] - qsl[b]) + (t - qsl[b]);
  const int c_first = gi * group;
  if (c_first * CHUNK > pos) return;
  const int c_last = min(pos / CHUNK, c_first + group - 1);
  const int G = hq / hkv;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int col = lane & 15;
  const bool used = col < G;
  u16x8 qop[NQ][4];
  load_q<NQ>(q, t, kvh * G + col, hq, used, qop);
  Seq sq{kc, vc, bt + static_cast<int64_t>(b) * max_pages, ps, hkv, kvh, L, max_pages, __builtin_ctz(ps)};
  float m = 0.f, l = 0.f;
  floatx4 o[2];
  for (int c = c_first; c <= c_last; ++c) {
    float m_c, l_c;
    floatx4 oc[2];
    chunk_partial<NQ>(sq, c, qop, used ? pos : -1, sl2, sh, m_c, l_c, oc);
    if (c == c_first) {
      m = m_c; l = l_c; o[0] = oc[0]; o[1] = oc[1];
    } else {
      float a, bb;
      merge_step(m, l, m_c, l_c, a, bb);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[j][r] = mix(o[j][r], oc[j][r], a, bb);
    }
  }
  if (!used) return;
  const int64_t slot = (static_cast<int64_t>(t) * hq + kvh * G + col) * max_groups + gi;
  float* po = ws_o + slot * HD + 4 * (lane >> 4);
#pragma unroll
  for (int j = 0; j < 2; ++j) *reinterpret_cast<floatx4*>(po + 16 * (2 * w + j)) = o[j];
  if (w == 0 && (lane >> 4) == 0) {
    ws_ml[2 * slot] = m;
    ws_ml[2 * slot + 1] = l;
  }
}

// ---------------------------------------------------------------- step 2b: prefill walk
// One workgroup per WALK_NG blocks of 16 / G consecutive tokens (aligned to the global token
// index) and kv head: WALK_NG groups of 16 columns.  It walks chunks 0.. in order; each
// chunk's K and V operands are loaded once and serve every group (chunk_scores and
// chunk_values per group, the V masking depending on the sequence only), and each group
// merges its chunks in registers (wave w keeps d-blocks 2w, 2w + 1).  A block that straddles
// two sequences is processed once per sequence with the other sequence's columns off.  Every
// workgroup re-reads its sequence's K/V prefix from L2, so the more tokens a workgroup holds
// the less of that traffic: four groups, whose q operands (the same in every wave) sit in
// LDS so that the per-group state fits the registers.
constexpr int WALK_NG = 4;

template <int NQ>
__global__ __launch_bounds__(256) void attn_walk_kernel(
    const void* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ bt,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ qsl, int batch,
    int max_pages, int hq, int hkv, int ps, int64_t num_tokens, float sl2, void* __restrict__ out,
    int out_f32) {
  __shared__ ChunkLDS sh;
  // the groups' q operands (lane l's of group gi, term j, d-step t at [gi][j][t][l]): the
  // same in every wave, so they sit here rather than in each wave's registers
  __shared__ u16x8 sqop[WALK_NG][NQ][4][64];
  const int G = hq / hkv;
  const int NT = 16 / G;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int col = lane & 15;
  const int kvh = blockIdx.y;
  const int64_t tok0 = static_cast<int64_t>(blockIdx.x) * NT * WALK_NG;
  if (tok0 >= num_tokens) return;
  const int head = kvh * G + col % G;
  int64_t my_tok[WALK_NG];
  int my_b[WALK_NG], my_pos[WALK_NG];
#pragma unroll
  for (int gi = 0; gi < WALK_NG; ++gi) {
    my_tok[gi] = tok0 + gi * NT + col / G;
    const bool tok_ok = my_tok[gi] < num_tokens;
    my_b[gi] = tok_ok ? find_seq(qsl, batch, static_cast<int>(my_tok[gi])) : -1;
    my_pos[gi] = tok_ok ? seq_lens[my_b[gi]] - (qsl[my_b[gi] + 1] - qsl[my_b[gi]]) +
                              (static_cast<int>(my_tok[gi]) - qsl[my_b[gi]])
                        : -1;
  }
  int b = find_seq(qsl, batch, static_cast<int>(tok0));
  const int64_t tok_last = (tok0 + NT * WALK_NG < num_tokens ? tok0 + NT * WALK_NG : num_tokens) - 1;
  const int b_last = find_seq(qsl, batch, static_cast<int>(tok_last));
  for (; b <= b_last; ++b) {
    if (qsl[b + 1] == qsl[b]) continue;
    int pcol[WALK_NG];
    int pmax = -1;
    __syncthreads();   // the previous sequence's q operands are no longer read
#pragma unroll
    for (int gi = 0; gi < WALK_NG; ++gi) {
      const bool mine = my_b[gi] == b;
      pcol[gi] = mine ? my_pos[gi] : -1;
      if (gi % 4 == w) {   // wave w stages group gi (WALK_NG is a multiple of 4 or below it)
        u16x8 qtmp[NQ][4];
        load_q<NQ>(q, mine ? my_tok[gi] : 0, head, hq, mine, qtmp);
#pragma unroll
        for (int j = 0; j < NQ; ++j)
#pragma unroll
          for (int t = 0; t < 4; ++t) sqop[gi][j][t][lane] = qtmp[j][t];
      }
      pmax = max(pmax, pcol[gi]);
    }
    __syncthreads();
    const int L = seq_lens[b];
    Seq sq{kc, vc, bt + static_cast<int64_t>(b) * max_pages, ps, hkv, kvh, L, max_pages, __builtin_ctz(ps)};
    // highest position among this sequence's columns (the same in every wave)
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) pmax = max(pmax, __shfl_xor(pmax, off, 64));
    // two merge levels, as the split path: chunks within each group of GROUP, then groups
    float m[WALK_NG], l[WALK_NG], mg[WALK_NG], lg[WALK_NG];
    floatx4 o[WALK_NG][2], og[WALK_NG][2];
#pragma unroll
    for (int gi = 0; gi < WALK_NG; ++gi) m[gi] = l[gi] = mg[gi] = lg[gi] = 0.f;
    for (int c = 0; c * CHUNK <= pmax; ++c) {
      const int pg = chunk_pages(sq, c);
      u16x8 kop[2][2][4], vop[2][8];
      chunk_load_k(sq, pg, kop);
      chunk_load_v(sq, pg, vop);
      issue_fence();
#pragma unroll
      for (int gi = 0; gi < WALK_NG; ++gi) {
        float m_c, l_c;
        floatx4 oc[2];
        {
          u16x8 qop[NQ][4];
#pragma unroll
          for (int j = 0; j < NQ; ++j)
#pragma unroll
            for (int t = 0; t < 4; ++t) qop[j][t] = sqop[gi][j][t][lane];
          floatx4 sc[2][2];
          float mx, lsum;
          chunk_scores<NQ>(c, kop, qop, pcol[gi], sl2, sh, sc, mx, lsum);
          chunk_values(sq, c, vop, sc, mx, lsum, sh, m_c, l_c, oc);
        }
        if (c * CHUNK > pcol[gi]) continue;
        if (c % GROUP == 0) {
          mg[gi] = m_c;
          lg[gi] = l_c;
          og[gi][0] = oc[0];
          og[gi][1] = oc[1];
        } else {
          float a, bb;
          merge_step(mg[gi], lg[gi], m_c, l_c, a, bb);
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) og[gi][j][r] = mix(og[gi][j][r], oc[j][r], a, bb);
        }
        if (c % GROUP != GROUP - 1 && c != pcol[gi] / CHUNK) continue;   // group not complete yet
        if (c < GROUP) {
          m[gi] = mg[gi];
          l[gi] = lg[gi];
          o[gi][0] = og[gi][0];
          o[gi][1] = og[gi][1];
        } else {
          float a, bb;
          merge_step(m[gi], l[gi], mg[gi], lg[gi], a, bb);
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) o[gi][j][r] = mix(o[gi][j][r], og[gi][j][r], a, bb);
        }
      }
    }
#pragma unroll
    for (int gi = 0; gi < WALK_NG; ++gi) {
      if (my_b[gi] != b) continue;
      const int64_t orow = my_tok[gi] * hq + head;
      const int d0 = 4 * (lane >> 4);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = o[gi][j][r] / l[gi];
          const int64_t idx = orow * HD + 16 * (2 * w + j) + d0 + r;
          if (out_f32) static_cast<float*>(out)[idx] = v;
          else static_cast<uint16_t*>(out)[idx] = f32_to_bf16(v);
        }
    }
  }
}

// Workgroups of attn_split_kernel<NQ> resident per CU (read once).
template <int NQ>
int split_resident() {
  static std::atomic<int> cached{0};
  int v = cached.load(std::memory_order_relaxed);
  if (v > 0) return v;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, attn_split_kernel<NQ>, 256, 0) != hipSuccess || v < 1)
    v = 1;
  cached.store(v, std::memory_order_relaxed);
  return v;
}

int64_t chunks_for(int64_t max_seq_len) { return max_seq_len <= 0 ? 1 : (max_seq_len + CHUNK - 1) / CHUNK; }

// (m, l) pairs first, padded so the partial outputs start on a 16-byte boundary.
int64_t ml_floats(int64_t rows) { return (2 * rows + 3) / 4 * 4; }

}  // namespace
}  // namespace bi

using namespace bi;

extern "C" size_t bi_attention_workspace_bytes(int64_t num_tokens, int32_t num_q_heads,
                                               int32_t head_dim, int64_t max_seq_len) {
  if (num_tokens <= 0 || num_tokens > SPLIT_MAX_TOKENS || num_q_heads <= 0 || head_dim <= 0)
    return 0;
  const int64_t rows = num_tokens * num_q_heads * chunks_for(max_seq_len);
  return static_cast<size_t>(ml_floats(rows) + rows * head_dim) * sizeof(float) +
         static_cast<size_t>(num_tokens) * sizeof(int4);
}

namespace bi {
namespace {

// Validation shared by bi_attention and bi_attention_noalloc (everything but the workspace).
int attention_check(const void* q, int q_dtype, const void* k_new, const void* v_new, void* k_cache,
                    void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                    const int32_t* query_start_loc, int32_t batch, int64_t num_tokens,
                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                    int32_t max_pages_per_seq, int64_t max_seq_len, void* out, int out_dtype) {
  if ((out_dtype != BI_BF16 && out_dtype != BI_F32) || (q_dtype != BI_BF16 && q_dtype != BI_F32))
    return BI_ERR_DTYPE;
  if (batch < 0 || num_tokens < 0 || num_q_heads < 1 || num_kv_heads < 1 || head_dim < 1 ||
      page_size < 1 || max_pages_per_seq < 1 || max_seq_len < 0)
    return BI_ERR_SHAPE;
  if (head_dim != HD) return BI_ERR_UNSUPPORTED;
  if (num_q_heads % num_kv_heads) return BI_ERR_SHAPE;
  const int G = num_q_heads / num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return BI_ERR_UNSUPPORTED;
  if (page_size % 16 || CHUNK % page_size) return BI_ERR_UNSUPPORTED;
  if (max_seq_len > static_cast<int64_t>(max_pages_per_seq) * page_size || num_tokens > (1 << 30) ||
      max_seq_len > (1 << 30))
    return BI_ERR_SHAPE;
  if (num_tokens == 0 || batch == 0) return BI_OK;
  // k_new and v_new both NULL: the keys and values are in the cache already
  if (!q || (!k_new != !v_new) || !k_cache || !v_cache || !block_table || !seq_lens ||
      !query_start_loc || !out)
    return BI_ERR_NULL;
  if (!aligned16(q) || (k_new && !aligned16(k_new)) || (v_new && !aligned16(v_new)) ||
      !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return BI_ERR_ALIGN;
  // the split path indexes its work items (token, chunk, kv head) with 32-bit integers
  if (num_tokens <= SPLIT_MAX_TOKENS &&
      num_tokens * chunks_for(max_seq_len) * num_kv_heads >= (int64_t(1) << 31))
    return BI_ERR_SHAPE;
  return BI_OK;
}

// Partials per (token, q head) on the split path: one per 4-chunk group, or, when that
// leaves fewer work units than two per CU (small batches), one per chunk.
bool split_fine(int64_t num_tokens, int64_t maxc, int32_t num_kv_heads) {
  const int64_t maxg = (maxc + GROUP - 1) / GROUP;
  return num_tokens * maxg * num_kv_heads < 2 * static_cast<int64_t>(cu_count());
}

// The kernels of a validated call.  Split path: ws_ml holds the (m, l) pairs of every partial
// slot, followed (16-byte aligned) by their o vectors; ws_tok the per-token records.
template <int NQ>
void attention_launch(const void* q, const void* k_new, const void* v_new, void* k_cache,
                      void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                      const int32_t* query_start_loc, int32_t batch, int64_t num_tokens,
                      int32_t num_q_heads, int32_t num_kv_heads, int32_t page_size,
                      int32_t max_pages_per_seq, int64_t max_seq_len, float scale, void* out,
                      int out_dtype, float* ws_ml, int4* ws_tok, hipStream_t s) {
  const bool split = num_tokens <= SPLIT_MAX_TOKENS;
  const int G = num_q_heads / num_kv_heads;
  const float sl2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  const int64_t maxc = chunks_for(max_seq_len);
  // the cache write and the split path's token records (with the keys and values in the
  // cache already, nothing: the split kernel derives the records itself)
  if (k_new)
    kv_write_kernel<<<dim3(static_cast<unsigned>(num_tokens)), dim3(256), 0, s>>>(
        static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
        static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache), block_table, seq_lens,
        query_start_loc, batch, max_pages_per_seq, num_kv_heads, page_size, split ? ws_tok : nullptr);
  const int of = out_dtype == BI_F32;
  if (split) {
    // Work units of GROUP chunks, whose partial is the group's in-register merge; when that
    // leaves fewer units than two per CU (small batches), units of one chunk, whose partials
    // the combine kernel merges in the same two levels (same bits, four times the units).
    const int64_t maxg = (maxc + GROUP - 1) / GROUP;
    const bool fine = split_fine(num_tokens, maxc, num_kv_heads);
    const int uc = fine ? 1 : GROUP;
    const int64_t slots = fine ? maxc : maxg;   // partials per (token, q head)
    float* ps_o = ws_ml + ml_floats(num_tokens * num_q_heads * slots);
    // as many workgroups as can be resident at once, never more than there are units
    const int64_t units = num_tokens * slots * num_kv_heads;   // an upper bound of the work units
    const int64_t grid = std::min<int64_t>(units, static_cast<int64_t>(split_resident<NQ>()) * cu_count());
    attn_split_kernel<NQ><<<dim3(static_cast<unsigned>(grid)), dim3(256), 0, s>>>(
        q, static_cast<const uint16_t*>(k_cache),
        static_cast<const uint16_t*>(v_cache), block_table, k_new ? ws_tok : nullptr, seq_lens,
        query_start_loc, batch, static_cast<int>(num_tokens),
        max_pages_per_seq, num_q_heads, num_kv_heads, page_size, static_cast<int>(slots), sl2,
        ws_ml, ps_o, uc);
    const int64_t rows = num_tokens * num_q_heads;
    attn_combine_kernel<<<dim3(static_cast<unsigned>((rows + 3) / 4)), dim3(256), 0, s>>>(
        ws_ml, ps_o, seq_lens, query_start_loc, batch, num_q_heads, static_cast<int>(slots), rows,
        out, of, uc, fine ? GROUP : 1);
  } else {
    const int NT = 16 / G * WALK_NG;
    const int64_t blocks = (num_tokens + NT - 1) / NT;
    attn_walk_kernel<NQ><<<dim3(static_cast<unsigned>(blocks), num_kv_heads), dim3(256), 0, s>>>(
        q, static_cast<const uint16_t*>(k_cache),
        static_cast<const uint16_t*>(v_cache), block_table, seq_lens, query_start_loc, batch,
        max_pages_per_seq, num_q_heads, num_kv_heads, page_size, num_tokens, sl2, out, of);
  }
}

void attention_launch_q(int q_dtype, const void* q, const void* k_new, const void* v_new, void* k_cache,
                        void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                        const int32_t* query_start_loc, int32_t batch, int64_t num_tokens,
                        int32_t num_q_heads, int32_t num_kv_heads, int32_t page_size,
                        int32_t max_pages_per_seq, int64_t max_seq_len, float scale, void* out,
                        int out_dtype, float* ws_ml, int4* ws_tok, hipStream_t s) {
  if (q_dtype == BI_F32)
    attention_launch<3>(q, k_new, v_new, k_cache, v_cache, block_table, seq_lens, query_start_loc, batch,
                        num_tokens, num_q_heads, num_kv_heads, page_size, max_pages_per_seq, max_seq_len,
                        scale, out, out_dtype, ws_ml, ws_tok, s);
  else
    attention_launch<1>(q, k_new, v_new, k_cache, v_cache, block_table, seq_lens, query_start_loc, batch,
                        num_tokens, num_q_heads, num_kv_heads, page_size, max_pages_per_seq, max_seq_len,
                        scale, out, out_dtype, ws_ml, ws_tok, s);
}

}  // namespace
}  // namespace bi

extern "C" int bi_attention(const void* q, int q_dtype, const void* k_new, const void* v_new,
                            void* k_cache, void* v_cache, const int32_t* block_table,
                            const int32_t* seq_lens, const int32_t* query_start_loc, int32_t batch,
                            int64_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t page_size, int32_t max_pages_per_seq,
                            int64_t max_seq_len, float scale, void* out, int out_dtype,
                            void* workspace, size_t workspace_bytes, void* stream) {
  const int st = attention_check(q, q_dtype, k_new, v_new, k_cache, v_cache, block_table, seq_lens,
                                 query_start_loc, batch, num_tokens, num_q_heads, num_kv_heads,
                                 head_dim, page_size, max_pages_per_seq, max_seq_len, out, out_dtype);
  if (st != BI_OK || num_tokens == 0 || batch == 0) return st;
  const bool split = num_tokens <= SPLIT_MAX_TOKENS;
  const size_t need = bi_attention_workspace_bytes(num_tokens, num_q_heads, head_dim, max_seq_len);
  if (split && (!workspace || workspace_bytes < need)) return BI_ERR_WORKSPACE;
  // workspace: (m, l) and o for every (token, q head, chunk), then the token records
  const int64_t maxc = chunks_for(max_seq_len);
  float* ws_ml = static_cast<float*>(workspace);
  float* ws_o = ws_ml + ml_floats(num_tokens * num_q_heads * maxc);
  int4* ws_tok = split ? reinterpret_cast<int4*>(ws_o + num_tokens * num_q_heads * maxc * HD) : nullptr;
  attention_launch_q(q_dtype, q, k_new, v_new, k_cache, v_cache, block_table, seq_lens, query_start_loc, batch,
                   num_tokens, num_q_heads, num_kv_heads, page_size, max_pages_per_seq, max_seq_len,
                   scale, out, out_dtype, ws_ml, ws_tok, as_stream(stream));
  return launch_status();
}

// ---------------------------------------------------------------- no-allocation entry point
// Scratch of bi_attention_noalloc: one copy per device, held until the process ends.  Host
// code never uses this name as an address (on the host it is a stand-in symbol): the
// device address of each GPU's copy is looked up once per device with hipGetSymbolAddress
// and kept in scratch_ptr.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace bi {
namespace {

constexpr int kMaxDevices = 64;
std::atomic<uintptr_t> scratch_ptr[kMaxDevices];

// This device's copy of the scratch array (0 on failure).  The first call on a device looks
// it up with that device current; racing first calls store the same address.
uintptr_t device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  uintptr_t p = scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return 0;
  p = reinterpret_cast<uintptr_t>(ptr);
  scratch_ptr[dev].store(p, std::memory_order_release);
  return p;
}

}  // namespace
}  // namespace bi

extern "C" int bi_attention_noalloc(const void* q, int q_dtype, const void* k_new, const void* v_new,
                                    void* k_cache, void* v_cache, const int32_t* block_table,
                                    const int32_t* seq_lens, const int32_t* query_start_loc,
                                    int32_t batch, int64_t num_tokens, int32_t num_q_heads,
                                    int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                                    int32_t max_pages_per_seq, int64_t max_seq_len, float scale,
                                    void* out, int out_dtype, void* stream) {
  const int st = attention_check(q, q_dtype, k_new, v_new, k_cache, v_cache, block_table, seq_lens,
                                 query_start_loc, batch, num_tokens, num_q_heads, num_kv_heads,
                                 head_dim, page_size, max_pages_per_seq, max_seq_len, out, out_dtype);
  if (st != BI_OK || num_tokens == 0 || batch == 0) return st;
  float* ws_ml = nullptr;
  int4* ws_tok = nullptr;
  if (num_tokens <= SPLIT_MAX_TOKENS) {
    // the partials this call writes, packed: (m, l) pairs, o vectors, token records
    const int64_t maxc = chunks_for(max_seq_len);
    const int64_t slots = split_fine(num_tokens, maxc, num_kv_heads) ? maxc : (maxc + GROUP - 1) / GROUP;
    const int64_t rows = num_tokens * num_q_heads * slots;
    const int64_t floats = ml_floats(rows) + rows * HD;
    const size_t need = static_cast<size_t>(floats) * sizeof(float) +
                        static_cast<size_t>(num_tokens) * sizeof(int4);
    if (need > kScratchBytes) return BI_ERR_WORKSPACE;
    const uintptr_t base = device_scratch();
    if (!base) return BI_ERR_HIP;
    ws_ml = reinterpret_cast<float*>(base);
    ws_tok = reinterpret_cast<int4*>(ws_ml + floats);
  }
  attention_launch_q(q_dtype, q, k_new, v_new, k_cache, v_cache, block_table, seq_lens, query_start_loc, batch,
                   num_tokens, num_q_heads, num_kv_heads, page_size, max_pages_per_seq, max_seq_len,
                   scale, out, out_dtype, ws_ml, ws_tok, as_stream(stream));
  return launch_status();
}

extern "C" int bi_attention_batchdep_split(
    const void* q, int q_dtype, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
    const int32_t* block_table, const int32_t* seq_lens, const int32_t* query_start_loc,
    int32_t batch, int64_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t page_size, int32_t max_pages_per_seq, int64_t max_seq_len, int64_t total_chunks,
    float scale, void* out, int out_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if ((out_dtype != BI_BF16 && out_dtype != BI_F32) || (q_dtype != BI_BF16 && q_dtype != BI_F32))
    return BI_ERR_DTYPE;
  if (batch < 0 || num_tokens < 0 || num_q_heads < 1 || num_kv_heads < 1 || page_size < 1 ||
      max_pages_per_seq < 1 || max_seq_len < 0 || total_chunks < 0)
    return BI_ERR_SHAPE;
  if (head_dim != HD) return BI_ERR_UNSUPPORTED;
  if (num_q_heads % num_kv_heads) return BI_ERR_SHAPE;
  const int G = num_q_heads / num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return BI_ERR_UNSUPPORTED;
  if (page_size % 16 || CHUNK % page_size) return BI_ERR_UNSUPPORTED;
  if (max_seq_len > static_cast<int64_t>(max_pages_per_seq) * page_size) return BI_ERR_SHAPE;
  if (num_tokens == 0 || batch == 0) return BI_OK;
  if (num_tokens > SPLIT_MAX_TOKENS) return BI_ERR_UNSUPPORTED;
  if (!q || (!k_new != !v_new) || !k_cache || !v_cache || !block_table || !seq_lens ||
      !query_start_loc || !out)
    return BI_ERR_NULL;
  if (!aligned16(q) || (k_new && !aligned16(k_new)) || (v_new && !aligned16(v_new)) ||
      !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return BI_ERR_ALIGN;
  const size_t need = bi_attention_workspace_bytes(num_tokens, num_q_heads, head_dim, max_seq_len);
  if (!workspace || workspace_bytes < need) return BI_ERR_WORKSPACE;
  // occupancy heuristic: about four workgroups per CU over the whole batch
  const int64_t work = (total_chunks > 0 ? total_chunks : num_tokens) * num_kv_heads;
  int64_t group = (work + 1023) / 1024;
  if (group < 1) group = 1;
  const int64_t maxc = chunks_for(max_seq_len);
  if (group > maxc) group = maxc;
  const int64_t maxg = (maxc + group - 1) / group;
  hipStream_t s = as_stream(stream);
  const float sl2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  if (k_new)
    kv_write_kernel<<<dim3(static_cast<unsigned>(num_tokens)), dim3(256), 0, s>>>(
        static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
        static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache), block_table, seq_lens,
        query_start_loc, batch, max_pages_per_seq, num_kv_heads, page_size, nullptr);
  float* ws_ml = static_cast<float*>(workspace);
  float* ws_o = ws_ml + ml_floats(num_tokens * num_q_heads * maxg);
  const dim3 ggrid(static_cast<unsigned>(num_tokens * maxg), num_kv_heads);
  if (q_dtype == BI_F32)
    attn_group_kernel<3><<<ggrid, dim3(256), 0, s>>>(
        q, static_cast<const uint16_t*>(k_cache), static_cast<const uint16_t*>(v_cache), block_table,
        seq_lens, query_start_loc, batch, max_pages_per_seq, num_q_heads, num_kv_heads, page_size,
        static_cast<int>(maxg), static_cast<int>(group), sl2, ws_ml, ws_o);
  else
    attn_group_kernel<1><<<ggrid, dim3(256), 0, s>>>(
        q, static_cast<const uint16_t*>(k_cache), static_cast<const uint16_t*>(v_cache), block_table,
        seq_lens, query_start_loc, batch, max_pages_per_seq, num_q_heads, num_kv_heads, page_size,
        static_cast<int>(maxg), static_cast<int>(group), sl2, ws_ml, ws_o);
  const int64_t rows = num_tokens * num_q_heads;
  attn_combine_kernel<<<dim3(static_cast<unsigned>((rows + 3) / 4)), dim3(256), 0, s>>>(
      ws_ml, ws_o, seq_lens, query_start_loc, batch, num_q_heads, static_cast<int>(maxg), rows, out,
      out_dtype == BI_F32, static_cast<int>(group), 1);
  return launch_status();
}

extern "C" int bi_rope_kv_write(const void* qkv, int64_t ldqkv, int qkv_dtype, void* q, int q_dtype,
                                void* k_cache, void* v_cache, const int32_t* block_table,
                                const int32_t* seq_lens, const int32_t* query_start_loc,
                                int32_t batch, int64_t num_tokens, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                                int32_t max_pages_per_seq, double base, void* stream) {
  if ((qkv_dtype != BI_BF16 && qkv_dtype != BI_F32) || (q_dtype != BI_BF16 && q_dtype != BI_F32))
    return BI_ERR_DTYPE;
  if (batch < 0 || num_tokens < 0 || num_q_heads < 1 || num_kv_heads < 1 || head_dim < 1 ||
      page_size < 1 || max_pages_per_seq < 1)
    return BI_ERR_SHAPE;
  if (head_dim != HD) return BI_ERR_UNSUPPORTED;
  if (page_size % 16 || CHUNK % page_size) return BI_ERR_UNSUPPORTED;
  if (ldqkv < static_cast<int64_t>(num_q_heads + 2 * num_kv_heads) * HD || num_tokens > (1 << 30))
    return BI_ERR_SHAPE;
  if (num_tokens == 0 || batch == 0) return BI_OK;
  if (!qkv || !q || !k_cache || !v_cache || !block_table || !seq_lens || !query_start_loc)
    return BI_ERR_NULL;
  if (!aligned16(k_cache) || !aligned16(v_cache)) return BI_ERR_ALIGN;
  const int qkv_vec = aligned16(qkv) && (ldqkv % (qkv_dtype == BI_F32 ? 4 : 8)) == 0;
  const int q_vec = aligned16(q);
  rope_kv_write_kernel<<<dim3(static_cast<unsigned>(num_tokens)), dim3(256), 0, as_stream(stream)>>>(
      qkv, ldqkv, qkv_dtype == BI_F32, qkv_vec, q, q_dtype == BI_F32, q_vec,
      static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache), block_table, seq_lens,
      query_start_loc, batch, max_pages_per_seq, num_q_heads, num_kv_heads, page_size, base);
  return launch_status();
}
