// bi_gemm: batch-invariant bf16 GEMM on the gfx950 matrix cores.
//
// "Defeating nondeterminism in LLM inference", section on batch-invariant matrix
// multiplication: parallelise over output tiles so every dot product stays inside one
// workgroup; do not split K (split-K changes the order with the batch) and do not use
// stream-K (it even loses batch-position invariance); use one kernel configuration, so
// that no shape switches to another reduction order.  Here the configuration that fixes
// the order is:
//   one instruction, v_mfma_f32_16x16x32_bf16; fp32 accumulators starting at +0; K walked
//   in ascending 32-wide steps from 0 to K, lane l of the instruction holding row (or
//   column) l % 16 and k offsets 8 (l / 16) .. + 7 of each step.  Products past K are exact
//   zeros; rows past M (columns past N) are never stored.
// Output element (i, j) is therefore the result of the same instruction sequence for
// every M, every position of row i inside its tile and every workgroup configuration; the
// configuration only decides which wave computes which outputs, and the tests check the
// bits across every switch.  Configurations, picked from the output grid:
//   256 x 256 (8 waves of 128 x 64) or 128 x 128 (4 waves of 64 x 64, two workgroups per CU;
//   8 waves of 64 x 32 when the grid has no more tiles than CUs), or for grids well under one
//   such tile per CU 64 x 128 / 64 x 64 (waves of 32 x 32): 64-wide K slices of both
//   tiles stream into an LDS ring by direct-to-LDS 16-byte loads; the 16-byte k-chunks of
//   row r sit at chunk position c ^ swz(r) so that the operand reads of consecutive rows hit
//   distinct banks; bf16 results leave through LDS as 16-byte row pieces.
//   Up to 64 rows: one wave per 16 (or 32) output columns and all rows loads its operands
//   straight into registers.
// The fp32-A path, B given as [K, N] (the torch.mm orientation; each 4 x 8 block of it is
// transposed on its way into LDS), operands of 4 GiB or more and the split-K comparison
// variant stage through registers instead (128 x 128 tile); they share the instruction, the
// lane-to-k assignment and the K order, so a [K, N] B gives the bits of its [N, K] copy.
//
// A may be fp32 ("FP32 upcast" of the cross-vendor mismatch abstract): each value is
// split exactly into bf16 hi + mid + lo (truncations, so hi + mid + lo == a for normal
// numbers) and the three products are accumulated into the same fp32 accumulator in
// the order hi, mid, lo for every 32-wide K step.
#include "contract_fp.h"   // (includes bi_common.h) rms_scale of the fused RMSNorm

namespace bi {
namespace {

constexpr int BM = 128, BN = 128, BK = 64;
// Output modes of the kernels' c_f32 argument: bf16 C, fp32 C, or SwiGLU of column pairs
// (bf16, half the columns; only the LDS-staged and few-row kernels implement it).
constexpr int kOutBF16 = 0, kOutF32 = 1, kOutSwiGLU = 2;
constexpr int kThreads = 256;
constexpr int LDS_LD = BK + 8;  // bf16 per LDS row: 144 bytes keeps 16-byte reads conflict-free

__device__ __forceinline__ bf16x8 as_bf16x8(u16x8 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint16_t bf16_trunc(float f) {
  return static_cast<uint16_t>(__float_as_uint(f) >> 16);
}

// Global -> register staging of one K step.  A tile: 128 rows x 64 k; each thread owns
// rows (tid / 8) + 32 i and the 8-wide k vector tid % 8.
template <bool AF32>
struct Stage {
  u16x8 a[AF32 ? 3 : 1][4];
  u16x8 b[4];
};

__device__ __forceinline__ u16x8 load_bf16x8(const uint16_t* p, int64_t k, int64_t K, bool row_ok) {
  u16x8 r = {0, 0, 0, 0, 0, 0, 0, 0};
  if (!row_ok) return r;
  if (k + 8 <= K) return *reinterpret_cast<const u16x8*>(p + k);
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (k + e < K) r[e] = p[k + e];
  return r;
}

__device__ __forceinline__ void split3(const float* p, int64_t k, int64_t K, bool row_ok,
                                       u16x8& hi, u16x8& mid, u16x8& lo) {
  float v[8];
  if (row_ok && k + 8 <= K) {
    floatx4 q0 = *reinterpret_cast<const floatx4*>(p + k);
    floatx4 q1 = *reinterpret_cast<const floatx4*>(p + k + 4);
    v[0] = q0[0]; v[1] = q0[1]; v[2] = q0[2]; v[3] = q0[3];
    v[4] = q1[0]; v[5] = q1[1]; v[6] = q1[2]; v[7] = q1[3];
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (row_ok && k + e < K) ? p[k + e] : 0.f;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    uint16_t h, m, l;
    split_bf16x3(v[e], h, m, l);
    hi[e] = h;
    mid[e] = m;
    lo[e] = l;
  }
}

// B given as [K, N] (torch.mm orientation): 8 consecutive columns of one k row, columns at
// or past N and rows at or past ke read as zeros (nothing past the matrix is touched).
__device__ __forceinline__ u16x8 load_kn_bf16x8(const uint16_t* B, int64_t ldb, int k, int n, int ke,
                                                int N) {
  u16x8 r = {0, 0, 0, 0, 0, 0, 0, 0};
  if (k >= ke || n >= N) return r;
  const uint16_t* p = B + static_cast<int64_t>(k) * ldb + n;
  if (n + 8 <= N) return *reinterpret_cast<const u16x8*>(p);
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (n + e < N) r[e] = p[e];
  return r;
}

// Register-staged kernel.  BKN: B is [K, N]; each thread loads a 4 (k) x 8 (n) block of it
// and writes the block transposed into the same [n][k] LDS layout the [N, K] operand fills,
// so the operand reads, instructions and K order -- and every output bit -- are those of
// the [N, K] layout.
template <bool AF32, bool BKN = false>
__global__ __launch_bounds__(kThreads) void gemm_kernel(
    const void* __restrict__ Ap, const uint16_t* __restrict__ B, void* __restrict__ C, int M,
    int N, int K, int64_t lda, int64_t ldb, int64_t ldc, int c_f32, int tiles_m, int tiles_n,
    int k_begin, int k_end, int64_t split_stride) {
  constexpr int NA = AF32 ? 3 : 1;
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][NA][BM * LDS_LD];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][BN * LDS_LD];

  // Tile order: consecutive workgroup ids land on different XCDs (round robin over 8),
  // so regroup them to give each XCD a contiguous band of tiles, then walk tiles
  // column-major inside bands of 8 tile-rows to share A rows and B columns in L2.
  const int nwg = tiles_m * tiles_n;
  int id = blockIdx.x;
  if ((nwg & 7) == 0) id = (id & 7) * (nwg >> 3) + (id >> 3);
  const int group = 8;
  const int per_group = group * tiles_n;
  const int g = id / per_group;
  const int first_m = g * group;
  const int gm = min(tiles_m - first_m, group);
  const int tm = first_m + (id % per_group) % gm;
  const int tn = (id % per_group) / gm;

  C = static_cast<char*>(C) + static_cast<int64_t>(blockIdx.y) * split_stride;
  const int kb = k_begin + static_cast<int>(blockIdx.y) * (k_end - k_begin);
  const int ke = min(K, kb + (k_end - k_begin));

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // staging coordinates
  const int st_row = tid >> 3;      // 0..31, +32 i
  const int st_k = (tid & 7) * 8;   // 0..56
  const uint16_t* Ab = static_cast<const uint16_t*>(Ap);
  const float* Af = static_cast<const float*>(Ap);
  bool a_ok[4], b_ok[4];
  int64_t a_off[4], b_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ra = tm * BM + st_row + 32 * i;
    const int rb = tn * BN + st_row + 32 * i;
    a_ok[i] = ra < M;
    b_ok[i] = rb < N;
    a_off[i] = static_cast<int64_t>(a_ok[i] ? ra : 0) * lda;
    b_off[i] = static_cast<int64_t>(b_ok[i] ? rb : 0) * ldb;
  }

  // [K, N] staging: thread tid owns columns 8 (tid / 16) .. + 7 and k rows 4 (tid % 16) .. + 3
  // of the 128 x 64 B stage, so the 16 threads that share a column chunk write 16 adjacent
  // 8-byte pieces of each transposed LDS row (no bank conflicts among them)
  const int kn_n = tn * BN + (tid >> 4) * 8, kn_k = (tid & 15) * 4;
  auto load_stage = [&](Stage<AF32>& s, int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (AF32) split3(Af + a_off[i], k0 + st_k, ke, a_ok[i], s.a[0][i], s.a[NA > 1 ? 1 : 0][i], s.a[NA - 1][i]);
      else s.a[0][i] = load_bf16x8(Ab + a_off[i], k0 + st_k, ke, a_ok[i]);
      if (BKN) s.b[i] = load_kn_bf16x8(B, ldb, k0 + kn_k + i, kn_n, ke, N);
      else s.b[i] = load_bf16x8(B + b_off[i], k0 + st_k, ke, b_ok[i]);
    }
  };
  auto store_stage = [&](const Stage<AF32>& s, int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int o = (st_row + 32 * i) * LDS_LD + st_k;
#pragma unroll
      for (int t = 0; t < NA; ++t) *reinterpret_cast<u16x8*>(&sA[buf][t][o]) = s.a[t][i];
      if (!BKN) *reinterpret_cast<u16x8*>(&sB[buf][o]) = s.b[i];
    }
    if (BKN) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const u16x4 col = {s.b[0][e], s.b[1][e], s.b[2][e], s.b[3][e]};
        *reinterpret_cast<u16x4*>(&sB[buf][((tid >> 4) * 8 + e) * LDS_LD + kn_k]) = col;
      }
    }
  };

  floatx4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.f;

  const int nk = ke > kb ? (ke - kb + BK - 1) / BK : 0;
  Stage<AF32> st;
  if (nk > 0) {
    load_stage(st, kb);
    store_stage(st, 0);
  }
  __syncthreads();

  // operand read coordinates: lane holds row (lane % 16) of each 16-row block and k
  // (lane / 16) * 8 .. +7 of each 32-wide step
  const int orow = lane & 15;
  const int okk = (lane >> 4) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_stage(st, kb + (kt + 1) * BK);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      bf16x8 bv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bv[j] = as_bf16x8(*reinterpret_cast<const u16x8*>(
            &sB[cur][(wn * 64 + j * 16 + orow) * LDS_LD + kk + okk]));
#pragma unroll
      for (int t = 0; t < NA; ++t) {
        bf16x8 av[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          av[i] = as_bf16x8(*reinterpret_cast<const u16x8*>(
              &sA[cur][t][(wm * 64 + i * 16 + orow) * LDS_LD + kk + okk]));
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
      }
    }
    if (kt + 1 < nk) store_stage(st, cur ^ 1);
    __syncthreads();
  }

  // epilogue: register r of block (i, j) is row 4 (lane / 16) + r, column lane % 16 of it
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = tn * BN + wn * 64 + j * 16 + (lane & 15);
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = tm * BM + wm * 64 + i * 16 + 4 * (lane >> 4) + r;
        if (row >= M) continue;
        if (c_f32)
          static_cast<float*>(C)[static_cast<int64_t>(row) * ldc + col] = acc[i][j][r];
        else
          static_cast<uint16_t*>(C)[static_cast<int64_t>(row) * ldc + col] = f32_to_bf16(acc[i][j][r]);
      }
    }
}

constexpr int DBK = 64;                  // K depth of one LDS stage in the main kernel
constexpr int KS = DBK / 32;             // 32-wide K steps per stage (two: see advance)
constexpr int CPR = DBK / 8;             // 16-byte chunks per LDS row
constexpr int RPI = 64 / CPR;            // tile rows filled by one 1 KB wave-wide load
constexpr uint32_t kBlkBytes = 16 * DBK * 2;   // LDS bytes of one 16-row block of a stage

// Workgroup tile: WAVES_M x WAVES_N waves, each wave BLK_M x BLK_N blocks of the one
// 16 x 16 x 32 matrix instruction.  Every configuration computes each output element with
// the same instruction sequence (one fp32 chain from +0 over ascending 32-wide K steps,
// lane l holding k = 8 (l / 16) .. + 7 of each step), so they give identical bits; the tile
// only decides which workgroup computes which outputs.
template <int WAVES_M_, int WAVES_N_, int BLK_M_, int BLK_N_, int STAGES_, int WAVES_PER_SIMD_ = 2,
          int DMA_WAVES_ = WAVES_M_ * WAVES_N_>
struct Tile {
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, BLK_M = BLK_M_, BLK_N = BLK_N_;
  static constexpr int STAGES = STAGES_;   // LDS ring depth
  static constexpr int WAVES_PER_SIMD = WAVES_PER_SIMD_;   // register budget: 512 / this
  static constexpr int NW = WAVES_M * WAVES_N;
  // waves 0 .. DW - 1 issue the operand loads of a stage; the others only read LDS and
  // multiply, so a wave held up issuing loads leaves its SIMD to one that is not
  static constexpr int DW = DMA_WAVES_;
  static constexpr int THREADS = NW * 64;
  static constexpr int TM = WAVES_M * BLK_M * 16;
  static constexpr int TN = WAVES_N * BLK_N * 16;
  static constexpr int NJA = TM / DW / RPI;  // A loads per issuing wave per stage
  static constexpr int NJB = TN / DW / RPI;  // B loads per issuing wave per stage
  static constexpr int PER = NJA + NJB;
  static constexpr int SA = TM * DBK, SB = TN * DBK;  // bf16 elements per stage
  // operands of the next K step read in place (see advance) rather than into a second set
  static constexpr bool INPLACE = BLK_M * BLK_N >= 32;
  static constexpr bool OTF = INPLACE;   // load offsets computed per load (see DmaCtx)
  static constexpr bool BKN = false;     // B as [N, K]
  static_assert(TM % (DW * RPI) == 0 && TN % (DW * RPI) == 0 && DW <= NW, "tile rows per wave");
  static_assert(STAGES >= 2, "unsupported staging");
};
// 128 x 128 as 8 waves of 64 x 32: with a 2-stage ring (64 KB, two workgroups and four waves
// per SIMD per CU), or for grids with no more tiles than CUs with a 3-stage ring (96 KB,
// one workgroup); 256 x 256, 8 waves of 128 x 64, 2-stage ring (128 KB, one per CU).  With
// 8 waves, one wave per SIMD issues the stage loads.
using Tile128 = Tile<2, 4, 4, 2, 2, 4, 4>;
using Tile128Deep = Tile<2, 4, 4, 2, 3, 2, 4>;
// Grids with well under one 128 x 128 tile per CU (a few hundred rows): 64 x 128 as 8 waves
// of 32 x 32, or 64 x 64 as 4 waves of 32 x 32, both with a 3-stage ring.
using Tile64x128 = Tile<2, 4, 2, 2, 3, 2, 4>;
using Tile64 = Tile<2, 2, 2, 2, 3>;
using Tile256 = Tile<2, 4, 8, 4, 2, 2, 4>;

// The same tile reading B as [K, N] (torch.mm orientation).  A B stage then holds DBK k rows
// of TN columns: a wave-wide 1 KB load fills RPK whole k rows, lane l taking 16-byte chunk
// position l % CPRN of its row.  Chunk c of k row r sits at position c ^ swzk(r), so that
// the transposing operand reads below (4 k rows x 32 bytes per group of 16 lanes, two groups
// per half-wave 8 rows apart) fall on distinct banks.  The operand values, and so the
// instruction sequence and every output bit, are those of the [N, K] tile.
template <class T>
struct KnTile : T {
  static constexpr bool BKN = true;
  static constexpr int CPRN = T::TN / 8;   // 16-byte chunks per k row
  static constexpr int RPK = 64 / CPRN;    // k rows per wave-wide load
  static_assert(!T::INPLACE && T::TN % 64 == 0 && (DBK / T::DW) == T::NJB * RPK, "[K, N] stage");
};
template <int CPRN>
__device__ __forceinline__ int swzk(int r) {
  return CPRN >= 16 ? (((r & 3) << 1) | (((r >> 3) & 1) << 3)) : ((r & 3) << 1);
}

// Chunk c of LDS row r (128 bytes) sits at position c ^ swz(r), swz(r) = (r / 2) % 8: the
// 16-byte reads of 16 consecutive rows at one chunk index (a quarter of the wave's lanes)
// then cover all 64 banks once.  The pattern repeats every 16 rows, so a lane's offsets in
// the 16-row blocks of a wave differ by multiples of kBlkBytes.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

// 16 bytes per lane from global memory straight into LDS at m0 + 16 * lane, addressed as
// a wave-uniform 64-bit base plus a per-lane 32-bit byte offset.  Written in asm so that
// the compiler does not order every later LDS read behind it; m0 is saved and restored
// and no register is written by the load.
__device__ __forceinline__ void dma16(const void* base, uint32_t off, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_addr), "v"(off), "s"(base)
      : "memory");
}

// Loads J .. N - 1 of one operand: load j lands 1024 j bytes past lds_base (added to m0
// inside the asm, so one scalar register holds the base of the whole run).
template <int J, int N, class Off>
__device__ __forceinline__ void dma16_run(const void* base, const Off& off, uint32_t lds_base) {
  if constexpr (J < N) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_add_u32 m0, %1, %4\n\t"
        "global_load_lds_dwordx4 %2, %3\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds_base), "v"(off(J)), "s"(base), "n"(J * 1024)
        : "memory", "scc");
    dma16_run<J + 1, N>(base, off, lds_base);
  }
}

// Wait until at most N of this wave's vector-memory operations are outstanding and all
// its LDS operations are done, then meet the other waves.
template <int N>
__device__ __forceinline__ void wait_and_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Wait for the oldest stage: `ahead` later stages (0..S) may stay in flight.
template <int PER, int S>
__device__ __forceinline__ void wait_stage(int ahead) {
  if constexpr (S == 0) {
    wait_and_barrier<0>();
  } else {
    if (ahead >= S) wait_and_barrier<S * PER>();
    else wait_stage<PER, S - 1>(ahead);
  }
}

// A and B must each span less than 4 GiB (byte offsets are 32-bit); the host checks.
template <class T>
struct DmaCtx {
  const uint16_t* A;
  const uint16_t* B;
  // per-lane byte offsets of this lane's chunks, kept (small tiles) or, for the tile whose
  // registers the accumulators fill, computed per load from the row of load 0 (load j is
  // RPI j rows further, clamped to the last row) and the row pitch in bytes
  uint32_t aoff[T::OTF ? 1 : T::NJA], boff[T::OTF ? 1 : T::NJB];
  int knrow[T::BKN ? T::NJB : 1];        // [K, N] B: k row (in the stage) of load j
  int64_t ldb;                           // [K, N] B: elements per k row
  int ra_share, rb_share;   // first tile row of this wave's A and B share (wave-uniform)
  int a_last, b_last;
  uint32_t lda2, ldb2;
  int kc[2];   // k offset inside a stage of this lane's chunk in loads j even / odd (A and B)
  uint32_t lds_a, lds_b;                 // LDS byte address of this wave's rows in stage 0
  int K, nk;
  bool ktail;
  bool issuer;                           // this wave issues loads (wave < T::DW)
};

// Per-load offsets, computed per load from the lane id.  They are loop-invariant, and the
// compiler would compute them all once before the loop and keep (or spill) them, so the
// lane id comes from an asm in every stage, which it cannot hoist.
template <class T>
struct LoadOffsets {
  int ra0, rb0, kc0, kc1;   // row of load 0 (A, B); k offset of the chunk of loads j even / odd
  __device__ __forceinline__ explicit LoadOffsets(const DmaCtx<T>& d) {
    if constexpr (T::OTF) {
      int l;   // the lane id, recomputed in every stage
      asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
      ra0 = d.ra_share + l / CPR;
      rb0 = d.rb_share + l / CPR;
      kc0 = ((l % CPR) ^ swz(l / CPR)) * 8;
      kc1 = ((l % CPR) ^ swz(RPI + l / CPR)) * 8;
    } else {
      ra0 = rb0 = 0;
      kc0 = d.kc[0];
      kc1 = d.kc[1];
    }
  }
};
template <class T>
__device__ __forceinline__ uint32_t a_off(const DmaCtx<T>& d, const LoadOffsets<T>& o, int j) {
  if constexpr (T::OTF)
    return static_cast<uint32_t>(min(o.ra0 + RPI * j, d.a_last)) * d.lda2 + 2 * ((j & 1) ? o.kc1 : o.kc0);
  else
    return d.aoff[j];
}
template <class T>
__device__ __forceinline__ uint32_t b_off(const DmaCtx<T>& d, const LoadOffsets<T>& o, int j) {
  if constexpr (T::OTF)
    return static_cast<uint32_t>(min(o.rb0 + RPI * j, d.b_last)) * d.ldb2 + 2 * ((j & 1) ? o.kc1 : o.kc0);
  else
    return d.boff[j];
}

// Stage kt into ring buffer `buf` (a template constant in the steady loop, a run-time
// value in the prologue and the tail, where it only moves the LDS base).
template <class T>
__device__ __forceinline__ void dma_stage_at(const DmaCtx<T>& d, uint32_t buf, int kt) {
  constexpr uint32_t sa_bytes = T::SA * 2, sb_bytes = T::SB * 2;
  const int k0 = kt * DBK;
  const uint32_t la = d.lds_a + buf * sa_bytes, lb = d.lds_b + buf * sb_bytes;
  const LoadOffsets<T> lo(d);
  if (d.ktail && kt == d.nk - 1) {
    // last, partial step: a chunk wholly past K re-reads the first 8 elements of its row
    // (always inside the row; zeroed after landing)
#pragma unroll
    for (int j = 0; j < T::NJA; ++j) {
      const int kc = (j & 1) ? lo.kc1 : lo.kc0;
      const uint32_t adv = (k0 + kc < d.K) ? static_cast<uint32_t>(k0) * 2 : static_cast<uint32_t>(-2 * kc);
      dma16(d.A, a_off<T>(d, lo, j) + adv, la + j * 1024);
    }
    if constexpr (T::BKN) {
      // [K, N] B: a k row at or past K reads the stage's first row instead (zeroed after
      // landing)
      const uint16_t* bk = d.B + static_cast<int64_t>(k0) * d.ldb;
#pragma unroll
      for (int j = 0; j < T::NJB; ++j) {
        const uint32_t off = (k0 + d.knrow[j] < d.K) ? d.boff[j] : d.boff[j] - static_cast<uint32_t>(d.knrow[j]) * d.ldb2;
        dma16(bk, off, lb + j * 1024);
      }
    } else {
#pragma unroll
      for (int j = 0; j < T::NJB; ++j) {
        const int kc = (j & 1) ? lo.kc1 : lo.kc0;
        const uint32_t adv = (k0 + kc < d.K) ? static_cast<uint32_t>(k0) * 2 : static_cast<uint32_t>(-2 * kc);
        dma16(d.B, b_off<T>(d, lo, j) + adv, lb + j * 1024);
      }
    }
  } else {
    dma16_run<0, T::NJA>(d.A + k0, [&](int j) { return a_off<T>(d, lo, j); }, la);
    if constexpr (T::BKN)
      dma16_run<0, T::NJB>(d.B + static_cast<int64_t>(k0) * d.ldb, [&](int j) { return d.boff[j]; }, lb);
    else
      dma16_run<0, T::NJB>(d.B + k0, [&](int j) { return b_off<T>(d, lo, j); }, lb);
  }
}

// Per-lane LDS byte offsets (from the start of the ring) of the wave's first A and first B
// block in K step 0 of a stage; block i lies i kBlkBytes further.  Step 1 reads chunks 4..7
// where step 0 reads 0..3, which under the swizzle is chunk position ^ 4, byte offset ^ 64
// (computed at each use, through an empty asm, so that it takes no register of its own).
struct Frag {
  uint32_t a0, b0;
  __device__ __forceinline__ static uint32_t step(uint32_t base, int ks) {
    if (ks == 0) return base;
    asm volatile("" : "+v"(base));
    return base ^ 64u;
  }
  __device__ __forceinline__ uint32_t a(int ks) const { return step(a0, ks); }
  __device__ __forceinline__ uint32_t b(int ks) const { return step(b0, ks); }
};

// Operands of one 32-wide K step: BLK_M A fragments and BLK_N B fragments, read from ring
// buffer `buf` (a template constant in the steady loop; with the block offsets it becomes
// the reads' immediate offset).
template <class T>
struct Ops {
  bf16x8 a[T::BLK_M], b[T::BLK_N];
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// [K, N] B operand of block j for one 32-wide K step whose k row 0 starts at `rows` (LDS):
// two transposing reads, each giving lane l rows k .. k + 3 (k = 8 (l / 16) + 4 h) of column
// 16 j + l % 16 of the wave's columns; lane l addresses row k + (l % 16) / 4 at column
// 4 (l % 4) of that block, which is how the read distributes a 16-lane group's 4 x 16
// elements (checked on the GPU).
template <class T>
__device__ __forceinline__ bf16x8 kn_operand(const char* rows, int wn, int j) {
  const int l = static_cast<int>(threadIdx.x & 63);
  u16x8 r;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int row = 8 * (l >> 4) + 4 * h + ((l & 15) >> 2);
    const int col = wn * T::BLK_N * 16 + 16 * j + 4 * (l & 3);
    const int off = row * T::TN * 2 + 16 * ((col >> 3) ^ swzk<T::CPRN>(row)) + 8 * ((col >> 2) & 1);
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(rows + off));
#pragma unroll
    for (int e = 0; e < 4; ++e) r[4 * h + e] = static_cast<uint16_t>(v[e]);
  }
  return as_bf16x8(r);
}

template <class T>
__device__ __forceinline__ void load_ops(const uint16_t* sA, uint32_t buf, int ks, const Frag& f,
                                         Ops<T>& o) {
  const char* a = reinterpret_cast<const char*>(sA) + f.a(ks) + buf * (T::SA * 2);
  const char* b = reinterpret_cast<const char*>(sA) + f.b(ks) + buf * (T::SB * 2);
  // in the order the MFMAs consume them: A0, every B, then A1 .. (the first MFMAs can
  // start after 1 + BLK_N reads)
  o.a[0] = as_bf16x8(*reinterpret_cast<const u16x8*>(a));
  if constexpr (T::BKN) {
    const int wn = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6)) % T::WAVES_N;
    const char* rows = reinterpret_cast<const char*>(sA) + T::STAGES * T::SA * 2 + buf * (T::SB * 2) +
                       ks * 32 * T::TN * 2;
#pragma unroll
    for (int j = 0; j < T::BLK_N; ++j) o.b[j] = kn_operand<T>(rows, wn, j);
  } else {
#pragma unroll
    for (int j = 0; j < T::BLK_N; ++j) o.b[j] = as_bf16x8(*reinterpret_cast<const u16x8*>(b + j * kBlkBytes));
  }
#pragma unroll
  for (int i = 1; i < T::BLK_M; ++i) o.a[i] = as_bf16x8(*reinterpret_cast<const u16x8*>(a + i * kBlkBytes));
}

template <class T>
__device__ __forceinline__ void mfma_ops(const Ops<T>& o, floatx4 (&acc)[T::BLK_M][T::BLK_N]) {
#pragma unroll
  for (int i = 0; i < T::BLK_M; ++i)
#pragma unroll
    for (int j = 0; j < T::BLK_N; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o.a[i], o.b[j], acc[i][j], 0, 0, 0);
}

// Zero every element at k >= K of stage kt (in ring buffer buf) in the pieces this lane's
// own loads wrote (issuing waves only); the caller then waits and meets the other waves.
template <class T>
__device__ __forceinline__ void zero_k_tail(const DmaCtx<T>& d, uint16_t* sA, uint16_t* sB, int buf,
                                            int kt, int wave, int lane) {
  const int k0 = kt * DBK;
  const LoadOffsets<T> lo(d);
#pragma unroll
  for (int j = 0; j < T::NJA; ++j) {
    const int pos = buf * T::SA + ((T::TM / T::DW) * wave + RPI * j + lane / CPR) * DBK + (lane % CPR) * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (k0 + ((j & 1) ? lo.kc1 : lo.kc0) + e >= d.K) sA[pos + e] = 0;
  }
  if constexpr (T::BKN) {
    // [K, N] B: load j's 16 bytes are one k row's chunk; clear it when that row is at or past K
#pragma unroll
    for (int j = 0; j < T::NJB; ++j) {
      const int pos = buf * T::SB + (DBK / T::DW) * wave * T::TN + j * 512 + lane * 8;
      if (k0 + d.knrow[j] >= d.K) {
#pragma unroll
        for (int e = 0; e < 8; ++e) sB[pos + e] = 0;
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < T::NJB; ++j) {
      const int pos = buf * T::SB + ((T::TN / T::DW) * wave + RPI * j + lane / CPR) * DBK + (lane % CPR) * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (k0 + ((j & 1) ? lo.kc1 : lo.kc0) + e >= d.K) sB[pos + e] = 0;
    }
  }
}

// Scheduling hint for one K step: alternate the step's MFMAs with the next step's LDS
// operand reads (one read after each MFMA), so the LDS works while the matrix core does.
template <class T>
__device__ __forceinline__ void interleave() {
  constexpr int NR = T::BLK_M + T::BLK_N, NM = T::BLK_M * T::BLK_N;
  constexpr int NP = NR < NM ? NR : NM;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
  }
  if constexpr (NM > NP) __builtin_amdgcn_sched_group_barrier(0x008, NM - NP, 0);
  if constexpr (NR > NP) __builtin_amdgcn_sched_group_barrier(0x100, NR - NP, 0);
}

// MFMAs of one 32-wide K step while the operands of the next step (ring buffer buf, step ks
// of that stage) are read from LDS.
//  - Two operand sets (o0 holds the even steps of a stage, o1 the odd ones): the next step's
//    reads go to the other set, alternated with this step's MFMAs.
//  - A in place (wave tiles whose two full sets would not fit beside the accumulators): B
//    fragments alternate between o0 (even steps) and o1 (odd steps) as above and are read
//    during the first BLK_N MFMAs; the A fragments live in o0, and next A fragment i
//    replaces current A fragment i right after the BLK_N MFMAs that use it.
template <class T, int PAR>
__device__ __forceinline__ void advance(const uint16_t* sA, uint32_t buf, int ks,
                                        const Frag& f, Ops<T>& o0, Ops<T>& o1,
                                        floatx4 (&acc)[T::BLK_M][T::BLK_N]) {
  if constexpr (T::INPLACE) {
    // B: o0 holds the even steps' fragments, o1 the odd ones'; A: always o0, in place
    const Ops<T>& cb = PAR == 0 ? o0 : o1;
    Ops<T>& nbo = PAR == 0 ? o1 : o0;
    const char* a = reinterpret_cast<const char*>(sA) + f.a(ks) + buf * (T::SA * 2);
    const char* b = reinterpret_cast<const char*>(sA) + f.b(ks) + buf * (T::SB * 2);
#pragma unroll
    for (int j = 0; j < T::BLK_N; ++j) nbo.b[j] = as_bf16x8(*reinterpret_cast<const u16x8*>(b + j * kBlkBytes));
#pragma unroll
    for (int i = 0; i < T::BLK_M; ++i) {
#pragma unroll
      for (int j = 0; j < T::BLK_N; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o0.a[i], cb.b[j], acc[i][j], 0, 0, 0);
      o0.a[i] = as_bf16x8(*reinterpret_cast<const u16x8*>(a + i * kBlkBytes));
    }
#pragma unroll
    for (int j = 0; j < T::BLK_N; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // B fragment j
    }
#pragma unroll
    for (int i = 1; i < T::BLK_M; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // A fragment i - 1
      __builtin_amdgcn_sched_group_barrier(0x008, T::BLK_N, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);     // A fragment BLK_M - 1
  } else if constexpr (PAR == 0) {
    load_ops<T>(sA, buf, ks, f, o1);
    mfma_ops<T>(o0, acc);
    interleave<T>();
  } else {
    load_ops<T>(sA, buf, ks, f, o0);
    mfma_ops<T>(o1, acc);
    interleave<T>();
  }
}

// The last K step (an odd step): its operands are in o1 (A in o0 when read in place).
template <class T>
__device__ __forceinline__ void last_step(const Ops<T>& o0, const Ops<T>& o1,
                                          floatx4 (&acc)[T::BLK_M][T::BLK_N]) {
#pragma unroll
  for (int i = 0; i < T::BLK_M; ++i)
#pragma unroll
    for (int j = 0; j < T::BLK_N; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(T::INPLACE ? o0.a[i] : o1.a[i], o1.b[j],
                                                           acc[i][j], 0, 0, 0);
}

static_assert(KS == 2, "a stage is two K steps: advance<0> inside it, advance<1> across stages");

// One K step kt whose stage sits in ring buffer BUF, while every later stage up to
// kt + T::STAGES - 1 is already issued: o0 holds the operands of its first 32-wide step.
// The second step's operands are read while the first step's MFMAs run; once every wave
// has them (and stage kt + 1 has landed), the buffer is refilled with stage kt + T::STAGES
// and the next stage's first operands are read while this stage's second MFMAs run.  The
// MFMA order per output element is unchanged: ascending K.
template <class T, int BUF>
__device__ __forceinline__ void steady_step(const DmaCtx<T>& d, const uint16_t* sA, int kt, const Frag& f,
                                            Ops<T>& o0, Ops<T>& o1, floatx4 (&acc)[T::BLK_M][T::BLK_N]) {
  advance<T, 0>(sA, BUF, 1, f, o0, o1, acc);
  wait_and_barrier<(T::STAGES - 2) * T::PER>();
  if (d.issuer) dma_stage_at<T>(d, BUF, kt + T::STAGES);
  advance<T, 1>(sA, (BUF + 1) % T::STAGES, 0, f, o0, o1, acc);
}

template <class T, int BUF>
__device__ __forceinline__ void unrolled_steps(const DmaCtx<T>& d, const uint16_t* sA, int kt,
                                               const Frag& f, Ops<T>& o0, Ops<T>& o1,
                                               floatx4 (&acc)[T::BLK_M][T::BLK_N]) {
  if constexpr (BUF < T::STAGES) {
    steady_step<T, BUF>(d, sA, kt + BUF, f, o0, o1, acc);
    unrolled_steps<T, BUF + 1>(d, sA, kt, f, o0, o1, acc);
  }
}

// k_split: K columns per blockIdx.y (K itself for bi_gemm, whose grid has one y); slice y
// reads A and B from k = y k_split on and writes its fp32 result split_stride bytes further
// into C (the split-K comparison variant and the fixed split).
template <class T>
__global__ __launch_bounds__(T::THREADS, T::WAVES_PER_SIMD) void gemm_dma_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, void* __restrict__ C, int M,
    int N, int K, int64_t lda, int64_t ldb, int64_t ldc, int c_f32, int tiles_m, int tiles_n,
    int k_split, int64_t split_stride) {
  if (blockIdx.y > 0) {
    const int kb = static_cast<int>(blockIdx.y) * k_split;
    A += kb;
    B += kb;
    K = min(k_split, K - kb);
    C = static_cast<char*>(C) + static_cast<int64_t>(blockIdx.y) * split_stride;
  } else {
    K = min(k_split, K);
  }
  // one LDS block: the A stages, then the B stages; reused by the epilogue
  __shared__ __attribute__((aligned(1024))) uint16_t smem[T::STAGES * (T::SA + T::SB)];
  uint16_t* const sA = smem;
  uint16_t* const sB = smem + T::STAGES * T::SA;

  // Tile order: consecutive workgroup ids land on different XCDs (round robin over 8), so
  // give each XCD a contiguous band of tiles, walked column-major inside bands of 8
  // tile-rows (A rows and B columns then stay in that XCD's L2).
  const int nwg = tiles_m * tiles_n;
  int id = blockIdx.x;
  if ((nwg & 7) == 0) id = (id & 7) * (nwg >> 3) + (id >> 3);
  const int group = 8;
  const int per_group = group * tiles_n;
  const int gi = id / per_group;
  const int first_m = gi * group;
  const int gm = min(tiles_m - first_m, group);
  const int tm = first_m + (id % per_group) % gm;
  const int tn = (id % per_group) / gm;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / T::WAVES_N, wn = wave % T::WAVES_N;

  // DMA assignment: load j of issuing wave w fills tile rows RPI j .. RPI j + RPI - 1 of
  // its share (A rows w TM/DW .., B rows w TN/DW ..); lane l writes chunk position l % CPR
  // of its row with k-chunk (l % CPR) ^ swz(row).
  DmaCtx<T> d;
  d.A = A;
  d.B = B;
  d.K = K;
  d.nk = (K + DBK - 1) / DBK;
  d.ktail = (K % DBK) != 0;
  d.issuer = wave < T::DW;
  const int dw = wave % T::DW;   // (only issuing waves use what follows)
  d.lds_a = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(sA)) + (T::TM / T::DW) * dw * DBK * 2;
  d.lds_b = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(sB)) + (T::TN / T::DW) * dw * DBK * 2;
  // every wave's share starts at a multiple of 16 rows, so swz(R) = swz(RPI j + l / CPR),
  // which depends on j only through its parity
  static_assert((T::TM / T::DW) % 16 == 0 && (T::TN / T::DW) % 16 == 0 && RPI == 8, "row shares");
  d.kc[0] = ((lane % CPR) ^ swz(lane / CPR)) * 8;
  d.kc[1] = ((lane % CPR) ^ swz(RPI + lane / CPR)) * 8;
  d.ra_share = tm * T::TM + (T::TM / T::DW) * dw;
  d.rb_share = tn * T::TN + (T::TN / T::DW) * dw;
  d.a_last = M - 1;
  d.b_last = N - 1;
  d.lda2 = static_cast<uint32_t>(lda * 2);
  d.ldb2 = static_cast<uint32_t>(ldb * 2);
  if constexpr (!T::OTF) {
#pragma unroll
    for (int j = 0; j < T::NJA; ++j) {
      const int ra = min(d.ra_share + lane / CPR + RPI * j, M - 1);
      d.aoff[j] = static_cast<uint32_t>((static_cast<int64_t>(ra) * lda + d.kc[j & 1]) * 2);
    }
    if constexpr (T::BKN) {
      // load j of issuing wave dw: k row (DBK / DW) dw + RPK j + l / CPRN of the stage, the
      // chunk of 8 columns that lands at position l % CPRN; a chunk past N reads columns 0..7
      // instead (those outputs are not stored)
#pragma unroll
      for (int j = 0; j < T::NJB; ++j) {
        const int row = (DBK / T::DW) * dw + T::RPK * j + lane / T::CPRN;
        int n = tn * T::TN + 8 * ((lane % T::CPRN) ^ swzk<T::CPRN>(row));
        if (n >= N) n = 0;
        d.knrow[j] = row;
        d.boff[j] = static_cast<uint32_t>((static_cast<int64_t>(row) * ldb + n) * 2);
      }
    } else {
#pragma unroll
      for (int j = 0; j < T::NJB; ++j) {
        const int rb = min(d.rb_share + lane / CPR + RPI * j, N - 1);
        d.boff[j] = static_cast<uint32_t>((static_cast<int64_t>(rb) * ldb + d.kc[j & 1]) * 2);
      }
    }
  }
  d.ldb = ldb;
  // operand reads: lane holds row (lane % 16) of each 16-row block and k-chunk
  // 4 ks + lane / 16 of each 32-wide K step (swz(row) = swz(lane % 16) in every block)
  Frag f;
  const int orow = lane & 15, okc = lane >> 4;
  {
    const int c = (okc ^ swz(orow)) * 8;
    f.a0 = static_cast<uint32_t>(((wm * T::BLK_M * 16 + orow) * DBK + c) * 2);
    f.b0 = static_cast<uint32_t>((T::STAGES * T::SA + (wn * T::BLK_N * 16 + orow) * DBK + c) * 2);
    // opaque to the compiler: the constant parts of a read's address (ring buffer, block)
    // then stay small enough for the read's immediate offset
    asm volatile("" : "+v"(f.a0), "+v"(f.b0));
  }

  floatx4 acc[T::BLK_M][T::BLK_N];
#pragma unroll
  for (int i = 0; i < T::BLK_M; ++i)
#pragma unroll
    for (int j = 0; j < T::BLK_N; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.f;

  // prologue: every ring buffer receives a stage
  const int nk = d.nk;
#pragma unroll
  for (int st = 0; st < T::STAGES; ++st)
    if (st < nk && d.issuer) dma_stage_at<T>(d, st, st);
  Ops<T> o0, o1;
  wait_stage<T::PER, T::STAGES - 1>(min(T::STAGES - 1, nk - 1));
  if (d.ktail && nk == 1) {
    if (d.issuer) zero_k_tail<T>(d, sA, sB, 0, 0, wave, lane);
    wait_and_barrier<0>();
  }
  load_ops<T>(sA, 0, 0, f, o0);

  // steady state: steps kt with stage kt + T::STAGES still to issue
  const int steady = nk - T::STAGES > 0 ? nk - T::STAGES : 0;
  int kt = 0;
  for (; kt + T::STAGES <= steady; kt += T::STAGES) unrolled_steps<T, 0>(d, sA, kt, f, o0, o1, acc);
  for (; kt < steady; ++kt) {
    const int buf = kt % T::STAGES;
    advance<T, 0>(sA, buf, 1, f, o0, o1, acc);
    wait_and_barrier<(T::STAGES - 2) * T::PER>();
    if (d.issuer) dma_stage_at<T>(d, buf, kt + T::STAGES);
    advance<T, 1>(sA, (kt + 1) % T::STAGES, 0, f, o0, o1, acc);
  }
  // drain: nothing left to issue; stages kt + 1 .. nk - 1 may still be in flight
  for (; kt < nk - 1; ++kt) {
    advance<T, 0>(sA, kt % T::STAGES, 1, f, o0, o1, acc);
    wait_stage<T::PER, T::STAGES - 2>(min(T::STAGES - 2, nk - 2 - kt));
    if (d.ktail && kt + 1 == nk - 1) {
      if (d.issuer) zero_k_tail<T>(d, sA, sB, (kt + 1) % T::STAGES, kt + 1, wave, lane);
      wait_and_barrier<0>();
    }
    advance<T, 1>(sA, (kt + 1) % T::STAGES, 0, f, o0, o1, acc);
  }
  advance<T, 0>(sA, (nk - 1) % T::STAGES, 1, f, o0, o1, acc);
  last_step<T>(o0, o1, acc);

  // epilogue: register r of block (i, j) is row 4 (lane / 16) + r and column lane % 16 of
  // that block
  if (c_f32 != kOutF32) {
    // bf16 output goes through LDS: each wave rounds its WM x WN sub-tile into its own
    // region (16-byte chunk c of row r at position c ^ (r % CW)), then reads it back as
    // 16-byte row pieces, so a store instruction writes whole sub-tile row segments
    constexpr int WM = T::BLK_M * 16, WN = T::BLK_N * 16;
    constexpr int CW = WN / 8, RPW = 64 / CW;   // chunks per row, rows per read
    static_assert(T::NW * WM * WN <= T::STAGES * (T::SA + T::SB) && WM % RPW == 0, "epilogue staging");
    __syncthreads();   // every wave is done with the stage buffers
    uint16_t* const st = smem + wave * (WM * WN);
#pragma unroll
    for (int i = 0; i < T::BLK_M; ++i)
#pragma unroll
      for (int j = 0; j < T::BLK_N; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int rw = i * 16 + 4 * (lane >> 4) + r;
          const int cw = j * 16 + (lane & 15);
          st[rw * WN + (((cw >> 3) ^ (rw % CW)) << 3) + (cw & 7)] = f32_to_bf16(acc[i][j][r]);
        }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");   // the region is this wave's own
    const bool vec = ((reinterpret_cast<uintptr_t>(C) | static_cast<uintptr_t>(ldc * 2)) & 15) == 0;
    if (c_f32 == kOutSwiGLU) {
      // each 32-column block holds 16 gate then 16 up columns; output chunk q of block b
      // (8 columns) pairs staged chunks 4 b + q and 4 b + 2 + q
      constexpr int OC = WN / 16, ORW = 64 / OC;   // output chunks per row, rows per pass
      const int oc = lane % OC;
      const int cg = 4 * (oc >> 1) + (oc & 1), cu = cg + 2;
      const int ocol = (tn * T::TN + wn * WN) / 2 + oc * 8;
      uint16_t* const Ob = static_cast<uint16_t*>(C);
#pragma unroll
      for (int it = 0; it < WM / ORW; ++it) {
        const int rw = it * ORW + lane / OC;
        const u16x8 g = *reinterpret_cast<const u16x8*>(st + rw * WN + ((cg ^ (rw % CW)) << 3));
        const u16x8 u = *reinterpret_cast<const u16x8*>(st + rw * WN + ((cu ^ (rw % CW)) << 3));
        const int row = tm * T::TM + wm * WM + rw;
        if (row >= M || 2 * ocol >= N) continue;
        u16x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = swiglu_bf16(g[e], u[e]);
        uint16_t* const dst = Ob + static_cast<int64_t>(row) * ldc + ocol;
        if (vec) {
          *reinterpret_cast<u16x8*>(dst) = o;
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) dst[e] = o[e];
        }
      }
      return;
    }
    const int cc = lane % CW;
    const int col = tn * T::TN + wn * WN + cc * 8;
    uint16_t* const Cb = static_cast<uint16_t*>(C);
#pragma unroll
    for (int it = 0; it < WM / RPW; ++it) {
      const int rw = it * RPW + lane / CW;
      const u16x8 v = *reinterpret_cast<const u16x8*>(st + rw * WN + ((cc ^ (rw % CW)) << 3));
      const int row = tm * T::TM + wm * WM + rw;
      if (row >= M || col >= N) continue;
      uint16_t* const dst = Cb + static_cast<int64_t>(row) * ldc + col;
      if (vec && col + 8 <= N) {
        *reinterpret_cast<u16x8*>(dst) = v;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (col + e < N) dst[e] = v[e];
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < T::BLK_M; ++i)
#pragma unroll
    for (int j = 0; j < T::BLK_N; ++j) {
      const int col = tn * T::TN + (wn * T::BLK_N + j) * 16 + (lane & 15);
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = tm * T::TM + (wm * T::BLK_M + i) * 16 + 4 * (lane >> 4) + r;
        if (row >= M) continue;
        static_cast<float*>(C)[static_cast<int64_t>(row) * ldc + col] = acc[i][j][r];
      }
    }
}

// Workgroup tile of the main kernel for an M x N output.  Every tile gives every output
// element the same bits (same instruction, same K order), so this choice changes only the
// time.  The 256 x 256 tile streams half the operand bytes per flop but runs one workgroup
// per CU; the 128 x 128 tile runs two per CU, or one with a deeper ring when the grid has
// no more tiles than CUs.  The cost counts rounds of the CU array, with round times
// measured on MI355X at K = 4096 (all scale with K): 256 x 256: 109; 128 x 128 two per CU:
// 59-66 (64 taken: at 59 wide-N grids of 2048 rows would pick the slower 128 x 128 tiles),
// one per CU: 46.
enum class TileKind { k64, k64x128, k128, k128deep, k256 };

TileKind pick_tile(int64_t M, int64_t N, int cus) {
  const int64_t n256 = ((M + 255) / 256) * ((N + 255) / 256);
  const int64_t n128 = ((M + 127) / 128) * ((N + 127) / 128);
  if (n128 <= cus) {
    // one round or less: the largest tile whose grid still covers three quarters of the CUs;
    // up to 64 rows (which reach these tiles only when N is too wide for the few-row kernel)
    // the 64 x 64 tile, whose grid of up to twice the CUs streams the weights faster
    // (measured at 33..64 x 28672 x 4096 and x 32000 x 4096: 0.92-1.01 of the time of the
    // 128 x 128 tile)
    if (M <= 64) return TileKind::k64;
    const int64_t n64x128 = ((M + 63) / 64) * ((N + 127) / 128);
    if (4 * n128 >= 3 * cus) return TileKind::k128deep;
    if (4 * n64x128 >= 3 * cus) return TileKind::k64x128;
    return TileKind::k64;
  }
  const int64_t cost256 = 109 * ((n256 + cus - 1) / cus);
  const int64_t rem = n128 % (2 * cus);
  const int64_t cost128 = 64 * (n128 / (2 * cus)) + (rem == 0 ? 0 : rem <= cus ? 46 : 64);
  return cost256 < cost128 ? TileKind::k256 : TileKind::k128;
}

// The residual add and RMSNorm in front of the few-row kernel (NORM): the kernel's A is the
// first addend a [M, K] (rows contiguous), b the second, s = a + b goes to `sum` (workgroup 0
// writes it), and the instruction's A operand is y = rmsnorm(s) with gamma, staged in LDS.
constexpr int kNormRows = 4;   // rows of a NORM call (4 x 4096: 32 KB of LDS per workgroup)
struct NormArgs {
  const uint16_t* b = nullptr;
  const uint16_t* gamma = nullptr;
  uint16_t* sum = nullptr;
  float eps = 0.f;
};

// The normalised rows of a NORM kernel, bf16 in LDS (row m at m Ks, zeros from K to Kp), with the
// bits of bi_add_rmsnorm: s = bf16(a + b); thread t of the 256 is tree lane t (T = min(256,
// K/8) lanes) and adds the squares of its 8-element vectors t, t + T (NV of them at most) in
// ascending order from +0; each wave's butterfly gives its tree wave's sum, and the four are
// combined as (w0 + w1) + (w2 + w3); r = rms_scale(sum, K, eps); y = (s r) g rounded once.
// Workgroup 0 also writes s to the sum output.  norm_load issues every load of the rows and
// of gamma (a slot past the row reads vector 0 and adds +0, which leaves a sum of squares
// unchanged), so they are all in flight together; norm_store waits for them.
template <int NV>
struct NormRows {
  int v[NV];
  bool ok[NV];
  u16x8 g[NV], a[kNormRows][NV], b[kNormRows][NV];
  __device__ void load(const uint16_t* __restrict__ pa, const NormArgs& na, int M, int K) {
    const int t = threadIdx.x, nvec = K / 8, T = min(256, nvec);
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int vv = t + j * T;
      ok[j] = t < T && vv < nvec;
      v[j] = ok[j] ? vv : 0;
      g[j] = *reinterpret_cast<const u16x8*>(na.gamma + 8 * v[j]);
    }
#pragma unroll
    for (int m = 0; m < kNormRows; ++m)
      if (m < M) {
#pragma unroll
        for (int j = 0; j < NV; ++j) {
          a[m][j] = *reinterpret_cast<const u16x8*>(pa + static_cast<int64_t>(m) * K + 8 * v[j]);
          b[m][j] = *reinterpret_cast<const u16x8*>(na.b + static_cast<int64_t>(m) * K + 8 * v[j]);
        }
      }
  }
  // row m of y at sy + m Ks (Ks = Kp + 32: rows 64 bytes apart in the banks, so the GEMM
  // wave's 16 lanes of one step, on up to 4 rows and 4 k offsets, read 16 disjoint bank groups)
  __device__ void store(const NormArgs& na, bool write_sum, int M, int K, int Kp, int Ks, uint16_t* sy,
                        float* part) {
    const int t = threadIdx.x;
#pragma unroll
    for (int m = 0; m < kNormRows; ++m)
      if (m < M) {
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
          u16x8 q;
#pragma unroll
          for (int i = 0; i < 8; ++i) q[i] = f32_to_bf16(bf16_to_f32(a[m][j][i]) + bf16_to_f32(b[m][j][i]));
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float x = bf16_to_f32(q[i]);
            acc = acc + (ok[j] ? x * x : 0.f);
          }
          if (ok[j]) {
            *reinterpret_cast<u16x8*>(sy + m * Ks + 8 * v[j]) = q;
            if (write_sum) *reinterpret_cast<u16x8*>(na.sum + static_cast<int64_t>(m) * K + 8 * v[j]) = q;
          }
        }
        const float ws = wave_tree_sum(acc);
        if ((t & 63) == 0) part[m * 4 + (t >> 6)] = ws;
      }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < kNormRows; ++m)
      if (m < M) {
        const float r = rms_scale((part[m * 4] + part[m * 4 + 1]) + (part[m * 4 + 2] + part[m * 4 + 3]), K, na.eps);
#pragma unroll
        for (int j = 0; j < NV; ++j) {
          if (!ok[j]) continue;
          uint16_t* p = sy + m * Ks + 8 * v[j];
          const u16x8 q = *reinterpret_cast<const u16x8*>(p);
          u16x8 qy;
#pragma unroll
          for (int i = 0; i < 8; ++i) qy[i] = f32_to_bf16((bf16_to_f32(q[i]) * r) * bf16_to_f32(g[j][i]));
          *reinterpret_cast<u16x8*>(p) = qy;
        }
        for (int vz = K / 8 + t; vz < Kp / 8; vz += 256) *reinterpret_cast<u16x8*>(sy + m * Ks + 8 * vz) = u16x8{};
      }
    __syncthreads();
  }
};

// Few-row GEMM (M <= 64).  At decode sizes the weight stream bounds the call, and a
// 128 x 128 grid leaves most CUs idle (N = 4096 gives 32 workgroups).  Here one wave owns CB
// 16-column blocks and RB 16-row blocks (all M rows, or with `split` = 2 or 4 one of that many
// row slices of 16 RB rows; the waves of a column block then sit on one XCD, whose L2 serves
// the later ones their weights) and loads its instruction operands straight from global memory into
// registers, PF K steps ahead: lane l takes the 16 bytes at row l % 16, k offset
// 32 t + 8 (l / 16) of K step t, which is exactly its operand of the instruction, so there
// is no LDS, no barrier and no other wave to wait for.  What is left is the chain itself:
// K / 32 dependent instructions per accumulator.  Every output element
// sees the instruction sequence of every other configuration (same instruction, +0 start,
// ascending 32-wide K steps, same lane-to-k assignment), so its bits do not change.
// K is a multiple of 8 with at least 2 PF whole steps; a last, partial step is loaded up
// front, with the chunks at or past K replaced by zeros.
// PAIR: two waves per workgroup, one 16-column block each (CB = 1, split = 1): for SwiGLU
// the second wave's block (the up columns) reaches the first through LDS, so a wave streams
// one block, as in the plain one-block kernel.
// PK: B in the tiled layout of bi_pack_b (tile (column block, 32-wide step) = 1 KB, the
// 16-byte piece of lane l at offset 16 l, which is lane l's instruction operand): each load
// of a wave reads one contiguous kilobyte instead of 64 bytes from each of 16 rows.  Only
// the addresses change; the operands, the instruction sequence and so the bits do not.
// NORM > 0 (one row block, one wave's blocks, no split): A and na describe a residual add +
// RMSNorm whose output is the A operand, staged in LDS by NormRows ([M][32 ceil(K/32) + 32]
// bf16, dynamic; NORM vectors per tree lane: 1 for K <= 2048, 2 for K <= 4096).  The workgroup has
// 256 threads, one per tree lane: wave 0 is the GEMM wave, waves 1..3 help normalise and
// then leave (no barrier follows).  The rows' loads, then the weight prefetch, go out before
// any of it is computed.
template <int RB, int CB, int PF, bool PAIR = false, bool PK = false, int NORM = 0>
__global__ __launch_bounds__(NORM > 0 ? 256 : (PAIR ? 128 : 64)) void gemm_rows_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, void* __restrict__ C, int M,
    int N, int K, int64_t lda, int64_t ldb, int64_t ldc, int c_f32, int split, int k_split,
    int64_t split_stride, NormArgs na) {
  static_assert(!PAIR || CB == 1, "paired waves hold one block each");
  static_assert(NORM == 0 || (RB == 1 && !PAIR), "the normalised rows are one row block of one wave");
  extern __shared__ __attribute__((aligned(16))) uint16_t sy[];
  // K slice of blockIdx.y (as in gemm_dma_kernel; the split-K variant and the fixed split)
  if (blockIdx.y > 0) {
    const int kb = static_cast<int>(blockIdx.y) * k_split;
    A += kb;
    B += kb;
    K = min(k_split, K - kb);
    C = static_cast<char*>(C) + static_cast<int64_t>(blockIdx.y) * split_stride;
  } else {
    K = min(k_split, K);
  }
  const int lane = threadIdx.x & 63;
  const int wave = PAIR || NORM > 0 ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : 0;
  // workgroup id -> (column block, row slice): ids 8 s + x, s = split c .. split c + split - 1
  // (one XCD) share column block 8 c + x; with split = 1 the id is the column block (the
  // pair's, for PAIR)
  int cblk = PAIR ? 2 * blockIdx.x + wave : blockIdx.x, row0 = 0;
  if (split > 1) {
    const int x = blockIdx.x & 7, slot = blockIdx.x >> 3;
    cblk = (slot / split) * 8 + x;
    row0 = (slot % split) * RB * 16;
    if (cblk * CB * 16 >= N || row0 >= M) return;   // grid padding (wave-uniform)
  }
  const int col0 = cblk * (CB * 16);
  const int kl = 8 * (lane >> 4);
  const uint16_t* pa[RB];
  const uint16_t* pb[CB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)   // rows past M repeat the last row; they are never stored
    pa[rb] = A + static_cast<int64_t>(min(row0 + rb * 16 + (lane & 15), M - 1)) * lda + kl;
  const int64_t nk32 = (K + 31) / 32;   // tiles per column block (PK)
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)   // (PK: blocks past N repeat the last one; never stored)
    pb[cb] = PK ? B + static_cast<int64_t>(min(cblk * CB + cb, (N - 1) / 16)) * nk32 * 512 + lane * 8
                : B + static_cast<int64_t>(min(col0 + cb * 16 + (lane & 15), N - 1)) * ldb + kl;
  bf16x8 ra[PF][RB], rv[PF][CB];
  // NORM: lane l's A operand row (clamped to M - 1 as above) in the staged rows
  const int Kp = static_cast<int>(nk32) * 32, Ks = Kp + 32;
  const int arow = NORM > 0 ? min(row0 + (lane & 15), M - 1) * Ks + kl : 0;
  auto load_a = [&](int t, bf16x8 (&dst_a)[RB]) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
      dst_a[rb] = NORM > 0 ? as_bf16x8(*reinterpret_cast<const u16x8*>(sy + arow + 32 * t))
                       : as_bf16x8(*reinterpret_cast<const u16x8*>(pa[rb] + 32 * t));
  };
  auto load_b = [&](int t, bf16x8 (&dst_b)[CB]) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) dst_b[cb] = as_bf16x8(*reinterpret_cast<const u16x8*>(pb[cb] + (PK ? 512 : 32) * t));
  };
  // (NORM: the A operand is read from LDS at the step that uses it, see mma_at; only the
  // weights ride the prefetch ring)
  auto load = [&](int t, bf16x8 (&dst_a)[RB], bf16x8 (&dst_b)[CB]) {
    if constexpr (NORM == 0) load_a(t, dst_a);
    load_b(t, dst_b);
  };
  floatx4 acc[RB][CB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[rb][cb][r] = 0.f;
  auto mma = [&](const bf16x8 (&a)[RB], const bf16x8 (&b)[CB]) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
        acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[rb], b[cb], acc[rb][cb], 0, 0, 0);
  };
  auto mma_at = [&](int t, const bf16x8 (&a)[RB], const bf16x8 (&b)[CB]) {
    if constexpr (NORM > 0) {
      bf16x8 an[RB];
      load_a(t, an);
      mma(an, b);
    } else {
      mma(a, b);
    }
  };
  const int nsteps = K / 32;   // whole steps, >= 2 PF (the host checks)
  // the partial last step (if any): a chunk at or past K re-reads k offset 0 of its row and
  // is zeroed once it has landed
  const int ktail = 32 * nsteps;
  const bool tin = ktail + kl < K;
  const int tofs = tin ? ktail : -kl;
  bf16x8 ta[RB], tb[CB];
  // (PK: the partial step's tile, index nsteps, exists only when K is not a multiple of 32;
  // its pieces past K hold zeros)
  const int64_t tofs_b = PK ? (ktail < K ? int64_t(512) * nsteps : 0) : tofs;
  if constexpr (NORM > 0) {
    // the rows and gamma, then (GEMM wave) the weights; the rows are normalised while the
    // weights stream in (zeros past K in LDS, so the partial step needs no mask)
    __shared__ float part[kNormRows * 4];
    NormRows<NORM> rows;
    rows.load(A, na, M, K);
    if (wave == 0) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) tb[cb] = as_bf16x8(*reinterpret_cast<const u16x8*>(pb[cb] + tofs_b));
#pragma unroll
      for (int p = 0; p < PF; ++p) load_b(p, rv[p]);
    }
    rows.store(na, blockIdx.x == 0, M, K, Kp, Ks, sy, part);
    if (wave != 0) return;   // the helpers' part is done
    const bf16x8 z = {};
    ta[0] = ktail < K ? as_bf16x8(*reinterpret_cast<const u16x8*>(sy + arow + ktail)) : z;
  } else {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) ta[rb] = as_bf16x8(*reinterpret_cast<const u16x8*>(pa[rb] + tofs));
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) tb[cb] = as_bf16x8(*reinterpret_cast<const u16x8*>(pb[cb] + tofs_b));
#pragma unroll
    for (int p = 0; p < PF; ++p) load(p, ra[p], rv[p]);
  }
  // full rounds: step t multiplies slot t % PF and refills it with step t + PF (straight-line
  // code, so the compiler's load counters stay exact and PF steps stay in flight)
  int t0 = 0;
  for (; t0 + 2 * PF <= nsteps; t0 += PF) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      mma_at(t0 + p, ra[p], rv[p]);
      load(t0 + PF + p, ra[p], rv[p]);
    }
  }
  // last (up to 2 PF - 1) whole steps
#pragma unroll
  for (int p = 0; p < PF; ++p) {
    if (t0 + p < nsteps) {
      mma_at(t0 + p, ra[p], rv[p]);
      if (t0 + PF + p < nsteps) load(t0 + PF + p, ra[p], rv[p]);
    }
  }
#pragma unroll
  for (int p = 0; p < PF; ++p)
    if (t0 + PF + p < nsteps) mma_at(t0 + PF + p, ra[p], rv[p]);
  if (ktail < K) {
    const bf16x8 z = {};
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) ta[rb] = tin ? ta[rb] : z;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) tb[cb] = tin ? tb[cb] : z;
    mma(ta, tb);
  }
  // register r of block (rb, cb) is row 16 rb + 4 (lane / 16) + r, column 16 cb + lane % 16
  if (PAIR && c_f32 == kOutSwiGLU) {
    // wave 0 holds 16 gate columns, wave 1 the matching 16 up columns
    __shared__ uint16_t up[RB][4][64];
    if (wave == 1) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r) up[rb][r][lane] = f32_to_bf16(acc[rb][0][r]);
    }
    __syncthreads();
    if (wave == 1) return;
    const int ocol = blockIdx.x * 16 + (lane & 15);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = row0 + rb * 16 + 4 * (lane >> 4) + r;
        if (row < M)   // (N is a multiple of 32: every block lies inside N)
          static_cast<uint16_t*>(C)[static_cast<int64_t>(row) * ldc + ocol] =
              swiglu_bf16(f32_to_bf16(acc[rb][0][r]), up[rb][r][lane]);
      }
    return;
  }
  if (c_f32 == kOutSwiGLU) {
    // CB == 2: block 0 holds 16 gate columns, block 1 the matching 16 up columns
    const int ocol = col0 / 2 + (lane & 15);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = row0 + rb * 16 + 4 * (lane >> 4) + r;
        if (row < M)   // (N is a multiple of 32: every block lies inside N)
          static_cast<uint16_t*>(C)[static_cast<int64_t>(row) * ldc + ocol] =
              swiglu_bf16(f32_to_bf16(acc[rb][0][r]), f32_to_bf16(acc[rb][CB - 1][r]));
      }
    return;
  }
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int col = col0 + cb * 16 + (lane & 15);
    if (col >= N) continue;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = row0 + rb * 16 + 4 * (lane >> 4) + r;
        if (row >= M) continue;
        if (c_f32)
          static_cast<float*>(C)[static_cast<int64_t>(row) * ldc + col] = acc[rb][cb][r];
        else
          static_cast<uint16_t*>(C)[static_cast<int64_t>(row) * ldc + col] = f32_to_bf16(acc[rb][cb][r]);
      }
  }
}

// Split-K comparison variant for up to 4 rows (NOT batch-invariant; bi_gemm never runs it):
// a workgroup of 4 waves owns one 16-column block, wave w runs the K steps [w S, w S + S)
// (S = 8, 16 or 32, the smallest with 4 S covering K) from +0 with every load of its segment
// issued at once, and the four partials are added in wave order -- so all four SIMDs of a CU
// stream weights, at the price of a different association than the unsplit chain.  The rows
// of A are staged in LDS and read from there as the instruction's A operand.  (Handing the
// one chain from wave to wave instead, which keeps bi_gemm's order, measured no faster than
// one wave per block: the launch and the weight stream, not the chain, bound these sizes.)
constexpr int kWcWaves = 4, kWcRows = 4;

template <int SEG>
__global__ __launch_bounds__(256, 2) void gemm_wsplit_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, void* __restrict__ C, int M,
    int N, int K, int64_t lda, int64_t ldb, int64_t ldc, int c_f32) {
  constexpr int KP = kWcWaves * SEG * 32;   // staged row length (zeros past K)
  constexpr int LDR = KP + 8;               // LDS row pitch: rows 16 bytes apart in the banks
  __shared__ __attribute__((aligned(16))) uint16_t sa[kWcRows * LDR];
  __shared__ floatx4 xfer[kWcWaves * 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col0 = blockIdx.x * 16;
  const int kl = 8 * (lane >> 4);
  const int k0 = wave * SEG * 32;           // first k of this wave's segment
  // 1. every B operand of the segment (a chunk at or past K reads offset 0 of its row and
  //    is replaced by zeros)
  const uint16_t* pb = B + static_cast<int64_t>(min(col0 + (lane & 15), N - 1)) * ldb + kl;
  u16x8 braw[SEG];
#pragma unroll
  for (int s = 0; s < SEG; ++s) {
    const int k = k0 + 32 * s;
    braw[s] = *reinterpret_cast<const u16x8*>(pb + (k + kl < K ? k : -kl));
  }
  // 2. A rows into LDS, zeros past K
  constexpr int cpr = KP / 8;               // 16-byte chunks per staged row
  for (int i = tid; i < M * cpr; i += 256) {
    const int r = i / cpr, k = (i % cpr) * 8;
    u16x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
    if (k < K) v = *reinterpret_cast<const u16x8*>(A + static_cast<int64_t>(r) * lda + k);
    *reinterpret_cast<u16x8*>(sa + r * LDR + k) = v;
  }
  __syncthreads();
  const uint16_t* pa = sa + min(lane & 15, M - 1) * LDR + k0 + kl;
  // this wave's steps (those below ceil(K / 32))
  auto run = [&](floatx4 acc) {
#pragma unroll
    for (int s = 0; s < SEG; ++s) {
      if (k0 + 32 * s >= K) break;          // wave-uniform
      const u16x8 b = (k0 + 32 * s + kl < K) ? braw[s] : u16x8{0, 0, 0, 0, 0, 0, 0, 0};
      const u16x8 a = *reinterpret_cast<const u16x8*>(pa + 32 * s);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), acc, 0, 0, 0);
    }
    return acc;
  };
  floatx4 acc = run(floatx4{0.f, 0.f, 0.f, 0.f});
  xfer[wave * 64 + lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  acc = xfer[lane];
#pragma unroll
  for (int w = 1; w < kWcWaves; ++w) {
    const floatx4 p = xfer[w * 64 + lane];
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = acc[r] + p[r];
  }
  // register r is row 4 (lane / 16) + r, column lane % 16 of the block
  const int col = col0 + (lane & 15);
  if (col >= N) return;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = 4 * (lane >> 4) + r;
    if (row >= M) continue;
    if (c_f32)
      static_cast<float*>(C)[static_cast<int64_t>(row) * ldc + col] = acc[r];
    else
      static_cast<uint16_t*>(C)[static_cast<int64_t>(row) * ldc + col] = f32_to_bf16(acc[r]);
  }
}

// The 4-wave split takes up to 4 rows with K a multiple of 8 in 512 .. 4096 and at most two
// 16-column blocks per CU.
bool use_wsplit(int64_t M, int64_t N, int64_t K) {
  return M >= 1 && M <= kWcRows && K % 8 == 0 && K >= 512 && K <= 4096 &&
         (N + 15) / 16 <= 2 * static_cast<int64_t>(cu_count());
}

void launch_wsplit(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                   int64_t lda, int64_t ldb, int64_t ldc, int cf, hipStream_t s) {
  const int64_t steps = (K + 31) / 32;
  const dim3 grid(static_cast<unsigned>((N + 15) / 16)), block(256);
  const uint16_t* a = static_cast<const uint16_t*>(A);
  const uint16_t* b = static_cast<const uint16_t*>(B);
  if (steps <= kWcWaves * 8)
    gemm_wsplit_kernel<8><<<grid, block, 0, s>>>(a, b, C, int(M), int(N), int(K), lda, ldb, ldc, cf);
  else if (steps <= kWcWaves * 16)
    gemm_wsplit_kernel<16><<<grid, block, 0, s>>>(a, b, C, int(M), int(N), int(K), lda, ldb, ldc, cf);
  else
    gemm_wsplit_kernel<32><<<grid, block, 0, s>>>(a, b, C, int(M), int(N), int(K), lda, ldb, ldc, cf);
}

// Few-row configurations (measured on MI355X at the decode shapes).  A wave's A operand reads
// (RB row blocks per step) come from L2 and hit the same few lines in every wave, so once
// there are several rows a wave takes at least half as many column blocks as row blocks: up
// to 16 rows one 16 x 16 block (16 x 32 from 9 rows on for wide N, and for SwiGLU, whose
// gate and up blocks pair up), up to 32 rows 32 x 32 blocks, above that 64 x 32 blocks, or
// two waves of 32 x 32 per column block (one per 32-row half) while the column blocks
// number under three quarters of the CUs.  Where waves of 16-row slices still fit one round
// (2 or 4 per 32-column block, at most one per CU), each takes a 16 x 32 block: two or four
// times the waves streaming weights, with A reads half the weight reads.
struct RowsCfg {
  int rb, cb, pf, split;
  bool pair = false;   // SwiGLU with one 16-column block per wave, two waves per workgroup
};
RowsCfg rows_cfg(int64_t M, int64_t N, int mode) {
  const int64_t cus = cu_count();
  if (M <= 8 && mode == kOutSwiGLU) return {1, 1, 16, 1, true};
  if (M <= 16) {
    const bool wide = mode == kOutSwiGLU || (M > 8 && (N + 15) / 16 >= 4 * cus);
    return {1, wide ? 2 : 1, 16, 1};
  }
  const int64_t ncb = (N + 31) / 32;
  if (M <= 32) return 2 * ncb <= cus ? RowsCfg{1, 2, 12, 2} : RowsCfg{2, 2, 12, 1};
  if (4 * ncb >= 3 * cus) return {4, 2, 12, 1};
  if (4 * ncb <= cus) return {1, 2, 12, 4};
  return {2, 2, 12, 2};
}

// The few-row kernel for up to 32 rows, and for 33..64 rows while its two waves per 32-column
// block number at most two per CU (wider grids go faster through the LDS-staged tiles, whose
// loads cover whole 128-byte lines), when K is a multiple of 8 with at least 2 PF whole
// 32-wide steps.
bool use_rows(int64_t M, int64_t N, int64_t K, int mode) {
  if (M > 64 || K % 8 != 0) return false;
  if (M > 32 && (N + 31) / 32 > static_cast<int64_t>(cu_count())) return false;
  return K / 32 >= 2 * rows_cfg(M, N, mode).pf;
}

// K-slice launches (the split-K comparison variant and the fixed split): `ks` slices of
// k_split columns along grid y, slice y's fp32 result split_stride bytes into C.  bi_gemm
// launches ks = 1, k_split = K.
struct KSplit {
  int ks = 1;
  int k_split = 0;   // 0: K
  int64_t stride = 0;
};

template <int RB, int CB, int PF, bool PAIR = false, bool PK = false>
void launch_rows_t(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                   int64_t lda, int64_t ldb, int64_t ldc, int cf, int split, hipStream_t s,
                   KSplit sk = {}) {
  const int64_t ncb = (N + CB * 16 - 1) / (CB * 16);
  const unsigned wgs = static_cast<unsigned>(PAIR ? (ncb + 1) / 2 : split == 1 ? ncb : 8 * split * ((ncb + 7) / 8));
  gemm_rows_kernel<RB, CB, PF, PAIR, PK><<<dim3(wgs, sk.ks), dim3(PAIR ? 128 : 64), 0, s>>>(
      static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(B), C, int(M), int(N), int(K),
      lda, ldb, ldc, cf, split, sk.k_split ? sk.k_split : int(K), sk.stride, NormArgs{});
}

// The residual add + RMSNorm fused in front of the few-row kernel (at most kNormRows rows):
// the configurations rows_cfg gives those rows (one 16-column block per wave, paired waves
// for SwiGLU), on an [N, K] or a tiled B.
template <int CB, bool PK>
void launch_rows_norm_t(const void* a, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                        int64_t ldb, int64_t ldc, int cf, NormArgs na, hipStream_t s) {
  const unsigned wgs = static_cast<unsigned>((N + 16 * CB - 1) / (16 * CB));
  const size_t lds = static_cast<size_t>(M) * ((K + 31) / 32 * 32 + 32) * sizeof(uint16_t);
  const uint16_t *pa = static_cast<const uint16_t*>(a), *pb = static_cast<const uint16_t*>(B);
  // K > 2048: two vectors per tree lane, and one-block waves prefetch 32 steps of weights
  // (K / 32 >= 64), which keeps the stream going while the rows are normalised
  if (K <= 2048)
    gemm_rows_kernel<1, CB, 16, false, PK, 1><<<dim3(wgs), dim3(256), lds, s>>>(
        pa, pb, C, int(M), int(N), int(K), K, ldb, ldc, cf, 1, int(K), 0, na);
  else
    gemm_rows_kernel<1, CB, CB == 1 ? 32 : 16, false, PK, 2><<<dim3(wgs), dim3(256), lds, s>>>(
        pa, pb, C, int(M), int(N), int(K), K, ldb, ldc, cf, 1, int(K), 0, na);
}

// The residual add + RMSNorm fused in front of the few-row kernel (at most kNormRows rows): one
// 16-column block per GEMM wave, two (the gate and up blocks) for SwiGLU.
void launch_rows_norm(const void* a, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                      int64_t ldb, int64_t ldc, int cf, bool tiled, NormArgs na, hipStream_t s) {
  if (cf == kOutSwiGLU) {
    if (tiled) launch_rows_norm_t<2, true>(a, B, C, M, N, K, ldb, ldc, cf, na, s);
    else launch_rows_norm_t<2, false>(a, B, C, M, N, K, ldb, ldc, cf, na, s);
  } else {
    if (tiled) launch_rows_norm_t<1, true>(a, B, C, M, N, K, ldb, ldc, cf, na, s);
    else launch_rows_norm_t<1, false>(a, B, C, M, N, K, ldb, ldc, cf, na, s);
  }
}

// The few-row kernel on a tiled B (bi_pack_b), in the configuration rows_cfg gives (for
// 33..64 rows also on grids wider than the CUs, which on an [N, K] B go to the LDS-staged
// tiles).
void launch_rows_tiled(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                       int64_t lda, int64_t ldc, int cf, hipStream_t s) {
  const RowsCfg c = rows_cfg(M, N, cf);
  if (c.pair) launch_rows_t<1, 1, 16, true, true>(A, B, C, M, N, K, lda, 0, ldc, cf, 1, s);
  else if (c.rb == 4) launch_rows_t<4, 2, 12, false, true>(A, B, C, M, N, K, lda, 0, ldc, cf, 1, s);
  else if (c.rb == 2) launch_rows_t<2, 2, 12, false, true>(A, B, C, M, N, K, lda, 0, ldc, cf, c.split, s);
  else if (c.split > 1) launch_rows_t<1, 2, 12, false, true>(A, B, C, M, N, K, lda, 0, ldc, cf, c.split, s);
  else if (c.cb == 2) launch_rows_t<1, 2, 16, false, true>(A, B, C, M, N, K, lda, 0, ldc, cf, 1, s);
  else launch_rows_t<1, 1, 16, false, true>(A, B, C, M, N, K, lda, 0, ldc, cf, 1, s);
}

// Tiled layout: tile (column block b, step t) holds B[16 b + r][32 t + 8 g + e] at
// ((b * ceil(K/32) + t) * 64 + r + 16 g) * 8 + e, zero where 16 b + r >= N or k >= K.
__global__ void pack_b_kernel(const uint16_t* __restrict__ B, int64_t N, int64_t K, int64_t ldb,
                              uint16_t* __restrict__ out, int64_t nk32, int64_t pieces) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= pieces) return;
  const int lane = static_cast<int>(i & 63);
  const int64_t tile = i >> 6;
  const int64_t b = tile / nk32, t = tile % nk32;
  const int64_t n = 16 * b + (lane & 15), k0 = 32 * t + 8 * (lane >> 4);
  u16x8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (n < N && k0 + e < K) ? B[n * ldb + k0 + e] : uint16_t(0);
  *reinterpret_cast<u16x8*>(out + i * 8) = v;
}

// A tiled B goes with calls of at most 64 rows that the few-row kernel takes (K a multiple
// of 8 with at least 32 whole 32-wide steps, which covers every configuration's 2 PF).
bool tiled_ok(int64_t M, int64_t K) { return M <= 64 && K % 8 == 0 && K / 32 >= 32; }

void launch_rows(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                 int64_t lda, int64_t ldb, int64_t ldc, int cf, hipStream_t s, KSplit sk = {}) {
  const RowsCfg c = rows_cfg(M, N, cf);
  if (c.pair) launch_rows_t<1, 1, 16, true>(A, B, C, M, N, K, lda, ldb, ldc, cf, 1, s, sk);
  else if (c.rb == 4) launch_rows_t<4, 2, 12>(A, B, C, M, N, K, lda, ldb, ldc, cf, 1, s, sk);
  else if (c.rb == 2) launch_rows_t<2, 2, 12>(A, B, C, M, N, K, lda, ldb, ldc, cf, c.split, s, sk);
  else if (c.split > 1) launch_rows_t<1, 2, 12>(A, B, C, M, N, K, lda, ldb, ldc, cf, c.split, s, sk);
  else if (c.cb == 2) launch_rows_t<1, 2, 16>(A, B, C, M, N, K, lda, ldb, ldc, cf, 1, s, sk);
  else launch_rows_t<1, 1, 16>(A, B, C, M, N, K, lda, ldb, ldc, cf, 1, s, sk);
}

template <class T>
void launch_dma(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K, int64_t lda,
                int64_t ldb, int64_t ldc, int cf, hipStream_t s, KSplit sk = {}) {
  const int tm = static_cast<int>((M + T::TM - 1) / T::TM), tn = static_cast<int>((N + T::TN - 1) / T::TN);
  gemm_dma_kernel<T><<<dim3(static_cast<unsigned>(static_cast<int64_t>(tm) * tn), sk.ks), dim3(T::THREADS), 0, s>>>(
      static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(B), C, int(M), int(N), int(K),
      lda, ldb, ldc, cf, tm, tn, sk.k_split ? sk.k_split : int(K), sk.stride);
}

// Fixed-order sum of K-slice partials: slice 0 + slice 1 + .. from +0 (the split-K comparison
// variant and the batch-invariant fixed split).
__global__ void splitk_reduce_kernel(const float* __restrict__ ws, void* __restrict__ C, int M,
                                     int N, int64_t ldc, int c_f32, int splits) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<int64_t>(M) * N) return;
  const int row = static_cast<int>(idx / N), col = static_cast<int>(idx % N);
  float s = 0.f;
  for (int k = 0; k < splits; ++k) s = s + ws[static_cast<int64_t>(k) * M * N + idx];
  if (c_f32) static_cast<float*>(C)[row * ldc + col] = s;
  else static_cast<uint16_t*>(C)[row * ldc + col] = f32_to_bf16(s);
}

// Comparison variant: slices of K chosen from the size of the output grid -- when the grid
// has fewer waves (few-row kernel) or tiles (LDS-staged tiles) than there are CUs, as many
// slices as fill the CUs (at most 16; none when the grid already fills them), each slice a
// whole number of 64-wide stages (at least 1024 columns for the few-row kernel, whose
// prefetch needs 32 steps).  So the number of slices, and with it every row's association of
// partial sums, changes with M.
KSplit splitk_plan(int64_t M, int64_t N, int64_t K) {
  const int64_t cus = cu_count();
  KSplit p;
  int64_t units, min_slice;
  if (use_rows(M, N, K, kOutF32)) {
    const RowsCfg c = rows_cfg(M, N, kOutF32);
    units = ((N + 16 * c.cb - 1) / (16 * c.cb)) * c.split;
    min_slice = 1024;
  } else {
    switch (pick_tile(M, N, cus)) {
      case TileKind::k256: units = ((M + 255) / 256) * ((N + 255) / 256); break;
      case TileKind::k64x128: units = ((M + 63) / 64) * ((N + 127) / 128); break;
      case TileKind::k64: units = ((M + 63) / 64) * ((N + 63) / 64); break;
      default: units = ((M + 127) / 128) * ((N + 127) / 128); break;
    }
    min_slice = 256;
  }
  int64_t ks = cus / std::max<int64_t>(units, 1);
  ks = std::min<int64_t>(ks, 16);
  ks = std::min<int64_t>(ks, std::max<int64_t>(1, K / min_slice));
  for (; ks > 1; --ks) {   // slices of whole stages, the last one at least min_slice long
    const int64_t per = ((K + ks - 1) / ks + 63) / 64 * 64;
    const int64_t n = (K + per - 1) / per;
    if (n > 1 && K - (n - 1) * per >= min_slice) {
      p.ks = static_cast<int>(n);
      p.k_split = static_cast<int>(per);
      p.stride = M * N * static_cast<int64_t>(sizeof(float));
      return p;
    }
  }
  return p;
}

// bf16 A and B, both under 4 GiB: the few-row kernel or the LDS-staged tiles by grid size.
void launch_bf16(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                 int64_t lda, int64_t ldb, int64_t ldc, int mode, hipStream_t s, KSplit sk = {}) {
  // the few-row kernel's prefetch depth must fit the shortest K slice (the last one)
  const int64_t k_short = sk.ks > 1 ? K - (sk.ks - 1) * static_cast<int64_t>(sk.k_split) : K;
  if (use_rows(M, N, k_short, mode)) {
    launch_rows(A, B, C, M, N, K, lda, ldb, ldc, mode, s, sk);
    return;
  }
  switch (pick_tile(M, N, cu_count())) {
    case TileKind::k256: launch_dma<Tile256>(A, B, C, M, N, K, lda, ldb, ldc, mode, s, sk); break;
    case TileKind::k128deep: launch_dma<Tile128Deep>(A, B, C, M, N, K, lda, ldb, ldc, mode, s, sk); break;
    case TileKind::k64x128: launch_dma<Tile64x128>(A, B, C, M, N, K, lda, ldb, ldc, mode, s, sk); break;
    case TileKind::k64: launch_dma<Tile64>(A, B, C, M, N, K, lda, ldb, ldc, mode, s, sk); break;
    default: launch_dma<Tile128>(A, B, C, M, N, K, lda, ldb, ldc, mode, s, sk); break;
  }
}


// bf16 A and [K, N] B, both under 4 GiB: the LDS-staged tiles with B landed as k rows and
// read transposed (the 256 x 256 tile, whose operands are read in place, is replaced by
// 128 x 128; the few-row kernel, which loads its operands straight into registers, has no
// [K, N] form).
void launch_bf16_kn(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                    int64_t lda, int64_t ldb, int64_t ldc, int mode, hipStream_t s) {
  switch (pick_tile(M, N, cu_count())) {
    case TileKind::k128deep: launch_dma<KnTile<Tile128Deep>>(A, B, C, M, N, K, lda, ldb, ldc, mode, s); break;
    case TileKind::k64x128: launch_dma<KnTile<Tile64x128>>(A, B, C, M, N, K, lda, ldb, ldc, mode, s); break;
    case TileKind::k64: launch_dma<KnTile<Tile64>>(A, B, C, M, N, K, lda, ldb, ldc, mode, s); break;
    default: launch_dma<KnTile<Tile128>>(A, B, C, M, N, K, lda, ldb, ldc, mode, s); break;
  }
}

}  // namespace
}  // namespace bi

using namespace bi;


extern "C" int bi_gemm(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                       int64_t lda, int64_t ldb, int64_t ldc, int b_layout, int a_dtype,
                       int c_dtype, void* stream) {
  if ((a_dtype != BI_BF16 && a_dtype != BI_F32) || (c_dtype != BI_BF16 && c_dtype != BI_F32) ||
      (b_layout != BI_B_NK && b_layout != BI_B_KN && b_layout != BI_B_TILED))
    return BI_ERR_DTYPE;
  if (M < 0 || N < 0 || K < 0) return BI_ERR_SHAPE;
  if (M == 0 || N == 0) return BI_OK;
  if (K < 1 || lda < K || ldc < N || M > (1 << 30) || N > (1 << 30) || K > (1 << 30))
    return BI_ERR_SHAPE;
  if (b_layout == BI_B_TILED) {   // ldb unused: the tiles are contiguous
    if (a_dtype != BI_BF16 || !tiled_ok(M, K)) return BI_ERR_UNSUPPORTED;
    if (!A || !B || !C) return BI_ERR_NULL;
    if (!aligned16(A) || !aligned16(B) || (lda % 8)) return BI_ERR_ALIGN;
    if (M * lda * 2 >= (int64_t(1) << 32)) return BI_ERR_UNSUPPORTED;
    launch_rows_tiled(A, B, C, M, N, K, lda, ldc, c_dtype == BI_F32, as_stream(stream));
    return launch_status();
  }
  if (b_layout == BI_B_NK ? ldb < K : ldb < N) return BI_ERR_SHAPE;
  if (!A || !B || !C) return BI_ERR_NULL;
  if (!aligned16(A) || !aligned16(B) || (lda % (a_dtype == BI_F32 ? 4 : 8)) || (ldb % 8))
    return BI_ERR_ALIGN;
  const int tm = static_cast<int>((M + BM - 1) / BM), tn = static_cast<int>((N + BN - 1) / BN);
  const int64_t nwg = static_cast<int64_t>(tm) * tn;
  if (nwg > 0x7fffffffLL) return BI_ERR_SHAPE;
  hipStream_t s = as_stream(stream);
  const int cf = c_dtype == BI_F32;
  if (b_layout == BI_B_KN && a_dtype == BI_BF16 && M * lda * 2 < (int64_t(1) << 32) &&
      K * ldb * 2 < (int64_t(1) << 32)) {
    launch_bf16_kn(A, B, C, M, N, K, lda, ldb, ldc, cf, s);
  } else if (b_layout == BI_B_KN) {   // fp32 A or 4 GiB operands: register-staged, transposed into LDS
    if (a_dtype == BI_F32)
      gemm_kernel<true, true><<<dim3(static_cast<unsigned>(nwg), 1), dim3(kThreads), 0, s>>>(
          A, static_cast<const uint16_t*>(B), C, int(M), int(N), int(K), lda, ldb, ldc, cf, tm, tn,
          0, int(K), 0);
    else
      gemm_kernel<false, true><<<dim3(static_cast<unsigned>(nwg), 1), dim3(kThreads), 0, s>>>(
          A, static_cast<const uint16_t*>(B), C, int(M), int(N), int(K), lda, ldb, ldc, cf, tm, tn,
          0, int(K), 0);
  } else if (a_dtype == BI_F32)
    gemm_kernel<true><<<dim3(static_cast<unsigned>(nwg), 1), dim3(kThreads), 0, s>>>(
        A, static_cast<const uint16_t*>(B), C, int(M), int(N), int(K), lda, ldb, ldc, cf, tm, tn,
        0, int(K), 0);
  else if (M * lda * 2 < (int64_t(1) << 32) && N * ldb * 2 < (int64_t(1) << 32))
    launch_bf16(A, B, C, M, N, K, lda, ldb, ldc, cf, s);
  else  // operands of 4 GiB or more: register-staged kernel (same tile, instruction, K order)
    gemm_kernel<false><<<dim3(static_cast<unsigned>(nwg), 1), dim3(kThreads), 0, s>>>(
        A, static_cast<const uint16_t*>(B), C, int(M), int(N), int(K), lda, ldb, ldc, cf, tm, tn,
        0, int(K), 0);
  return launch_status();
}

extern "C" int bi_gemm_tile(int64_t M, int64_t N, int64_t K, int a_dtype, int32_t* tile_m,
                            int32_t* tile_n, int32_t* stages) {
  if (!tile_m || !tile_n || !stages) return BI_ERR_NULL;
  if (M < 0 || N < 0 || K < 0) return BI_ERR_SHAPE;
  if (a_dtype != BI_BF16 && a_dtype != BI_F32) return BI_ERR_DTYPE;
  if (a_dtype == BI_F32 || M == 0 || N == 0) {  // register-staged kernel (or nothing to do)
    *tile_m = BM;
    *tile_n = BN;
    *stages = 2;
    return BI_OK;
  }
  if (use_rows(M, N, K, kOutBF16)) {   // few-row kernel: one wave per 16 x 16 .. 32 x 32 block
    const RowsCfg c = rows_cfg(M, N, kOutBF16);
    *tile_m = 16 * c.rb;
    *tile_n = 16 * c.cb;
    *stages = c.pf;
    return BI_OK;
  }
  switch (pick_tile(M, N, cu_count())) {
    case TileKind::k256: *tile_m = Tile256::TM; *tile_n = Tile256::TN; *stages = Tile256::STAGES; break;
    case TileKind::k128deep:
      *tile_m = Tile128Deep::TM; *tile_n = Tile128Deep::TN; *stages = Tile128Deep::STAGES; break;
    case TileKind::k64x128:
      *tile_m = Tile64x128::TM; *tile_n = Tile64x128::TN; *stages = Tile64x128::STAGES; break;
    case TileKind::k64: *tile_m = Tile64::TM; *tile_n = Tile64::TN; *stages = Tile64::STAGES; break;
    default: *tile_m = Tile128::TM; *tile_n = Tile128::TN; *stages = Tile128::STAGES; break;
  }
  return BI_OK;
}

extern "C" size_t bi_gemm_splitk_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0 || M > (1 << 30) || N > (1 << 30) || K > (1 << 30)) return 0;
  if (use_wsplit(M, N, K)) return 0;   // split over the waves of a workgroup
  const KSplit p = splitk_plan(M, N, K);
  return p.ks > 1 ? static_cast<size_t>(p.ks) * M * N * sizeof(float) : 0;
}

extern "C" int bi_gemm_splitk(const void* A, const void* B, void* C, int64_t M, int64_t N,
                              int64_t K, int64_t lda, int64_t ldb, int64_t ldc, int c_dtype,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (c_dtype != BI_BF16 && c_dtype != BI_F32) return BI_ERR_DTYPE;
  if (M < 0 || N < 0 || K < 0) return BI_ERR_SHAPE;
  if (M == 0 || N == 0) return BI_OK;
  if (K < 1 || lda < K || ldb < K || ldc < N || M > (1 << 30) || N > (1 << 30) || K > (1 << 30))
    return BI_ERR_SHAPE;
  if (!A || !B || !C) return BI_ERR_NULL;
  if (!aligned16(A) || !aligned16(B) || (lda % 8) || (ldb % 8)) return BI_ERR_ALIGN;
  if (!(M * lda * 2 < (int64_t(1) << 32) && N * ldb * 2 < (int64_t(1) << 32))) return BI_ERR_UNSUPPORTED;
  hipStream_t s = as_stream(stream);
  const int cf = c_dtype == BI_F32;
  if (use_wsplit(M, N, K)) {   // up to 4 rows: K split over the 4 waves of a workgroup
    launch_wsplit(A, B, C, M, N, K, lda, ldb, ldc, cf, s);
    return launch_status();
  }
  const KSplit p = splitk_plan(M, N, K);
  if (p.ks == 1) {   // one slice: the plain kernels write C
    launch_bf16(A, B, C, M, N, K, lda, ldb, ldc, cf, s);
    return launch_status();
  }
  if (!workspace || workspace_bytes < bi_gemm_splitk_workspace_bytes(M, N, K)) return BI_ERR_WORKSPACE;
  // the few-row or LDS-staged kernels, each slice's fp32 result into the workspace, then the
  // slices added in ascending order
  launch_bf16(A, B, workspace, M, N, K, lda, ldb, N, kOutF32, s, p);
  const int64_t total = M * N;
  splitk_reduce_kernel<<<dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, s>>>(
      static_cast<const float*>(workspace), C, int(M), int(N), ldc, cf, p.ks);
  return launch_status();
}

namespace bi {
namespace {
// Slices of a batch-invariant split: k_slice columns each at absolute offsets 0, k_slice, ..
// (the last one shorter when k_slice does not divide K), a function of K and k_slice alone.
int64_t fixed_slices(int64_t K, int64_t k_slice) { return (K + k_slice - 1) / k_slice; }
}  // namespace
}  // namespace bi

extern "C" size_t bi_gemm_fixed_split_workspace_bytes(int64_t M, int64_t N, int64_t K,
                                                      int64_t k_slice) {
  if (M <= 0 || N <= 0 || K <= 0 || M > (1 << 30) || N > (1 << 30) || K > (1 << 30) ||
      k_slice < 64 || k_slice % 64 != 0)
    return 0;
  const int64_t ks = fixed_slices(K, k_slice);
  return ks > 1 ? static_cast<size_t>(ks) * M * N * sizeof(float) : 0;
}

extern "C" int bi_gemm_fixed_split(const void* A, const void* B, void* C, int64_t M, int64_t N,
                                   int64_t K, int64_t lda, int64_t ldb, int64_t ldc, int c_dtype,
                                   int64_t k_slice, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  if (c_dtype != BI_BF16 && c_dtype != BI_F32) return BI_ERR_DTYPE;
  if (M < 0 || N < 0 || K < 0) return BI_ERR_SHAPE;
  if (M == 0 || N == 0) return BI_OK;
  if (K < 1 || lda < K || ldb < K || ldc < N || M > (1 << 30) || N > (1 << 30) || K > (1 << 30) ||
      k_slice < 64 || k_slice % 64 != 0)
    return BI_ERR_SHAPE;
  if (!A || !B || !C) return BI_ERR_NULL;
  if (!aligned16(A) || !aligned16(B) || (lda % 8) || (ldb % 8)) return BI_ERR_ALIGN;
  if (!(M * lda * 2 < (int64_t(1) << 32) && N * ldb * 2 < (int64_t(1) << 32))) return BI_ERR_UNSUPPORTED;
  const int64_t ks = fixed_slices(K, k_slice);
  if (ks > 65535) return BI_ERR_UNSUPPORTED;   // one grid row per slice
  hipStream_t s = as_stream(stream);
  const int cf = c_dtype == BI_F32;
  if (ks == 1) {   // one slice: bi_gemm itself
    launch_bf16(A, B, C, M, N, K, lda, ldb, ldc, cf, s);
    return launch_status();
  }
  if (!workspace || workspace_bytes < bi_gemm_fixed_split_workspace_bytes(M, N, K, k_slice))
    return BI_ERR_WORKSPACE;
  KSplit p;
  p.ks = static_cast<int>(ks);
  p.k_split = static_cast<int>(k_slice);
  p.stride = M * N * static_cast<int64_t>(sizeof(float));
  // each slice's fp32 chain (bi_gemm's instruction and order over the slice's columns) into
  // the workspace, then the slices added in ascending order from +0
  launch_bf16(A, B, workspace, M, N, K, lda, ldb, N, kOutF32, s, p);
  const int64_t total = M * N;
  splitk_reduce_kernel<<<dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, s>>>(
      static_cast<const float*>(workspace), C, int(M), int(N), ldc, cf, p.ks);
  return launch_status();
}

extern "C" int bi_gemm_swiglu(const void* A, const void* W, void* out, int64_t M, int64_t F, int64_t K,
                              int64_t lda, int64_t ldw, int64_t ldo, int w_layout, void* stream) {
  if (w_layout != BI_B_NK && w_layout != BI_B_TILED) return BI_ERR_DTYPE;
  if (M < 0 || F < 0 || K < 0) return BI_ERR_SHAPE;
  if (M == 0 || F == 0) return BI_OK;
  if (K < 1 || F % 16 != 0 || lda < K || ldo < F || M > (1 << 30) || F > (1 << 29) || K > (1 << 30) ||
      (w_layout == BI_B_NK && ldw < K))
    return BI_ERR_SHAPE;
  if (w_layout == BI_B_TILED) {   // the tiles of interleave(W); ldw unused
    if (!tiled_ok(M, K)) return BI_ERR_UNSUPPORTED;
    if (!A || !W || !out) return BI_ERR_NULL;
    if (!aligned16(A) || !aligned16(W) || (lda % 8)) return BI_ERR_ALIGN;
    if (M * lda * 2 >= (int64_t(1) << 32)) return BI_ERR_UNSUPPORTED;
    launch_rows_tiled(A, W, out, M, 2 * F, K, lda, ldo, kOutSwiGLU, as_stream(stream));
    return launch_status();
  }
  if (!A || !W || !out) return BI_ERR_NULL;
  if (!aligned16(A) || !aligned16(W) || (lda % 8) || (ldw % 8)) return BI_ERR_ALIGN;
  const int64_t N = 2 * F;
  if (!(M * lda * 2 < (int64_t(1) << 32) && N * ldw * 2 < (int64_t(1) << 32))) return BI_ERR_UNSUPPORTED;
  launch_bf16(A, W, out, M, N, K, lda, ldw, ldo, kOutSwiGLU, as_stream(stream));
  return launch_status();
}

namespace {
// Checks shared by the two fused add + RMSNorm + GEMM calls (N = output columns of the
// product: 2F for SwiGLU).
int norm_gemm_check(const void* a, const void* b, const void* sum, const void* gamma, const void* W,
                    const void* C, int64_t M, int64_t N, int64_t K, int64_t ldw, int64_t ldc,
                    int64_t ldc_min, int w_layout) {
  if (w_layout != BI_B_NK && w_layout != BI_B_TILED) return BI_ERR_DTYPE;
  if (M < 0 || N < 0 || K < 1 || ldc < ldc_min || (w_layout == BI_B_NK && ldw < K) ||
      N > (1 << 30) || K > (1 << 30))
    return BI_ERR_SHAPE;
  if (M == 0 || N == 0) return BI_OK;
  if (M > kNormRows || K % 8 != 0 || K > 4096 || K / 32 < 32) return BI_ERR_UNSUPPORTED;
  if (!a || !b || !sum || !gamma || !W || !C) return BI_ERR_NULL;
  if (!aligned16(a) || !aligned16(b) || !aligned16(sum) || !aligned16(gamma) || !aligned16(W) ||
      (w_layout == BI_B_NK && ldw % 8))
    return BI_ERR_ALIGN;
  // sum is written by one workgroup while the others still read a and b
  const char *pa = static_cast<const char*>(a), *pb = static_cast<const char*>(b),
             *ps = static_cast<const char*>(sum);
  const int64_t bytes = M * K * 2;
  if ((ps < pa + bytes && pa < ps + bytes) || (ps < pb + bytes && pb < ps + bytes)) return BI_ERR_SHAPE;
  if (w_layout == BI_B_NK && N * ldw * 2 >= (int64_t(1) << 32)) return BI_ERR_UNSUPPORTED;
  return 1;   // go ahead
}
}  // namespace

extern "C" int bi_add_rmsnorm_gemm(const void* a, const void* b, void* sum, const void* gamma, float eps,
                                   const void* W, void* C, int64_t M, int64_t N, int64_t K, int64_t ldw,
                                   int64_t ldc, int w_layout, int c_dtype, void* stream) {
  if (c_dtype != BI_BF16 && c_dtype != BI_F32) return BI_ERR_DTYPE;
  const int st = norm_gemm_check(a, b, sum, gamma, W, C, M, N, K, ldw, ldc, N, w_layout);
  if (st != 1) return st;
  const NormArgs na{static_cast<const uint16_t*>(b), static_cast<const uint16_t*>(gamma),
                    static_cast<uint16_t*>(sum), eps};
  launch_rows_norm(a, W, C, M, N, K, ldw, ldc, c_dtype == BI_F32, w_layout == BI_B_TILED, na,
                   as_stream(stream));
  return launch_status();
}

extern "C" int bi_add_rmsnorm_gemm_swiglu(const void* a, const void* b, void* sum, const void* gamma,
                                          float eps, const void* W, void* out, int64_t M, int64_t F,
                                          int64_t K, int64_t ldw, int64_t ldo, int w_layout,
                                          void* stream) {
  if (F < 0) return BI_ERR_SHAPE;
  if (F % 16 != 0 || F > (1 << 29)) return BI_ERR_SHAPE;
  const int st = norm_gemm_check(a, b, sum, gamma, W, out, M, 2 * F, K, ldw, ldo, F, w_layout);
  if (st != 1) return st;
  const NormArgs na{static_cast<const uint16_t*>(b), static_cast<const uint16_t*>(gamma),
                    static_cast<uint16_t*>(sum), eps};
  launch_rows_norm(a, W, out, M, 2 * F, K, ldw, ldo, kOutSwiGLU, w_layout == BI_B_TILED, na,
                   as_stream(stream));
  return launch_status();
}

extern "C" size_t bi_pack_b_bytes(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0 || N > (1 << 30) || K > (1 << 30)) return 0;
  return static_cast<size_t>((N + 15) / 16) * static_cast<size_t>((K + 31) / 32) * 1024;
}

extern "C" int bi_pack_b(const void* B, int64_t N, int64_t K, int64_t ldb, void* out, void* stream) {
  if (N < 0 || K < 0) return BI_ERR_SHAPE;
  if (N == 0 || K == 0) return BI_OK;
  if (ldb < K || N > (1 << 30) || K > (1 << 30)) return BI_ERR_SHAPE;
  if (!B || !out) return BI_ERR_NULL;
  if (!aligned16(out)) return BI_ERR_ALIGN;
  const int64_t nk32 = (K + 31) / 32;
  const int64_t pieces = (N + 15) / 16 * nk32 * 64;
  if ((pieces + 255) / 256 > 0x7fffffffLL) return BI_ERR_SHAPE;
  pack_b_kernel<<<dim3(static_cast<unsigned>((pieces + 255) / 256)), dim3(256), 0, as_stream(stream)>>>(
      static_cast<const uint16_t*>(B), N, K, ldb, static_cast<uint16_t*>(out), nk32, pieces);
  return launch_status();
}
