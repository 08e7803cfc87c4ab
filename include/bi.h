/*
 * bi.h -- batch-invariant, run-to-run deterministic reductions of an LLM forward
 * pass on AMD Instinct MI355X (gfx950).  C ABI.
 *
 * Sources (web pages; cited by title and section):
 *   [DN]  "Defeating nondeterminism in LLM inference" (Chinese translation):
 *         sections on floating-point non-associativity, atomic adds, batch
 *         invariance, batch-invariant RMSNorm, matrix multiplication and attention.
 *   [GPU] "Does the same LLM give different outputs on different GPUs? Why?":
 *         sections on the experiment set-up (greedy decoding, token probabilities).
 *   [XV]  arXiv abstract "cross-vendor mismatch of language models" (FP32 upcast,
 *         MLPs kept in BF16).
 *   [SM]  "Same model, same input, different answer": section on sampling (near-tie
 *         argmax flips).
 *   [VER] "How to verify GPU program correctness before deployment": sections on
 *         validation data (bad shapes, illegal types) and error thresholds.
 *
 * The contract every entry point keeps ([DN], batch invariance): identical input
 * bytes give identical output bits for every batch size M, every position of a row
 * in the batch, every set of co-batched rows, every stream and every call history.
 * No entry point uses atomics ([DN], atomic adds), no reduction order depends on M.
 *
 * Conventions shared by every call
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library never
 *     allocates or frees device memory.  Its only process-wide state is read-only
 *     after first use: the compute-unit count of each device and the number of
 *     attention workgroups resident per CU, each queried from the HIP runtime on first
 *     use and cached in an atomic (a race stores the same value twice).  They choose
 *     launch shapes only, never a reduction order.  Calls may be issued from several
 *     threads.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls enqueue work on it
 *     and return without waiting.
 *   - Arguments are validated before anything is launched.  On a validation error
 *     the call returns a negative bi_status and writes nothing.  A failed launch
 *     returns BI_ERR_HIP.  No exception or abort crosses the ABI.
 *   - Outputs must not alias inputs unless a call says otherwise.
 *   - bf16 is IEEE binary32's upper 16 bits; every rounding to bf16 is
 *     round-to-nearest-even (a NaN stays a quiet NaN).  fp32 denormals are kept.
 *   - A dimension of 0 is valid and launches nothing (returns BI_OK).
 */
#ifndef BI_H_
#define BI_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BI_OK = 0,
  BI_ERR_NULL = -1,        /* a required pointer is NULL                              */
  BI_ERR_SHAPE = -2,       /* a size or leading dimension is negative or inconsistent  */
  BI_ERR_DTYPE = -3,       /* unknown dtype / layout code                              */
  BI_ERR_ALIGN = -4,       /* pointer or leading dimension breaks the stated alignment */
  BI_ERR_WORKSPACE = -5,   /* workspace missing or smaller than required               */
  BI_ERR_UNSUPPORTED = -6, /* a valid request this build does not implement            */
  BI_ERR_HIP = -7          /* the HIP runtime reported an error at launch              */
} bi_status;

enum { BI_BF16 = 1, BI_F32 = 2 };
enum { BI_B_KN = 0, BI_B_NK = 1, BI_B_TILED = 2 };

/* Compile-time constants of the reduction strategy.  They never vary at run time,
 * because a run-time choice would be a way to break invariance. */
typedef struct bi_config {
  int32_t version;          /* layout of this struct                                   */
  int32_t tree_max_lanes;   /* 256: lanes of the RMSNorm / log-softmax tree            */
  int32_t wave_size;        /* 64                                                      */
  int32_t gemm_tile_m;      /* output tile rows per workgroup (small tile)             */
  int32_t gemm_tile_n;      /* output tile columns per workgroup (small tile)          */
  int32_t gemm_tile_k;      /* K depth of one LDS stage of the main kernel             */
  int32_t gemm_mfma_m, gemm_mfma_n, gemm_mfma_k; /* the one matrix instruction shape     */
  int32_t attn_chunk;       /* 256: split-KV chunk, at absolute positions 256c          */
  int32_t attn_max_group;   /* largest supported q heads per kv head                   */
  int32_t gemm_big_tile_m;  /* rows of the large workgroup tile (same bits, see bi_gemm) */
  int32_t gemm_big_tile_n;  /* columns of the large workgroup tile                     */
  int32_t attn_merge_group; /* 4: chunk partials merge within groups of 4 chunks, then the
                               groups, in ascending order (version >= 3)                 */
} bi_config;

/* Fills *out.  Returns BI_ERR_NULL if out is NULL. */
int bi_get_config(bi_config* out);

/* Static text for a status code ("BI_OK", "BI_ERR_SHAPE", ...). */
const char* bi_status_string(int status);

/* ------------------------------------------------------------------ RMSNorm
 * [DN] batch-invariant RMSNorm: y = x * rsqrt(mean(x^2)) * weight, one row per
 * workgroup, reduction order fixed per row whatever M is.  Readings: eps inside the
 * square root; rsqrt is a correctly rounded sqrt followed by a correctly rounded
 * divide; y = bf16((x * r) * gamma) multiplied in that order.
 *
 *   x      [M, D] row-major, row stride ldx elements, dtype x_dtype (BI_BF16|BI_F32)
 *   gamma  [D] bf16
 *   y      [M, D] row stride ldy, dtype y_dtype (BI_BF16|BI_F32)
 *   eps    added to mean(x^2) in fp32
 * Sum of squares: fixed fp32 tree, a function of D only:
 *   T = min(256, ceil(D / w)) lanes (w = 8 for bf16 x, 4 for fp32 x); lane t owns the
 *   w-element vectors t, t+T, ...; each lane adds its squares in ascending order
 *   starting from +0; a wave64 butterfly with offsets 1,2,4,8,16,32; waves combined
 *   as (w0 + w1) + (w2 + w3).  No fused multiply-add anywhere.
 * Errors: NULL pointers (when M*D > 0) -> BI_ERR_NULL; M < 0, D < 1 with M > 0,
 * ldx < D or ldy < D -> BI_ERR_SHAPE; bad dtype -> BI_ERR_DTYPE.
 */
int bi_rmsnorm(const void* x, const void* gamma, void* y, int64_t M, int64_t D, int64_t ldx,
               int64_t ldy, float eps, int x_dtype, int y_dtype, void* stream);

/* ------------------------------------------------------------------ GEMM
 * [DN] introduction (torch.mm of bf16 matrices) and batch-invariant matrix
 * multiplication: data-parallel over output tiles, every dot product inside one
 * workgroup, ONE kernel configuration for every shape, no split-K, no stream-K.
 *
 *   C[M, N] = A[M, K] . op(B)   fp32 accumulation
 *   A     dtype a_dtype: BI_BF16, or BI_F32 (each fp32 value is split exactly into
 *         three bf16 terms hi + mid + lo and the three products are accumulated in the
 *         same fp32 accumulator: fp32-operand products at three times the work, the
 *         upcast of [XV]); row stride lda
 *   B     bf16; b_layout BI_B_NK: B is [N, K] (a Linear weight, C = A . B^T), row
 *         stride ldb;  BI_B_KN: B is [K, N] (torch.mm orientation), row stride ldb;
 *         BI_B_TILED: an [N, K] B as bi_pack_b wrote it (ldb unused), for calls of at most
 *         64 rows with K a multiple of 8 and at least 1024 (the few-row kernel's calls;
 *         other calls return BI_ERR_UNSUPPORTED) -- the same bits as BI_B_NK.  Above 32
 *         rows with more 32-column blocks than the device has CUs the [N, K] call, which
 *         takes the LDS-staged tiles there, is the faster one
 *   C     dtype c_dtype (BI_BF16: one RNE rounding of the fp32 sum; BI_F32), stride ldc
 * Every output element is produced by the same sequence of matrix instructions
 * (v_mfma_f32_16x16x32_bf16, one fp32 accumulator from +0, K in ascending 32-wide steps,
 * the k offsets of a step assigned to the instruction's lanes the same way every time)
 * whatever M is, wherever its row sits and whichever workgroup tile computes it; the
 * workgroup tile (bi_gemm_tile) follows the size of the output grid and changes no bit.
 * Alignment: A and B 16-byte aligned; lda, ldb multiples of 8 elements (4 for fp32 A).
 * Rows are read in 16-byte pieces: row i of A (of a [N, K] B) must be readable up to
 * element round_up(K, 8) (round_up(K, 4) for fp32 A), which lda (ldb) >= that guarantees
 * for every row but the last.
 * BI_B_KN with bf16 A (operands under 4 GiB) runs the LDS-staged tiles below, B landing in
 * on-chip memory as k rows and each instruction's B operand read with two transposing LDS
 * reads; the few-row grids and the 256 x 256 tile are replaced by the tile the grid would
 * otherwise take (64 x 64 .. 128 x 128).  With fp32 A (or 4 GiB operands) a register-staged
 * 128 x 128 tile transposes each 4 x 8 block of B on its way into on-chip memory.  Either
 * way every output element sees the same operands, lanes and instruction sequence as with
 * the [N, K] copy of B, so C is bit for bit the BI_B_NK result.  A [K, N] B is read only
 * inside its N columns (a 16-byte piece that starts inside reads up to the next multiple of
 * 8 columns, within ldb) and its K rows.
 * Errors: BI_ERR_NULL, BI_ERR_SHAPE (negative sizes, K < 1 with M*N > 0, strides too
 * small), BI_ERR_DTYPE, BI_ERR_ALIGN.
 */
int bi_gemm(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K, int64_t lda,
            int64_t ldb, int64_t ldc, int b_layout, int a_dtype, int c_dtype, void* stream);

/* The workgroup tile bi_gemm uses for an M x N x K product with A of dtype a_dtype on the
 * current device: *tile_m x *tile_n outputs per workgroup and *stages K slices in flight.
 * Up to 32 rows (up to 64 while ceil(N / 32) is at most the CU count), with K a multiple of
 * 8 and at least 2 x (16 or 12) whole 32-wide steps: one wave per output block with its
 * instruction operands loaded straight into registers 16 (or 12) K steps ahead; the block
 * is 16 x 16 up to 16 rows (16 x 32 from 9 rows when N / 16 is at least four times the CU
 * count), 32 x 32 up to 32 rows, 64 x 32 above (or, while N / 32 is under three quarters of
 * the CU count, two waves of 32 x 32 per column block, one per 32-row half); 16 x 32 in two
 * (up to 32 rows) or four (above) waves per column block, one per 16-row slice, while those
 * waves number at most the CU count.
 * Otherwise 256 x 256
 * (2-stage LDS ring) when that grid finishes in fewer rounds of the CU array; else
 * 128 x 128, with a 3-stage ring when the grid has no more tiles than CUs and a 2-stage
 * ring (two workgroups per CU) otherwise; when fewer than three quarters of the CUs would
 * get a 128 x 128 tile, 64 x 128 or (fewer still) 64 x 64 with a 3-stage ring; fp32 A:
 * 128 x 128, register staged.  (For a [K, N] B bi_gemm takes the same choice among the
 * LDS-staged tiles without the few-row and 256 x 256 forms; this call reports the [N, K]
 * choice.)
 * Informational: the bits of C do not depend on it.  Errors: BI_ERR_NULL, BI_ERR_SHAPE
 * (negative sizes), BI_ERR_DTYPE. */
int bi_gemm_tile(int64_t M, int64_t N, int64_t K, int a_dtype, int32_t* tile_m, int32_t* tile_n,
                 int32_t* stages);

/* Comparison variant, NOT batch-invariant ([DN], split-K matmul): same arguments as
 * bi_gemm with bf16 A and B_NK, on the same kernels, but K is split into slices whose number
 * grows as M shrinks (so that small batches fill the GPU): up to 4 rows (K in 512 .. 4096),
 * over the 4 waves of a workgroup, whose partials are added in LDS; otherwise, when the
 * output grid has fewer waves or tiles than there are CUs, into as many slices (up to 16) as
 * fill the CUs, each slice's fp32 partial in `workspace`, then added in ascending order by a
 * second kernel (no split when the grid already fills the CUs).  The association of a row's
 * sums therefore depends on M.
 * workspace >= bi_gemm_splitk_workspace_bytes(M, N, K) bytes (0 when none is used). */
size_t bi_gemm_splitk_workspace_bytes(int64_t M, int64_t N, int64_t K);
int bi_gemm_splitk(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                   int64_t lda, int64_t ldb, int64_t ldc, int c_dtype, void* workspace,
                   size_t workspace_bytes, void* stream);

/* Batch-invariant split of K ([DN], batch-invariant RMSNorm, last paragraph: a reduction
 * strategy with enough parallelism for tiny batches stays batch-invariant when it is used
 * for every batch size; [DN], batch-invariant matmul: split-K for small M and N).  Same
 * arguments as bi_gemm with bf16 A and B_NK, plus k_slice: K is cut into slices of k_slice
 * columns at absolute offsets 0, k_slice, 2 k_slice, .. (the last one shorter when k_slice
 * does not divide K), a function of K and k_slice alone, never of M.  Each slice's partial is
 * bi_gemm's fp32 chain over the slice's columns (same instruction and ascending order, from
 * +0), written to `workspace`; a second kernel adds the slices in ascending order from +0
 * and rounds once to c_dtype.  For a fixed k_slice the bits of a row therefore do not depend
 * on M or on the row's place in the batch (they differ from bi_gemm's when K > k_slice; with
 * K <= k_slice the call is bi_gemm).  k_slice: a multiple of 64, at least 64 (BI_ERR_SHAPE
 * otherwise); at most 65535 slices (BI_ERR_UNSUPPORTED).
 * workspace >= bi_gemm_fixed_split_workspace_bytes(M, N, K, k_slice) = slices x M x N x 4
 * bytes (0 with one slice), caller-owned, on the device (BI_ERR_WORKSPACE if smaller);
 * the function returns 0 for invalid sizes. */
size_t bi_gemm_fixed_split_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t k_slice);
int bi_gemm_fixed_split(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                        int64_t lda, int64_t ldb, int64_t ldc, int c_dtype, int64_t k_slice,
                        void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------ attention
 * [DN] batch-invariant attention: the K/V cache and page table are updated BEFORE
 * the attention kernel runs, so that a query token reduces over the same keys in the
 * same order whether it arrives in a prefill (0 cached tokens) or a decode (p cached
 * tokens); a consistent block size; split-KV (FlashDecoding) for decode.  The split
 * is one fixed chunk of 256 keys at absolute positions [256c, 256c + 256) that never
 * depends on the batch or on the number of query tokens.
 *
 * Batch: `batch` sequences; sequence b has seq_lens[b] tokens after this call, of which
 * the last q_b = query_start_loc[b+1] - query_start_loc[b] are new (0 <= q_b <=
 * seq_lens[b]).  New token i of sequence b (row query_start_loc[b] + i of q/k_new/v_new/
 * out) sits at absolute position p = seq_lens[b] - q_b + i.
 *   q        [num_tokens, Hq, D], contiguous, dtype q_dtype: BI_BF16, or BI_F32 (the FP32 upcast
 *            of [XV]: each value split exactly into bf16 hi + mid + lo, the three products
 *            accumulated in that order in every 32-wide step of the score's d-sum, so the
 *            scores see q at full fp32 precision; keys stay the cache's bf16)
 *   k_new    [num_tokens, Hkv, D] bf16 (keys already rotated), contiguous
 *   v_new    [num_tokens, Hkv, D] bf16, contiguous
 *            k_new = v_new = NULL: the call's new keys and values are in their pages
 *            already (written by bi_rope_kv_write); step 1 is skipped
 *   k_cache  [num_pages, Hkv, D/8, page_size, 8] bf16: per page and kv head, D is cut
 *            into 8-element groups; group j holds d = 8j..8j+7 of every slot.  Inside each
 *            aligned block of 16 slots the slot order is permuted by swapping bits 2 and 3
 *            of the slot index (0-3, 8-11, 4-7, 12-15), so that the 8 keys one matrix
 *            instruction reads from a page are adjacent (whole 128-byte lines per load)
 *   v_cache  [num_pages, Hkv, D, page_size] bf16: each page stores V transposed (slot
 *            fastest, natural slot order), the operand order of the P.V product
 *   block_table [batch, max_pages_per_seq] int32: physical page of logical page j
 *            (entries at j >= ceil(seq_lens[b] / page_size) may be read, their values
 *            are never used)
 *   seq_lens [batch] int32, query_start_loc [batch + 1] int32 (device)
 *   out      [num_tokens, Hq, D], dtype out_dtype (BI_BF16 | BI_F32)
 *   scale    softmax scale (1/sqrt(D) for the standard reading)
 * Step 1 writes k_new/v_new into their pages (unless both are NULL).  Step 2: token at
 * position p of q head
 * h (kv head h / (Hq/Hkv)) computes, for each chunk c <= p/256, the partial
 * (m_c, l_c, o_c) over keys [256c, min(256c + 256, p + 1)) with fp32 scores, P kept
 * as an exact bf16 hi + lo pair, fp32 accumulation.  Step 3 merges in two fixed levels,
 * both set by absolute positions: the chunks of each group of 4 (keys [1024g,
 * 1024g + 1024)) in ascending c, then the groups in ascending g; each level copies its
 * first partial, then m' = max(m, m_c), a = 2^(m - m'), b = 2^(m_c - m'),
 * l' = a l + b l_c, o' = a o + b o_c;  out = o / l.  Decode-sized calls reduce the
 * groups in parallel and merge them in a second kernel, longer calls walk the chunks in
 * registers; both use the same arithmetic, so the bits never depend on which is used.
 * Supported: D = 128, Hq/Hkv in {1, 2, 4, 8, 16}, page_size a multiple of 16 dividing
 * 256.  max_seq_len is an upper bound of seq_lens (sizes the grid); every seq_len must
 * be <= max_pages_per_seq * page_size.
 * workspace >= bi_attention_workspace_bytes(num_tokens, Hq, D, max_seq_len): for calls
 * of at most 1024 tokens, room for fp32 partials (m, l and o) of every token, q head and
 * 256-key chunk (bi_attention fills a quarter of it, one per 4-chunk group; the
 * comparison variant below may use all of it) and a 16-byte record per token; 0 for
 * longer calls (no workspace is used).
 * Errors: BI_ERR_NULL (also when exactly one of k_new, v_new is NULL), BI_ERR_SHAPE (also
 * when num_tokens * ceil(max_seq_len / 256) * Hkv reaches 2^31 on the split path),
 * BI_ERR_UNSUPPORTED, BI_ERR_WORKSPACE, BI_ERR_ALIGN (16-byte alignment of every tensor).
 */
size_t bi_attention_workspace_bytes(int64_t num_tokens, int32_t num_q_heads, int32_t head_dim,
                                    int64_t max_seq_len);
int bi_attention(const void* q, int q_dtype, const void* k_new, const void* v_new, void* k_cache,
                 void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                 const int32_t* query_start_loc, int32_t batch, int64_t num_tokens,
                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                 int32_t max_pages_per_seq, int64_t max_seq_len, float scale, void* out,
                 int out_dtype, void* workspace, size_t workspace_bytes, void* stream);

/* bi_attention without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).  Same
 * arguments, layouts, validation and bits as bi_attention.  Its split-KV partials and token
 * records live in a 64 MiB scratch array that the library holds on every device it runs on
 * until the process ends (looked up on the first call on a device); the call allocates and
 * frees nothing.  A call needs, for at most 1024 tokens,
 *   4 * (R2 + R * D) + 16 * num_tokens bytes,  R = num_tokens * Hq * S, R2 = 2R rounded up to
 *   a multiple of 4, S = ceil(max_seq_len / 256) when num_tokens * ceil(max_seq_len / 1024) *
 *   Hkv is below twice the CU count, else ceil(max_seq_len / 1024)
 * (about 34 MB for 64 tokens of 32768-token contexts, 32 q heads); longer calls need none.
 * Every call on a device shares that device's scratch and overwrites it: calls that overlap in
 * time on one device (concurrent streams, several host threads) race and must be serialised by
 * the caller.  Nothing in the scratch has to start at zero.
 * Errors: as bi_attention; BI_ERR_WORKSPACE when the call needs more than the 64 MiB;
 * BI_ERR_HIP when the scratch's device address cannot be obtained. */
int bi_attention_noalloc(const void* q, int q_dtype, const void* k_new, const void* v_new, void* k_cache,
                         void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                         const int32_t* query_start_loc, int32_t batch, int64_t num_tokens,
                         int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t page_size, int32_t max_pages_per_seq, int64_t max_seq_len,
                         float scale, void* out, int out_dtype, void* stream);

/* Comparison variant, NOT batch-invariant (split-KV / FlashDecoding with a number of
 * splits chosen from the batch, as [DN] describes for decode kernels): same arguments and
 * layouts as bi_attention (at most 1024 tokens per call) plus total_chunks = sum over
 * tokens of (position / 256 + 1).  Each workgroup walks a group of consecutive 256-key
 * chunks, merging in registers; the group size is about total_chunks * Hkv / 1024, so the
 * association of a token's merges -- and its bits -- depends on the rest of the batch.
 * workspace >= bi_attention_workspace_bytes(num_tokens, Hq, D, max_seq_len). */
int bi_attention_batchdep_split(const void* q, int q_dtype, const void* k_new, const void* v_new,
                                void* k_cache, void* v_cache, const int32_t* block_table,
                                const int32_t* seq_lens, const int32_t* query_start_loc,
                                int32_t batch, int64_t num_tokens, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                                int32_t max_pages_per_seq, int64_t max_seq_len,
                                int64_t total_chunks, float scale, void* out, int out_dtype,
                                void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------ log-softmax + argmax
 * [GPU] greedy decoding and token probabilities from normalised scores; [DN]
 * temperature 0 = always the most likely token; [SM] near ties decide the token.
 * Per row of fp32 logits x: a = lowest index of the maximum (a NaN counts as the
 * maximum, -0 == +0); m = x[a]; d_i = x_i - m; s = tree sum of EXP(d_i) with the fixed
 * tree of bi_rmsnorm over 4-element vectors; logprob_i = d_i - LOG(s).  EXP is a
 * Cody-Waite reduction with the degree-7 Taylor polynomial, LOG the atanh series to
 * z^15, both with separately rounded fp32 operations, so the result is reproducible
 * bit for bit on any IEEE machine.
 *   logits   [M, V] fp32, row stride ld
 *   logprobs [M, V] fp32, row stride ld, or NULL to skip
 *   argmax   [M] int32
 * With logprobs NULL only the argmax is computed (the same index).
 * Errors: BI_ERR_NULL, BI_ERR_SHAPE (V < 1 with M > 0, ld < V, logprobs overlapping
 * logits).
 */
int bi_logsoftmax_argmax(const float* logits, int64_t M, int64_t V, int64_t ld, float* logprobs,
                         int32_t* argmax, void* stream);

/* ------------------------------------------------------------------ pointwise glue
 * [DN] section on making kernels batch-invariant: pointwise operations are invariant
 * as long as every element runs the same code.  All of these compute in fp32 and
 * round once to the output dtype.
 *
 * bi_embedding: out[t, :] = table[ids[t], :] (a row gather: the embedding lookup, and
 *   the pick of each sequence's last hidden row before the LM head).  table [vocab, D]
 *   of table_dtype, out [T, D] of out_dtype (exact when widening; one RNE rounding for
 *   fp32 -> bf16).  ids outside [0, vocab) produce zeros.
 */
int bi_embedding(const int32_t* ids, const void* table, int table_dtype, void* out, int64_t T,
                 int64_t D, int64_t vocab, int out_dtype, void* stream);

/* bi_rope_qkv: splits a fused projection qkv [T, (Hq + 2 Hkv) * D] (row stride ldqkv,
 *   dtype qkv_dtype) into q [T, Hq, D] (dtype q_dtype), k [T, Hkv, D], v [T, Hkv, D] (bf16,
 *   the type of the KV cache; all contiguous) and rotates q and k by position ("rotate half":
 *   pairs (i, i + D/2), angle pos * base^(-2i/D), angle, cos and sin evaluated in fp64 and
 *   rounded to fp32; the rotation in fp32, one rounding to the output type).
 *   positions [T] int32. */
int bi_rope_qkv(const void* qkv, int64_t ldqkv, int qkv_dtype, const int32_t* positions,
                void* q, int q_dtype, void* k, void* v, int64_t T, int32_t num_q_heads,
                int32_t num_kv_heads, int32_t head_dim, double base, void* stream);

/* bi_rope_kv_write: bi_rope_qkv fused with step 1 of bi_attention (the fused neighbours
 *   of "Defeating nondeterminism in LLM inference", section on making kernels
 *   batch-invariant: pointwise work riding on the cache write).  q [num_tokens, Hq, D]
 *   (dtype q_dtype) receives the rotated queries; the rotated keys and the values of qkv
 *   go straight into k_cache / v_cache at each new token's page slot, in the layouts of
 *   bi_attention, with no k or v tensor in between.  A token's rotation position is its
 *   cache position p = seq_lens[b] - q_b + i (the batch description of bi_attention).
 *   q, k_cache and v_cache then hold exactly the bits of bi_rope_qkv at those positions
 *   followed by bi_attention's step 1; call bi_attention with k_new = v_new = NULL next.
 *   qkv [num_tokens, (Hq + 2 Hkv) * D] (row stride ldqkv, qkv_dtype BI_BF16 | BI_F32).
 *   Supported: D = 128, page_size a multiple of 16 dividing 256.
 *   Errors: BI_ERR_DTYPE, BI_ERR_SHAPE, BI_ERR_UNSUPPORTED, BI_ERR_NULL, BI_ERR_ALIGN
 *   (k_cache, v_cache not 16-byte aligned). */
int bi_rope_kv_write(const void* qkv, int64_t ldqkv, int qkv_dtype, void* q, int q_dtype,
                     void* k_cache, void* v_cache, const int32_t* block_table,
                     const int32_t* seq_lens, const int32_t* query_start_loc, int32_t batch,
                     int64_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                     int32_t head_dim, int32_t page_size, int32_t max_pages_per_seq, double base,
                     void* stream);

/* bi_swiglu: out[t, j] = silu(g) * u with g = gu[t, j], u = gu[t, F + j];
 *   silu(g) = g / (1 + 2^(-g log2 e)) in fp32 with the hardware base-2 exponential
 *   (graded against fp64 within tolerance, the same code for every element).
 *   gu [T, 2F] bf16 (row stride ldgu, a multiple of 8), out [T, F] bf16. */
int bi_swiglu(const void* gu, int64_t ldgu, void* out, int64_t T, int64_t F, void* stream);

/* bi_gemm_swiglu: the gate/up projection and bi_swiglu in one call (the fusion of
 *   pointwise work into the producing kernel that "Defeating nondeterminism in LLM
 *   inference" allows because pointwise operations are batch-invariant): out[M, F] =
 *   swiglu(A . W^T) where W [2F, K] bf16 holds the gate and up rows interleaved in blocks
 *   of 16 (rows 32 b .. 32 b + 15 = gate rows 16 b .., rows 32 b + 16 .. = up rows 16 b ..).
 *   Each gate and up value is the bi_gemm element (same instruction sequence) rounded to
 *   bf16, and the pair goes through bi_swiglu's arithmetic, so out equals
 *   bi_swiglu(bi_gemm(A, W_gate_up)) bit for bit without writing the [M, 2F] intermediate.
 *   A [M, K] bf16 (row stride lda), W row stride ldw, out row stride ldo (bf16).
 *   w_layout BI_B_NK: W as above; BI_B_TILED: bi_pack_b of that [2F, K] W (ldw unused; at
 *   most 64 rows, K a multiple of 8 and at least 1024), the same bits.
 *   Errors: BI_ERR_DTYPE (w_layout), BI_ERR_NULL, BI_ERR_SHAPE (F not a multiple of 16,
 *   strides too small), BI_ERR_ALIGN (16-byte pointers, lda and ldw multiples of 8),
 *   BI_ERR_UNSUPPORTED (A or W spanning 4 GiB or more: use bi_gemm and bi_swiglu; a tiled W
 *   outside its row and K range). */
int bi_gemm_swiglu(const void* A, const void* W, void* out, int64_t M, int64_t F, int64_t K,
                   int64_t lda, int64_t ldw, int64_t ldo, int w_layout, void* stream);

/* bi_pack_b: B [N, K] bf16 (row stride ldb) rewritten in the tiled layout of BI_B_TILED,
 *   for weights read by calls of a few rows (greedy decode): 16-row x 32-column tiles,
 *   stored one after another (row block b, then the 32-wide K step t), each 1 KB tile in
 *   the order the few-row kernel's 64 lanes take their matrix-instruction operands --
 *   B[16 b + r][32 t + 8 g + e] at ((b * ceil(K/32) + t) * 64 + r + 16 g) * 8 + e, zero past
 *   N and K -- so each of a wave's loads reads one contiguous kilobyte, not 64 bytes from
 *   each of 16 rows (no bit changes: the same operands reach the same instruction).
 *   out: bi_pack_b_bytes(N, K) bytes, 16-byte aligned.  Layout chosen for MI355X's HBM,
 *   not taken from the pages.
 *   Errors: BI_ERR_SHAPE, BI_ERR_NULL, BI_ERR_ALIGN. */
size_t bi_pack_b_bytes(int64_t N, int64_t K);
int bi_pack_b(const void* B, int64_t N, int64_t K, int64_t ldb, void* out, void* stream);

/* bi_residual_add: out = a + b elementwise over n elements, each operand of its own
 *   dtype (BI_BF16 | BI_F32); out may alias a or b. */
int bi_residual_add(const void* a, int a_dtype, const void* b, int b_dtype, void* out,
                    int out_dtype, int64_t n, void* stream);

/* bi_add_rmsnorm: the residual add and the RMSNorm after it in one pass over M contiguous
 *   rows of D (pointwise work fused into the producing kernel, which keeps batch invariance):
 *   sum = a + b (fp32 add, rounded to dtype, exactly bi_residual_add) and
 *   y = rmsnorm(sum, gamma, eps) from the rounded sum with bi_rmsnorm's tree for that dtype,
 *   so both outputs equal the two calls bit for bit.  a, b, sum of dtype (BI_BF16 | BI_F32);
 *   sum may alias a or b; y of y_dtype; gamma bf16 [D].
 *   Errors: BI_ERR_DTYPE, BI_ERR_SHAPE, BI_ERR_NULL, BI_ERR_UNSUPPORTED (D not a multiple of
 *   8 or above 8192: use the two calls), BI_ERR_ALIGN (a, b, sum, y not 16-byte aligned). */
int bi_add_rmsnorm(const void* a, const void* b, void* sum, int dtype, const void* gamma, void* y,
                   int y_dtype, int64_t M, int64_t D, float eps, void* stream);

/* bi_add_rmsnorm_gemm, bi_add_rmsnorm_gemm_swiglu: the residual add, the RMSNorm after it
 *   and the projection that reads the normalised rows in one launch, for calls of a few rows
 *   (greedy decode), where each launch costs more than its bytes ("Defeating nondeterminism
 *   in LLM inference", section on batch-invariant RMSNorm: each row keeps its own fixed
 *   reduction; pointwise work fused with its neighbours).  Every workgroup replays the row's
 *   tree (bi_add_rmsnorm's, bf16) and multiplies the normalised bf16 rows from LDS, so
 *     sum = a + b                         equals bi_add_rmsnorm's sum,
 *     C   = rmsnorm(sum) . W^T            equals bi_gemm of bi_add_rmsnorm's y (c_dtype),
 *     out = swiglu(rmsnorm(sum) . W^T)    equals bi_gemm_swiglu of that y,
 *   bit for bit, without writing or re-reading y.
 *   a, b, sum [M, K] bf16, rows contiguous (stride K); sum must not overlap a or b (one
 *   workgroup writes it while the others read them), and C / out must overlap none of the
 *   inputs (checked for sum only); gamma bf16 [K]; W as in bi_gemm (N rows)
 *   or bi_gemm_swiglu (2F interleaved rows): w_layout BI_B_NK with row stride ldw, or
 *   BI_B_TILED (ldw unused); C [M, N] (c_dtype BI_BF16 | BI_F32), out [M, F] bf16, row
 *   strides ldc / ldo.
 *   Supported: 1 <= M <= 4, K a multiple of 8 with 1024 <= K <= 4096 (the normalised rows
 *   sit in at most 32 KB of LDS); otherwise BI_ERR_UNSUPPORTED (use bi_add_rmsnorm and the
 *   projection).
 *   Errors: BI_ERR_DTYPE (w_layout, c_dtype), BI_ERR_SHAPE (strides too small, F not a
 *   multiple of 16, sum overlapping a or b), BI_ERR_NULL, BI_ERR_ALIGN (16-byte pointers,
 *   ldw a multiple of 8), BI_ERR_UNSUPPORTED. */
int bi_add_rmsnorm_gemm(const void* a, const void* b, void* sum, const void* gamma, float eps,
                        const void* W, void* C, int64_t M, int64_t N, int64_t K, int64_t ldw,
                        int64_t ldc, int w_layout, int c_dtype, void* stream);
int bi_add_rmsnorm_gemm_swiglu(const void* a, const void* b, void* sum, const void* gamma, float eps,
                               const void* W, void* out, int64_t M, int64_t F, int64_t K,
                               int64_t ldw, int64_t ldo, int w_layout, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* BI_H_ */
