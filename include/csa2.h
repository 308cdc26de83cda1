/*
 * csa2.h -- C ABI of the CSA2 (Compressed Sparse Attention 2) global-attention
 * hot path on AMD Instinct MI355X (gfx950).
 *
 * The calls follow how the pages on DeepSeek-V4.1-Flash state the problem:
 *   - eogee.com report "DeepSeek V4.1-Flash 技术报告深度解析", 3.2: a light
 *     indexer scores main-KV entries with an indexer Q and an indexer K (32
 *     heads x 128 dims), each query keeps its Top-K (512) entries and attends
 *     to them plus its layer's sliding-window (SWA, 128 tokens) KV with 64
 *     query heads of dim 512 sharing one KV head. Layers run in Full (score
 *     every visible entry), Reindex (own indexer Q over the shared indexer K)
 *     or Reuse (inherit the indices) mode.
 *   - same report, 3.3: the decoder's first Full layer also keeps the 2048 best
 *     blocks of 8 positions (block score = best position score) as a candidate
 *     pool of 16384 positions; later Reindex layers score only that pool.
 *   - same report, 3.4, and the nxbn.cn walkthrough 2.3: the main KV is stored
 *     as FP4 E2M1 with one E4M3 scale per 16 channels and dequantized before the
 *     attention math.
 * Details the pages leave open are fixed as: score = sum_h w_h * max(q_h.k, 0);
 * block score = max of its positions; each main-KV entry is both key and
 * value; RoPE is already applied; softmax scale is an argument (1/sqrt(512));
 * ties go to the lower position.
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers owned by the caller, unless stated.
 *   - bf16 values travel as uint16_t bit patterns; sizes are int64_t/int32_t.
 *   - Work is enqueued on `stream` (0 = the null stream); the call returns
 *     without synchronizing. Faults inside kernels surface at the caller's
 *     next synchronization.
 *   - The library never allocates device memory and keeps no state between
 *     calls: calls on different streams may run concurrently if their outputs
 *     do not overlap.
 *   - Return value: CSA2_OK, or a negative code. CSA2_EINVAL: an argument
 *     check failed, nothing was launched and no output was touched.
 *     CSA2_ELAUNCH: the HIP runtime refused a launch (outputs unspecified).
 *     CSA2_EWORKSPACE: the workspace passed is smaller than the matching
 *     *_workspace_bytes() result. csa2_last_error() gives a message for the
 *     calling thread's last failure.
 *   - Geometry is fixed: 512-channel main entries in 288-byte records, 32 x 128
 *     indexer heads, 64 x 512 attention heads, sliding windows of at most 128.
 *   - Query, key, record, window, output and workspace arrays are accessed
 *     with 16-byte vector loads and stores: their base pointers must be
 *     16-byte aligned (hipMalloc and torch allocations are). csa2_topk's score
 *     rows may start at any 4-byte boundary (unaligned rows take scalar loads).
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA2_OK 0
#define CSA2_EINVAL (-1)
#define CSA2_ELAUNCH (-2)
#define CSA2_EWORKSPACE (-3)

#define CSA2_DIM 512        /* attention head dim = main-KV entry channels */
#define CSA2_HEADS 64       /* query heads sharing the single KV head */
#define CSA2_IDX_HEADS 32   /* indexer heads */
#define CSA2_IDX_DIM 128    /* indexer head dim */
#define CSA2_GROUP 16       /* channels per E4M3 scale */
#define CSA2_RECORD 288     /* bytes per FP4 main-KV entry: 256 code bytes + 32 scale bytes */
#define CSA2_KIDX_RECORD 68 /* bytes per FP4 indexer-K entry: 64 code bytes + 4 E8M0 scales */
#define CSA2_SWA_RECORD 528 /* bytes per FP8 window-KV row: 512 E4M3 codes + 16 E8M0 scales */
#define CSA2_MAX_WINDOW 128 /* sliding-window length limit */
#define CSA2_MAX_TOPK 4096  /* largest k accepted by csa2_topk */

/* Status bits the attention calls OR into the first 4 bytes of their
 * workspace for inputs outside the documented domain (device data the host
 * cannot check without synchronizing). The library never clears the word:
 * the caller zeroes it, runs one or more calls, synchronizes and reads it. The
 * outputs of a query that set a bit are unspecified. */
#define CSA2_STATUS_IDX 1u        /* a selected id outside [-1, N) (the slot is skipped) */
#define CSA2_STATUS_WIN_LEN 2u    /* swa_len outside [0, 128] (at most 128 rows are used) */
#define CSA2_STATUS_WIN_RANGE 4u  /* window rows outside [0, T) (those rows are skipped) */
#define CSA2_STATUS_NONFINITE 8u  /* a non-finite output element: a window value fp16 cannot hold (magnitude
                                   * >= 65536; FP8 rows: a block scale byte above 134), a NaN E4M3 scale byte,
                                   * or another non-finite input */

/* Layout version of the 288-byte record (below); bumps if the layout changes. */
int csa2_format_version(void);

/* Message describing the calling thread's last non-OK return (static storage). */
const char* csa2_last_error(void);

/*
 * fp4_kv_pack -- write FP4 main-KV records (eogee.com report 3.4; nxbn.cn 2.3).
 *   x_bf16 [n][512] bf16 row-major, values after RoPE.
 *   out    [n][288] bytes. Record: byte j (0..255) holds channel 2j in bits 3:0
 *          and channel 2j+1 in bits 7:4 as E2M1 codes (bit 3 sign); byte 256+g
 *          (g = 0..31) holds the E4M3 scale of channels 16g..16g+15.
 *   Per 16-channel group: S = E4M3(amax/6) (amax/6 in fp32, rounded to nearest
 *   even, saturating at 448); each channel takes the E2M1 code whose value
 *   times S is nearest to x (ties to the even code, beyond 6S -> 6S; zero
 *   magnitude -> +0 code); S == 0 gives all-zero codes. Inputs must be finite.
 *   n >= 0 (n == 0 launches nothing). Records are independent, so a caller may
 *   pack one new token's entry at a time.
 */
int fp4_kv_pack(const uint16_t* x_bf16, int64_t n, uint8_t* out, hipStream_t stream);

/*
 * fp4_kv_unpack -- decode FP4 records to bf16: y = E2M1(code) * E4M3(scale),
 * exact in bf16. in [n][288] -> y_bf16 [n][512]. Test and inspection export;
 * the attention kernel decodes records on the fly and never calls it.
 */
int fp4_kv_unpack(const uint8_t* in, int64_t n, uint16_t* y_bf16, hipStream_t stream);

/*
 * csa2_index_full -- Full-mode indexer scoring (eogee.com report 3.2, 3.3).
 *   q_idx     [nq][32][128] bf16: the layer's indexer query heads.
 *   w         [nq][32] fp32: per-head weights.
 *   k_idx     [nseq][N][128] bf16: shared indexer-K cache, nseq = nq/q_per_seq.
 *   N         entries per sequence (1 .. 2^31-1).
 *   q_per_seq queries per sequence; query q reads sequence q / q_per_seq
 *             (decode: 1, prefill chunk on one sequence: nq). Must divide nq.
 *   n_visible [nq] int32 or NULL (= N): entries [0, n_visible[q]) are visible
 *             and the rest score -inf; values above N act as N, negative
 *             values as 0.
 *   scores    [nq][N] fp32 out: sum_h w[q][h] * max(q_idx[q][h] . k, 0).
 *   block_size 0 (no block scores) or 8.
 *   block_scores [nq][ceil(N/8)] fp32 out (when block_size == 8): max of the
 *             block's scores (-inf if none visible). NULL when block_size == 0.
 */
int csa2_index_full(const uint16_t* q_idx, const float* w, const uint16_t* k_idx, int64_t N, int32_t nq,
                    int32_t q_per_seq, const int32_t* n_visible, float* scores, int32_t block_size,
                    float* block_scores, hipStream_t stream);

/*
 * csa2_index_reindex -- Reindex-mode scoring restricted to the candidate pool
 * (eogee.com report 3.3: later indexers score only inside the pool).
 *   q_idx, w, k_idx, N, nq, q_per_seq, n_visible: as csa2_index_full, with the
 *             Reindex layer's own q_idx and w.
 *   cand_blocks [nq][nb] int32: block ids chosen by the Full layer (ascending
 *             for lower-position tie-breaks downstream; -1 = padding).
 *   nb        blocks per query (1 .. 65536); block_size must be 8.
 *   pool_scores [nq][nb*8] fp32 out: score of entry cand_blocks[q][j]*8 + t at
 *             position j*8 + t; -inf for padding, invisible or >= N entries.
 *   pool_ids  [nq][nb*8] int32 out or NULL: the entry id at each position
 *             (-1 where the score is -inf because of padding or range).
 */
int csa2_index_reindex(const uint16_t* q_idx, const float* w, const uint16_t* k_idx, int64_t N, int32_t nq,
                       int32_t q_per_seq, const int32_t* n_visible, const int32_t* cand_blocks, int32_t nb,
                       int32_t block_size, float* pool_scores, int32_t* pool_ids, hipStream_t stream);

/*
 * kidx_fp4_pack -- FP4 indexer-K entries, the storage precision the pages'
 * byte accounting implies (890 B/token = 2.5 entries x (288 B main KV + 68 B
 * indexer K): titansim blog, eogee.com report 5.3), in the OCP MXFP4 format
 * eogee.com report 3.4 names (that passage also notes FP4 indexer Q/K in the
 * predecessor).
 *   x_bf16 [n][128] bf16 row-major.
 *   out    [n][68] bytes. Entry: byte j (0..63) holds channel 2j in bits 3:0
 *          and channel 2j+1 in bits 7:4 as E2M1 codes (bit 3 sign); byte 64+g
 *          (g = 0..3) holds the E8M0 scale (value 2^(b-127)) of channels
 *          32g..32g+31. Per block X = 2^(floor(log2 amax) - 2), clamped to
 *          [2^-127, 2^127] (an all-zero block gets 2^-127); each channel takes
 *          the E2M1 code nearest to x / X (ties to the even code, beyond 6 ->
 *          6, zero magnitude -> +0). Inputs must be finite. n >= 0; entries
 *          are independent.
 *   value(channel c) = E2M1(code_c) * 2^(scale_byte(c/32) - 127).
 */
int kidx_fp4_pack(const uint16_t* x_bf16, int64_t n, uint8_t* out, hipStream_t stream);

/*
 * swa_fp8_pack -- FP8 window-KV rows (eogee.com report 3.4: the window KV,
 * sensitive to quantization, stays in FP8; the block scaling is the OCP MX
 * format the same passage names for the cache: MXFP8 with E4M3 elements).
 *   x_bf16 [n][512] bf16 row-major.
 *   out    [n][528] bytes. Bytes 0..511: the E4M3 code of each channel in
 *          channel order; byte 512+g: the E8M0 scale (value 2^(b-127)) of
 *          channels 32g..32g+31. Per block X = 2^(floor(log2 amax) - 8),
 *          clamped to [2^-127, 2^127] (an all-zero block gets 2^-127); each
 *          channel is the E4M3 value nearest to x / X (ties to even, beyond
 *          448 -> 448, zero magnitude -> +0). Inputs must be finite. n >= 0.
 *   value(channel c) = E4M3(code_c) * 2^(scale_byte - 127).
 */
int swa_fp8_pack(const uint16_t* x_bf16, int64_t n, uint8_t* out, hipStream_t stream);

/*
 * csa2_index_full_fp4k / csa2_index_reindex_fp4k -- csa2_index_full and
 * csa2_index_reindex over the FP4 indexer-K cache k_fp4 [nseq][N][68] (entries
 * of kidx_fp4_pack) instead of bf16 k_idx; every other argument, output and
 * error rule is the same. The score uses the decoded key E2M1(code) * 2^(b-127),
 * which enters the bf16 products exactly for scale bytes b in [2, 252] (the
 * packer writes 0..252; blocks with a byte below 2 have all magnitudes under
 * 2^-123 and decode to subnormal numbers, which the products may flush to 0).
 */
int csa2_index_full_fp4k(const uint16_t* q_idx, const float* w, const uint8_t* k_fp4, int64_t N, int32_t nq,
                         int32_t q_per_seq, const int32_t* n_visible, float* scores, int32_t block_size,
                         float* block_scores, hipStream_t stream);
int csa2_index_reindex_fp4k(const uint16_t* q_idx, const float* w, const uint8_t* k_fp4, int64_t N, int32_t nq,
                            int32_t q_per_seq, const int32_t* n_visible, const int32_t* cand_blocks, int32_t nb,
                            int32_t block_size, float* pool_scores, int32_t* pool_ids, hipStream_t stream);

/*
 * csa2_index_topk -- Full-mode scoring fused with the per-query Top-K, for
 * decode (one query per sequence): the Top-k of csa2_index_full's score row
 * without writing that row (titansim blog: each Full layer keeps its own
 * Top-512; eogee.com report 3.5 names a fused Top-K selection kernel).
 *   q_idx, w, k_idx, N, n_visible: as csa2_index_full with q_per_seq = 1
 *           (k_idx [nq][N][128], sequence q belongs to query q).
 *   k       1 .. CSA2_MAX_TOPK; the chunks' candidates must fit two merge
 *           levels of 16384 (for k = 512: N up to 4,194,304), else EINVAL.
 *   top_idx [nq][k] int32 out: exactly csa2_topk(scores, k, row_len =
 *           n_visible) of the row csa2_index_full would produce: ascending
 *           entry ids, then -1 padding; order of merit score desc, equal
 *           scores (-0 == +0) by lower entry id.
 *   block_size 0 or 8; with 8, block_scores [nq][ceil(N/8)] fp32 out as in
 *           csa2_index_full (the hierarchical pool's input).
 *   scores  [nq][N] fp32 out or NULL: the score row itself (checking aid).
 *   workspace / ws_bytes: at least csa2_index_topk_workspace_bytes(nq, N, k)
 *           bytes (per-chunk candidates); may be NULL when that is 0.
 *           Contents on entry do not matter.
 * The call is two launches on `stream`: scoring with a per-chunk Top-k (a
 * query's row is cut into chunks of 4096 or 8192 entries; with one chunk the
 * result is final), then the merge of the chunks' candidates. The two halves
 * are also exported on their own: csa2_index_topk_select (k_is_fp4 selects
 * the key format) leaves the candidates in the workspace, and
 * csa2_index_topk_merge, called next on the same stream with the same
 * (N, nq, k, top_idx, workspace), completes top_idx.
 */
size_t csa2_index_topk_workspace_bytes(int32_t nq, int64_t N, int32_t k);
int csa2_index_topk(const uint16_t* q_idx, const float* w, const uint16_t* k_idx, int64_t N, int32_t nq,
                    const int32_t* n_visible, int32_t k, int32_t* top_idx, int32_t block_size, float* block_scores,
                    float* scores, void* workspace, size_t ws_bytes, hipStream_t stream);
/* csa2_index_topk over FP4 indexer-K entries (k_fp4 [nq][N][68], kidx_fp4_pack). */
int csa2_index_topk_fp4k(const uint16_t* q_idx, const float* w, const uint8_t* k_fp4, int64_t N, int32_t nq,
                         const int32_t* n_visible, int32_t k, int32_t* top_idx, int32_t block_size,
                         float* block_scores, float* scores, void* workspace, size_t ws_bytes, hipStream_t stream);
int csa2_index_topk_select(const uint16_t* q_idx, const float* w, const void* k, int32_t k_is_fp4, int64_t N,
                           int32_t nq, const int32_t* n_visible, int32_t topk, int32_t* top_idx, int32_t block_size,
                           float* block_scores, float* scores, void* workspace, size_t ws_bytes, hipStream_t stream);
int csa2_index_topk_merge(int64_t N, int32_t nq, int32_t k, int32_t* top_idx, void* workspace, size_t ws_bytes,
                          hipStream_t stream);

/*
 * csa2_index_topk_merge_pool -- the rest of a hierarchical Full layer after
 * csa2_index_topk_select with block_size 8: completes the layer's Top-k (as
 * csa2_index_topk_merge) and selects the candidate pool's best blocks from the
 * block maxima (as csa2_topk(block_scores, pool_k); eogee.com report 3.3: the
 * Full layer keeps the 2048 best 8-position blocks for the Reindex layers).
 * The two selections do not depend on each other and share launches.
 *   N, nq, k, top_idx: as the csa2_index_topk_select call before it, on the
 *           same stream.
 *   block_scores [nq][ceil(N/8)] fp32 in: the block maxima that call wrote.
 *   pool_k  1 .. CSA2_MAX_TOPK.
 *   cand_blocks [nq][pool_k] int32 out: exactly csa2_topk(block_scores,
 *           pool_k): ascending block ids, then -1 padding.
 *   workspace / ws_bytes: at least csa2_index_topk_pool_workspace_bytes(nq, N,
 *           k, pool_k) bytes, the same buffer the select call wrote its
 *           candidates to (the pool's selection uses the bytes after them).
 */
size_t csa2_index_topk_pool_workspace_bytes(int32_t nq, int64_t N, int32_t k, int32_t pool_k);
int csa2_index_topk_merge_pool(int64_t N, int32_t nq, int32_t k, int32_t* top_idx, const float* block_scores,
                               int32_t pool_k, int32_t* cand_blocks, void* workspace, size_t ws_bytes,
                               hipStream_t stream);

/*
 * csa2_index_topk_noalloc -- csa2_index_topk with no workspace argument and no
 * allocation, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *   Arguments, outputs and errors as csa2_index_topk (k_is_fp4 != 0: `k` holds
 *   FP4 entries [nq][N][68], else bf16 keys [nq][N][128]), except:
 *   - the per-chunk candidates go to a static device array of
 *     csa2_index_topk_noalloc_scratch_bytes() bytes (16 MiB) that each GPU
 *     the library runs on holds until the process ends; a call whose
 *     csa2_index_topk_workspace_bytes(nq, N, topk) exceeds it returns
 *     CSA2_EINVAL (Top-512 fits up to 128 queries x 262144 entries or 16 x
 *     1048576);
 *   - the scratch of the calling thread's current device is used, so the
 *     stream must belong to that device;
 *   - every call on one GPU shares that scratch: calls that overlap in time on
 *     one GPU (different streams, or different host threads) race and give
 *     undefined results. Calls in order on one stream are safe.
 *   The first call on a device looks up the scratch address (CSA2_ELAUNCH if
 *   that fails). No hipMalloc, hipFree or memset is made.
 */
size_t csa2_index_topk_noalloc_scratch_bytes(void);
int csa2_index_topk_noalloc(const uint16_t* q_idx, const float* w, const void* k, int32_t k_is_fp4, int64_t N,
                            int32_t nq, const int32_t* n_visible, int32_t topk, int32_t* top_idx, int32_t block_size,
                            float* block_scores, float* scores, hipStream_t stream);

/*
 * csa2_index_prefill_topk -- Full-mode scoring fused with the per-query Top-K
 * for a prefill chunk (many queries over one sequence): the Top-k of
 * csa2_index_full's score row without writing that row (eogee.com report 3.5
 * names the fused Top-K selection kernel; titansim blog: Top-512 per query).
 *   q_idx, w, k_idx, N, nq, q_per_seq, n_visible: as csa2_index_full;
 *           q_per_seq must be a multiple of 8 (the kernel scores 8 queries of
 *           one sequence together).
 *   k       1 .. 512.
 *   top_idx [nq][k] int32 out: exactly csa2_topk(scores, k, row_len =
 *           n_visible) of the row csa2_index_full would produce (ascending
 *           entry ids, then -1 padding; equal scores by lower entry id).
 *   scores  [nq][N] fp32 out or NULL: the score row itself (checking aid).
 *   workspace / ws_bytes: at least csa2_index_prefill_topk_workspace_bytes(nq,
 *           N, k) bytes (0 when a row is scored by one workgroup; then the
 *           call is one launch). Contents on entry do not matter.
 *   EINVAL also when the chunks' candidates would not fit two merge levels of
 *   16384 (the workspace-size call then returns 0).
 * _fp4k: the same over FP4 indexer-K entries (k_fp4 [nseq][N][68]).
 */
size_t csa2_index_prefill_topk_workspace_bytes(int32_t nq, int64_t N, int32_t k);
int csa2_index_prefill_topk(const uint16_t* q_idx, const float* w, const uint16_t* k_idx, int64_t N, int32_t nq,
                            int32_t q_per_seq, const int32_t* n_visible, int32_t k, int32_t* top_idx, float* scores,
                            void* workspace, size_t ws_bytes, hipStream_t stream);
int csa2_index_prefill_topk_fp4k(const uint16_t* q_idx, const float* w, const uint8_t* k_fp4, int64_t N, int32_t nq,
                                 int32_t q_per_seq, const int32_t* n_visible, int32_t k, int32_t* top_idx,
                                 float* scores, void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * The *_fp4qk calls -- every indexer call with the indexer Q in FP4 as well
 * (eogee.com report 3.4: the predecessor model already trained the indexer Q
 * and K in FP4): q_fp4 [nq][32][68] holds one MXFP4 entry per query head, in
 * the indexer-K entry format (kidx_fp4_pack of the [nq * 32][128] bf16
 * query), in place of the bf16 q_idx, and the indexer K is the FP4 cache
 * k_fp4 [nseq][N][68]. The score is sum_h w[q][h] * max(q_h . k, 0) over the
 * decoded values of both entries: E2M1 products times their two blocks'
 * 2^(b - 127), exact, accumulated in fp32 on the gfx950 scaled FP4 matrix
 * instruction (no decode step). Every other argument, output, workspace and
 * error rule is that of the matching _fp4k call:
 *   csa2_index_full_fp4qk          csa2_index_full_fp4k
 *   csa2_index_reindex_fp4qk       csa2_index_reindex_fp4k
 *   csa2_index_topk_fp4qk          csa2_index_topk_fp4k (decode, fused Top-K)
 *   csa2_index_topk_select_fp4qk   its first launch alone (as csa2_index_topk_select;
 *                                  csa2_index_topk_merge finishes it)
 *   csa2_index_reindex_topk_fp4qk  csa2_index_reindex_topk_fp4k
 *   csa2_index_prefill_topk_fp4qk  csa2_index_prefill_topk_fp4k (q_per_seq a multiple of 8)
 * Caller-owned device buffers; nothing is allocated.
 */
int csa2_index_full_fp4qk(const uint8_t* q_fp4, const float* w, const uint8_t* k_fp4, int64_t N, int32_t nq,
                          int32_t q_per_seq, const int32_t* n_visible, float* scores, int32_t block_size,
                          float* block_scores, hipStream_t stream);
int csa2_index_reindex_fp4qk(const uint8_t* q_fp4, const float* w, const uint8_t* k_fp4, int64_t N, int32_t nq,
                             int32_t q_per_seq, const int32_t* n_visible, const int32_t* cand_blocks, int32_t nb,
                             int32_t block_size, float* pool_scores, int32_t* pool_ids, hipStream_t stream);
int csa2_index_topk_fp4qk(const uint8_t* q_fp4, const float* w, const uint8_t* k_fp4, int64_t N, int32_t nq,
                          const int32_t* n_visible, int32_t k, int32_t* top_idx, int32_t block_size,
                          float* block_scores, float* scores, void* workspace, size_t ws_bytes, hipStream_t stream);
int csa2_index_topk_select_fp4qk(const uint8_t* q_fp4, const float* w, const uint8_t* k_fp4, int64_t N, int32_t nq,
                                 const int32_t* n_visible, int32_t k, int32_t* top_idx, int32_t block_size,
                                 float* block_scores, float* scores, void* workspace, size_t ws_bytes,
                                 hipStream_t stream);
int csa2_index_reindex_topk_fp4qk(const uint8_t* q_fp4, const float* w, const uint8_t* k_fp4, int64_t N, int32_t nq,
                                  int32_t q_per_seq, const int32_t* n_visible, const int32_t* cand_blocks, int32_t nb,
                                  int32_t k, int32_t* top_idx, float* pool_scores, void* workspace, size_t ws_bytes,
                                  hipStream_t stream);
int csa2_index_prefill_topk_fp4qk(const uint8_t* q_fp4, const float* w, const uint8_t* k_fp4, int64_t N, int32_t nq,
                                  int32_t q_per_seq, const int32_t* n_visible, int32_t k, int32_t* top_idx,
                                  float* scores, void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * csa2_index_reindex_topk -- Reindex-mode scoring fused with the layer's
 * Top-K (eogee.com report 3.3: a Reindex layer scores only the candidate pool
 * with its own indexer query and keeps its own Top-K; report 3.5 names the
 * fused selection kernel; titansim blog: Top-512). One launch scores chunks
 * of the pool and selects each chunk's top-k; a second merges the chunks when
 * a row has more than one.
 *   q_idx, w, k_idx, N, nq, q_per_seq, n_visible, cand_blocks, nb: as
 *           csa2_index_reindex (block_size 8).
 *   k       1 .. CSA2_MAX_TOPK; the chunks' candidates must fit two merge
 *           levels of 16384, else EINVAL (k = 512 always fits).
 *   top_idx [nq][k] int32 out: csa2_topk(pool_scores, k, id_map = pool_ids)
 *           of csa2_index_reindex's outputs -- entry ids in pool-position
 *           order (ascending when cand_blocks is ascending), then -1 padding;
 *           equal scores by lower pool position.
 *   pool_scores [nq][nb*8] fp32 out or NULL: the pool row itself (checking aid).
 *   workspace / ws_bytes: at least csa2_index_reindex_topk_workspace_bytes(nq,
 *           nb, k) bytes (per-chunk candidates); may be NULL when that is 0.
 * _fp4k: the same over the FP4 indexer-K cache (k_fp4 [nseq][N][68]).
 */
size_t csa2_index_reindex_topk_workspace_bytes(int32_t nq, int32_t nb, int32_t k);
int csa2_index_reindex_topk(const uint16_t* q_idx, const float* w, const uint16_t* k_idx, int64_t N, int32_t nq,
                            int32_t q_per_seq, const int32_t* n_visible, const int32_t* cand_blocks, int32_t nb,
                            int32_t k, int32_t* top_idx, float* pool_scores, void* workspace, size_t ws_bytes,
                            hipStream_t stream);
int csa2_index_reindex_topk_fp4k(const uint16_t* q_idx, const float* w, const uint8_t* k_fp4, int64_t N, int32_t nq,
                                 int32_t q_per_seq, const int32_t* n_visible, const int32_t* cand_blocks, int32_t nb,
                                 int32_t k, int32_t* top_idx, float* pool_scores, void* workspace, size_t ws_bytes,
                                 hipStream_t stream);

/*
 * csa2_topk -- per-row Top-K selection (titansim blog, CSA2 modes: Top-512;
 * eogee.com report 3.3: Top-2048 blocks).
 *   scores  [rows][ld] fp32, columns [0, ncols) are candidates.
 *   row_len [rows] int32 or NULL: only columns [0, row_len[r]) of row r compete
 *           (values above ncols act as ncols, negative values as 0).
 *   k       1 .. CSA2_MAX_TOPK.
 *   id_map  [rows][ld] int32 or NULL: output column c of row r as id_map[r][c]
 *           (used to turn pool positions into entry ids).
 *   out_idx [rows][k] int32 out: the chosen columns (mapped), ascending by
 *           column, then -1 padding. Order of merit: higher score first, equal
 *           scores (-0 == +0) by lower column. -inf and NaN are never chosen;
 *           a row with fewer than k candidates returns all of them.
 *   workspace / ws_bytes: device scratch of at least
 *           csa2_topk_workspace_bytes(rows, ncols, k) bytes (may be NULL when
 *           that is 0). Contents on entry do not matter.
 */
size_t csa2_topk_workspace_bytes(int32_t rows, int64_t ncols, int32_t k);
int csa2_topk(const float* scores, int32_t rows, int64_t ncols, int64_t ld, const int32_t* row_len, int32_t k,
              const int32_t* id_map, int32_t* out_idx, void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * csa2_sparse_attn -- sparse MQA attention over selected FP4 entries plus the
 * sliding window (eogee.com report 3.2 and 3.4).
 *   q       [nq][64][512] bf16: query heads (RoPE applied).
 *   kv      [nseq][N][288] FP4 records (layout of fp4_kv_pack); entry = key = value.
 *   idx     [nq][k] int32: selected entry ids of query q (in sequence q/q_per_seq);
 *           -1 = empty slot; other values must lie in [0, N). k 0 .. 4096.
 *   swa     [nseq][T][512] bf16: the layer's window KV rows (key = value).
 *   swa_start, swa_len [nq] int32: query q also attends to rows
 *           [swa_start[q], swa_start[q]+swa_len[q]) of its sequence's window
 *           buffer; 0 <= swa_len <= 128 and the range must lie inside [0, T)
 *           (else CSA2_STATUS_WIN_LEN / _WIN_RANGE). Both may be NULL (no
 *           window keys).
 *   softmax_scale: multiplies q.k before the softmax (1/sqrt(512)).
 *           The products run in fp16 with fp32 accumulation: decoded FP4 values
 *           are exact in fp16; each head's q is scaled by a power of two (undone
 *           in its logits) so every finite bf16 q converts exactly, except
 *           elements below 2^-28 of the head's largest, which round; window
 *           values must lie below 65504 in magnitude (else the output is not
 *           finite and CSA2_STATUS_NONFINITE is set; bf16 values of 2^-14 or
 *           more convert exactly, smaller ones to within 2^-25).
 *   out     [nq][64][512] bf16 out: softmax over all of the query's keys jointly.
 *   lse     [nq][64] fp32 out or NULL: natural-log sum of exp of the scaled logits.
 *           A query with no keys gets out = 0 and lse = -inf.
 *   workspace / ws_bytes: at least csa2_sparse_attn_workspace_bytes(nq, k) bytes
 *           (>= 256: the status word, then partial results when a query's keys
 *           are split across workgroups). Bytes [0, 4) hold the status word
 *           (CSA2_STATUS_* bits, ORed in, never cleared); the rest need no
 *           initialization.
 */
size_t csa2_sparse_attn_workspace_bytes(int32_t nq, int32_t k);
int csa2_sparse_attn(const uint16_t* q, const uint8_t* kv, int64_t N, int32_t nq, int32_t q_per_seq,
                     const int32_t* idx, int32_t k, const uint16_t* swa, int64_t T, const int32_t* swa_start,
                     const int32_t* swa_len, float softmax_scale, uint16_t* out, float* lse, void* workspace,
                     size_t ws_bytes, hipStream_t stream);

/*
 * csa2_sparse_attn_fp8w -- csa2_sparse_attn with the window KV stored as FP8
 * rows (eogee.com report 3.4; layout of swa_fp8_pack).
 *   swa_fp8 [nseq][T][528] FP8 window rows; every other argument, the output
 *           and the errors as for csa2_sparse_attn. A decoded window value is
 *           exact in the fp16 products while its 32-channel block maximum
 *           lies in [2^-7, 2^16) (smaller blocks lose bits below 2^-24).
 */
int csa2_sparse_attn_fp8w(const uint16_t* q, const uint8_t* kv, int64_t N, int32_t nq, int32_t q_per_seq,
                          const int32_t* idx, int32_t k, const uint8_t* swa_fp8, int64_t T, const int32_t* swa_start,
                          const int32_t* swa_len, float softmax_scale, uint16_t* out, float* lse, void* workspace,
                          size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* CSA2_H */
