// Internal launchers behind the C ABI (include/csa2.h). Arguments are already
// validated by the caller; each returns 0 after enqueueing on `s`.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa2 {

int launch_fp4_pack(const uint16_t* x, int64_t n, uint8_t* out, hipStream_t s);
int launch_fp4_unpack(const uint8_t* in, int64_t n, uint16_t* y, hipStream_t s);

int launch_kidx_fp4_pack(const uint16_t* x, int64_t n, uint8_t* out, hipStream_t s);
int launch_swa_fp8_pack(const uint16_t* x, int64_t n, uint8_t* out, hipStream_t s);

// Indexer scoring; k is bf16 [nseq][N][128] (kfp4 false) or FP4 entries
// [nseq][N][68] (kfp4 true). qfp4 (with kfp4): q_idx points to MXFP4 query
// entries [nq][32][68] instead of bf16 [nq][32][128] (every scoring launcher).
int launch_index_full(const uint16_t* q_idx, const float* w, const void* k, bool kfp4, int64_t N, int32_t nq,
                      int32_t q_per_seq, const int32_t* n_visible, float* scores, int32_t block_size,
                      float* block_scores, hipStream_t s, bool qfp4 = false);
int launch_index_reindex(const uint16_t* q_idx, const float* w, const void* k, bool kfp4, int64_t N, int32_t nq,
                         int32_t q_per_seq, const int32_t* n_visible, const int32_t* cand_blocks, int32_t nb,
                         float* pool_scores, int32_t* pool_ids, hipStream_t s, bool qfp4 = false);

// Full-mode scoring fused with Top-K for decode (one query per sequence), in
// two launches: scoring + per-chunk selection (writes out_idx itself when the
// row is one chunk), then the merge of the chunks' candidates held in ws.
// block_scores and scores_dbg optional.
size_t index_topk_workspace_bytes(int32_t nq, int64_t N, int32_t k);
bool index_topk_fits(int32_t nq, int64_t N, int32_t k);
int launch_index_topk(const uint16_t* q_idx, const float* w, const void* k, bool kfp4, int64_t N, int32_t nq,
                      const int32_t* n_visible, int32_t topk, int32_t* out_idx, float* block_scores,
                      float* scores_dbg, void* ws, hipStream_t s, bool qfp4 = false);
int launch_index_topk_merge(int64_t N, int32_t nq, int32_t topk, int32_t* out_idx, void* ws, hipStream_t s);
// The merge above and the pool's Top-pool_k blocks over the block maxima
// (rows of ceil(N / 8)), sharing launches; ws holds the merge's candidates
// first (as for launch_index_topk), then the block selection's.
size_t index_topk_pool_workspace_bytes(int32_t nq, int64_t N, int32_t k, int32_t pool_k);
int launch_index_topk_merge_pool(int64_t N, int32_t nq, int32_t topk, int32_t* out_idx, const float* block_scores,
                                 int32_t pool_k, int32_t* cand_blocks, void* ws, hipStream_t s);
// Static device scratch of csa2_index_topk_noalloc: its size, and its address
// on the current device (nullptr and *err set when the lookup fails).
size_t index_topk_noalloc_capacity();
void* index_topk_noalloc_scratch(hipError_t* err);
bool reindex_topk_fits(int32_t nq, int32_t nb, int32_t k);
size_t reindex_topk_workspace_bytes(int32_t nq, int32_t nb, int32_t k);
int launch_index_reindex_topk(const uint16_t* q_idx, const float* w, const void* k, bool kfp4, int64_t N, int32_t nq,
                              int32_t q_per_seq, const int32_t* n_visible, const int32_t* cand_blocks, int32_t nb,
                              int32_t topk, int32_t* out_idx, float* pool_scores, void* ws, hipStream_t s,
                              bool qfp4 = false);

// Prefill scoring (q_per_seq a multiple of 8) fused with the per-query Top-k
// (k <= 512): one launch scores and selects per chunk of the row (final
// indices when a row is one chunk), a second merges chunks' candidates.
bool prefill_topk_fits(int32_t nq, int64_t N, int32_t k);
size_t prefill_topk_workspace_bytes(int32_t nq, int64_t N, int32_t k);
int launch_index_prefill_topk(const uint16_t* q_idx, const float* w, const void* k, bool kfp4, int64_t N, int32_t nq,
                              int32_t q_per_seq, const int32_t* n_visible, int32_t topk, int32_t* out_idx,
                              float* scores_dbg, void* ws, hipStream_t s);

// MXFP4 indexer Q [nq][32][68] with MXFP4 K [nseq][N][68] on the scaled FP4
// MFMA, for prefill chunks (q_per_seq a multiple of 8): scoring alone, and
// scoring fused with the per-query Top-k (workspace as launch_index_prefill_topk).
int launch_index_full_fp4qk(const uint8_t* q_fp4, const float* w, const uint8_t* k_fp4, int64_t N, int32_t nq,
                            int32_t q_per_seq, const int32_t* n_visible, float* scores, int32_t block_size,
                            float* block_scores, hipStream_t s);
int launch_index_prefill_topk_fp4qk(const uint8_t* q_fp4, const float* w, const uint8_t* k_fp4, int64_t N,
                                    int32_t nq, int32_t q_per_seq, const int32_t* n_visible, int32_t topk,
                                    int32_t* out_idx, float* scores_dbg, void* ws, hipStream_t s);

size_t topk_workspace_bytes(int32_t rows, int64_t ncols, int32_t k);
// Merge of per-chunk Top-K candidates: rows x nchunks x k (key, column) pairs
// in column order (unused slots key 0) -> out_idx [rows][k]. Above 16384
// candidates per row a first level merges groups into ck2/cc2
// (rows x topk_merge_groups(nchunks, k) x k pairs).
int32_t topk_merge_groups(int32_t nchunks, int32_t k);
int launch_topk_merge(int32_t rows, int32_t k, int32_t nchunks, const uint32_t* ck, const int32_t* cc,
                      int32_t* out_idx, uint32_t* ck2, int32_t* cc2, hipStream_t s);
// That merge together with an independent Top-k_b over rows_b x ncols_b
// scores (as launch_topk, no row_len or id_map; its chunks' candidates in
// ws_b), each level of the two in one launch. Returns false, launching
// nothing, when the second selection needs the global-memory path.
bool launch_topk_merge_select(int32_t rows_a, int32_t k_a, int32_t nchunks_a, const uint32_t* ck, const int32_t* cc,
                              int32_t* out_a, uint32_t* ck2, int32_t* cc2, const float* scores_b, int32_t rows_b,
                              int64_t ncols_b, int32_t k_b, int32_t* out_b, void* ws_b, hipStream_t s);
int launch_topk(const float* scores, int32_t rows, int64_t ncols, int64_t ld, const int32_t* row_len, int32_t k,
                const int32_t* id_map, int32_t* out_idx, void* ws, hipStream_t s);

size_t attn_workspace_bytes(int32_t nq, int32_t k);
// swa: bf16 rows [nseq][T][512] (swa_fp8 false) or FP8 rows [nseq][T][528].
int launch_sparse_attn(const uint16_t* q, const uint8_t* kv, int64_t N, int32_t nq, int32_t q_per_seq,
                       const int32_t* idx, int32_t k, const void* swa, bool swa_fp8, int64_t T, const int32_t* swa_start,
                       const int32_t* swa_len, float softmax_scale, uint16_t* out, float* lse, void* ws,
                       hipStream_t s);

}  // namespace csa2
