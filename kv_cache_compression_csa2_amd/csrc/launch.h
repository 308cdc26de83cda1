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
// [nseq][N][68] (kfp4 true).
int launch_index_full(const uint16_t* q_idx, const float* w, const void* k, bool kfp4, int64_t N, int32_t nq,
                      int32_t q_per_seq, const int32_t* n_visible, float* scores, int32_t block_size,
                      float* block_scores, hipStream_t s);
int launch_index_reindex(const uint16_t* q_idx, const float* w, const void* k, bool kfp4, int64_t N, int32_t nq,
                         int32_t q_per_seq, const int32_t* n_visible, const int32_t* cand_blocks, int32_t nb,
                         float* pool_scores, int32_t* pool_ids, hipStream_t s);

size_t topk_workspace_bytes(int32_t rows, int64_t ncols, int32_t k);
int launch_topk(const float* scores, int32_t rows, int64_t ncols, int64_t ld, const int32_t* row_len, int32_t k,
                const int32_t* id_map, int32_t* out_idx, void* ws, hipStream_t s);

size_t attn_workspace_bytes(int32_t nq, int32_t k);
// swa: bf16 rows [nseq][T][512] (swa_fp8 false) or FP8 rows [nseq][T][528].
int launch_sparse_attn(const uint16_t* q, const uint8_t* kv, int64_t N, int32_t nq, int32_t q_per_seq,
                       const int32_t* idx, int32_t k, const void* swa, bool swa_fp8, int64_t T, const int32_t* swa_start,
                       const int32_t* swa_len, float softmax_scale, uint16_t* out, float* lse, void* ws,
                       hipStream_t s);

}  // namespace csa2
