// C ABI of the CSA2 hot path (declared in include/csa2.h): argument checks on
// the host, then kernel launches on the caller's stream. No allocation, no
// state besides the calling thread's last error message.
#include <stdarg.h>
#include <stdio.h>

#include "../../include/csa2.h"
#include "launch.h"

namespace {

thread_local char g_err[256] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int launched(const char* what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(CSA2_ELAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
    return CSA2_OK;
}

constexpr int64_t kMaxN = 2147483647LL;

}  // namespace

extern "C" {

int csa2_format_version(void) { return 1; }

const char* csa2_last_error(void) { return g_err; }

int fp4_kv_pack(const uint16_t* x_bf16, int64_t n, uint8_t* out, hipStream_t stream) {
    if (n < 0) return fail(CSA2_EINVAL, "fp4_kv_pack: n < 0");
    if (n > 0 && (!x_bf16 || !out)) return fail(CSA2_EINVAL, "fp4_kv_pack: null pointer");
    (void)hipGetLastError();
    csa2::launch_fp4_pack(x_bf16, n, out, stream);
    return launched("fp4_kv_pack");
}

int fp4_kv_unpack(const uint8_t* in, int64_t n, uint16_t* y_bf16, hipStream_t stream) {
    if (n < 0) return fail(CSA2_EINVAL, "fp4_kv_unpack: n < 0");
    if (n > 0 && (!in || !y_bf16)) return fail(CSA2_EINVAL, "fp4_kv_unpack: null pointer");
    (void)hipGetLastError();
    csa2::launch_fp4_unpack(in, n, y_bf16, stream);
    return launched("fp4_kv_unpack");
}

static int check_index_common(const char* who, const uint16_t* q_idx, const float* w, const void* k_idx,
                              int64_t N, int32_t nq, int32_t q_per_seq) {
    if (nq < 0) return fail(CSA2_EINVAL, "%s: nq < 0", who);
    if (N < 1 || N > kMaxN) return fail(CSA2_EINVAL, "%s: N must be in [1, 2^31-1]", who);
    if (q_per_seq < 1) return fail(CSA2_EINVAL, "%s: q_per_seq < 1", who);
    if (nq % q_per_seq != 0) return fail(CSA2_EINVAL, "%s: q_per_seq must divide nq", who);
    if (nq > 0 && (!q_idx || !w || !k_idx)) return fail(CSA2_EINVAL, "%s: null pointer", who);
    return CSA2_OK;
}

// Full scoring over bf16 (kfp4 == false) or FP4 (kfp4 == true) indexer K.
static int index_full_impl(const char* who, const uint16_t* q_idx, const float* w, const void* k, bool kfp4,
                           int64_t N, int32_t nq, int32_t q_per_seq, const int32_t* n_visible, float* scores,
                           int32_t block_size, float* block_scores, hipStream_t stream, bool qfp4 = false) {
    int rc = check_index_common(who, q_idx, w, k, N, nq, q_per_seq);
    if (rc) return rc;
    if (nq > 0 && !scores) return fail(CSA2_EINVAL, "%s: null scores", who);
    if (block_size != 0 && block_size != 8) return fail(CSA2_EINVAL, "%s: block_size must be 0 or 8", who);
    if (block_size == 8 && nq > 0 && !block_scores)
        return fail(CSA2_EINVAL, "%s: block_scores required when block_size == 8", who);
    (void)hipGetLastError();
    csa2::launch_index_full(q_idx, w, k, kfp4, N, nq, q_per_seq, n_visible, scores, block_size, block_scores, stream,
                            qfp4);
    return launched(who);
}

static int index_reindex_impl(const char* who, const uint16_t* q_idx, const float* w, const void* k, bool kfp4,
                              int64_t N, int32_t nq, int32_t q_per_seq, const int32_t* n_visible,
                              const int32_t* cand_blocks, int32_t nb, int32_t block_size, float* pool_scores,
                              int32_t* pool_ids, hipStream_t stream, bool qfp4 = false) {
    int rc = check_index_common(who, q_idx, w, k, N, nq, q_per_seq);
    if (rc) return rc;
    if (block_size != 8) return fail(CSA2_EINVAL, "%s: block_size must be 8", who);
    if (nb < 1 || nb > 65536) return fail(CSA2_EINVAL, "%s: nb must be in [1, 65536]", who);
    if (nq > 0 && (!cand_blocks || !pool_scores)) return fail(CSA2_EINVAL, "%s: null pointer", who);
    (void)hipGetLastError();
    csa2::launch_index_reindex(q_idx, w, k, kfp4, N, nq, q_per_seq, n_visible, cand_blocks, nb, pool_scores, pool_ids,
                               stream, qfp4);
    return launched(who);
}

int csa2_index_full(const uint16_t* q_idx, const float* w, const uint16_t* k_idx, int64_t N, int32_t nq,
                    int32_t q_per_seq, const int32_t* n_visible, float* scores, int32_t block_size,
                    float* block_scores, hipStream_t stream) {
    return index_full_impl("csa2_index_full", q_idx, w, k_idx, false, N, nq, q_per_seq, n_visible, scores,
                           block_size, block_scores, stream);
}

int csa2_index_full_fp4k(const uint16_t* q_idx, const float* w, const uint8_t* k_fp4, int64_t N, int32_t nq,
                         int32_t q_per_seq, const int32_t* n_visible, float* scores, int32_t block_size,
                         float* block_scores, hipStream_t stream) {
    return index_full_impl("csa2_index_full_fp4k", q_idx, w, k_fp4, true, N, nq, q_per_seq, n_visible, scores,
                           block_size, block_scores, stream);
}

int csa2_index_reindex(const uint16_t* q_idx, const float* w, const uint16_t* k_idx, int64_t N, int32_t nq,
                       int32_t q_per_seq, const int32_t* n_visible, const int32_t* cand_blocks, int32_t nb,
                       int32_t block_size, float* pool_scores, int32_t* pool_ids, hipStream_t stream) {
    return index_reindex_impl("csa2_index_reindex", q_idx, w, k_idx, false, N, nq, q_per_seq, n_visible, cand_blocks,
                              nb, block_size, pool_scores, pool_ids, stream);
}

int csa2_index_reindex_fp4k(const uint16_t* q_idx, const float* w, const uint8_t* k_fp4, int64_t N, int32_t nq,
                            int32_t q_per_seq, const int32_t* n_visible, const int32_t* cand_blocks, int32_t nb,
                            int32_t block_size, float* pool_scores, int32_t* pool_ids, hipStream_t stream) {
    return index_reindex_impl("csa2_index_reindex_fp4k", q_idx, w, k_fp4, true, N, nq, q_per_seq, n_visible,
                              cand_blocks, nb, block_size, pool_scores, pool_ids, stream);
}

size_t csa2_index_topk_workspace_bytes(int32_t nq, int64_t N, int32_t k) {
    if (nq <= 0 || N < 1 || N > kMaxN || k < 1 || k > CSA2_MAX_TOPK) return 0;
    return csa2::index_topk_workspace_bytes(nq, N, k);
}

// Argument checks of the fused scoring + Top-K calls (everything but the workspace).
static int index_topk_args(const char* who, const uint16_t* q_idx, const float* w, const void* kc, int64_t N,
                           int32_t nq, int32_t k, int32_t* top_idx, int32_t block_size, float* block_scores) {
    int rc = check_index_common(who, q_idx, w, kc, N, nq, 1);
    if (rc) return rc;
    if (k < 1 || k > CSA2_MAX_TOPK) return fail(CSA2_EINVAL, "%s: k must be in [1, %d]", who, CSA2_MAX_TOPK);
    if (!csa2::index_topk_fits(nq, N, k))
        return fail(CSA2_EINVAL, "%s: N too large for this k (use csa2_index_full and csa2_topk)", who);
    if (nq > 0 && !top_idx) return fail(CSA2_EINVAL, "%s: null top_idx", who);
    if (block_size != 0 && block_size != 8) return fail(CSA2_EINVAL, "%s: block_size must be 0 or 8", who);
    if (block_size == 8 && nq > 0 && !block_scores)
        return fail(CSA2_EINVAL, "%s: block_scores required when block_size == 8", who);
    return CSA2_OK;
}

static int index_topk_impl(const char* who, bool merge, const uint16_t* q_idx, const float* w, const void* kc,
                           bool kfp4, int64_t N, int32_t nq, const int32_t* n_visible, int32_t k, int32_t* top_idx,
                           int32_t block_size, float* block_scores, float* scores, void* workspace, size_t ws_bytes,
                           hipStream_t stream, bool qfp4 = false) {
    const int rc = index_topk_args(who, q_idx, w, kc, N, nq, k, top_idx, block_size, block_scores);
    if (rc) return rc;
    const size_t need = csa2_index_topk_workspace_bytes(nq, N, k);
    if (nq > 0 && need > 0 && (!workspace || ws_bytes < need))
        return fail(CSA2_EWORKSPACE, "%s: workspace needs %zu bytes", who, need);
    (void)hipGetLastError();
    csa2::launch_index_topk(q_idx, w, kc, kfp4, N, nq, n_visible, k, top_idx, block_size ? block_scores : nullptr,
                            scores, workspace, stream, qfp4);
    if (merge) csa2::launch_index_topk_merge(N, nq, k, top_idx, workspace, stream);
    return launched(who);
}

int csa2_index_topk(const uint16_t* q_idx, const float* w, const uint16_t* k_idx, int64_t N, int32_t nq,
                    const int32_t* n_visible, int32_t k, int32_t* top_idx, int32_t block_size, float* block_scores,
                    float* scores, void* workspace, size_t ws_bytes, hipStream_t stream) {
    return index_topk_impl("csa2_index_topk", true, q_idx, w, k_idx, false, N, nq, n_visible, k, top_idx,
                           block_size, block_scores, scores, workspace, ws_bytes, stream);
}

int csa2_index_topk_fp4k(const uint16_t* q_idx, const float* w, const uint8_t* k_fp4, int64_t N, int32_t nq,
                         const int32_t* n_visible, int32_t k, int32_t* top_idx, int32_t block_size,
                         float* block_scores, float* scores, void* workspace, size_t ws_bytes, hipStream_t stream) {
    return index_topk_impl("csa2_index_topk_fp4k", true, q_idx, w, k_fp4, true, N, nq, n_visible, k, top_idx,
                           block_size, block_scores, scores, workspace, ws_bytes, stream);
}

int csa2_index_topk_select(const uint16_t* q_idx, const float* w, const void* k, int32_t k_is_fp4, int64_t N,
                           int32_t nq, const int32_t* n_visible, int32_t topk, int32_t* top_idx, int32_t block_size,
                           float* block_scores, float* scores, void* workspace, size_t ws_bytes, hipStream_t stream) {
    return index_topk_impl("csa2_index_topk_select", false, q_idx, w, k, k_is_fp4 != 0, N, nq, n_visible, topk,
                           top_idx, block_size, block_scores, scores, workspace, ws_bytes, stream);
}

size_t csa2_index_topk_noalloc_scratch_bytes(void) { return csa2::index_topk_noalloc_capacity(); }

int csa2_index_topk_noalloc(const uint16_t* q_idx, const float* w, const void* k, int32_t k_is_fp4, int64_t N,
                            int32_t nq, const int32_t* n_visible, int32_t topk, int32_t* top_idx, int32_t block_size,
                            float* block_scores, float* scores, hipStream_t stream) {
    const char* who = "csa2_index_topk_noalloc";
    const int rc = index_topk_args(who, q_idx, w, k, N, nq, topk, top_idx, block_size, block_scores);
    if (rc) return rc;
    const size_t need = csa2_index_topk_workspace_bytes(nq, N, topk);
    const size_t cap = csa2::index_topk_noalloc_capacity();
    if (need > cap)
        return fail(CSA2_EINVAL, "%s: this call needs %zu bytes of scratch; the static scratch holds %zu", who, need,
                    cap);
    void* ws = nullptr;
    if (nq > 0 && need > 0) {
        hipError_t e = hipSuccess;
        ws = csa2::index_topk_noalloc_scratch(&e);
        if (!ws) return fail(CSA2_ELAUNCH, "%s: scratch address lookup failed: %s", who, hipGetErrorString(e));
    }
    (void)hipGetLastError();
    csa2::launch_index_topk(q_idx, w, k, k_is_fp4 != 0, N, nq, n_visible, topk, top_idx,
                            block_size ? block_scores : nullptr, scores, ws, stream);
    csa2::launch_index_topk_merge(N, nq, topk, top_idx, ws, stream);
    return launched(who);
}

int csa2_index_topk_merge(int64_t N, int32_t nq, int32_t k, int32_t* top_idx, void* workspace, size_t ws_bytes,
                          hipStream_t stream) {
    if (nq < 0) return fail(CSA2_EINVAL, "csa2_index_topk_merge: nq < 0");
    if (N < 1 || N > kMaxN) return fail(CSA2_EINVAL, "csa2_index_topk_merge: N must be in [1, 2^31-1]");
    if (k < 1 || k > CSA2_MAX_TOPK)
        return fail(CSA2_EINVAL, "csa2_index_topk_merge: k must be in [1, %d]", CSA2_MAX_TOPK);
    if (!csa2::index_topk_fits(nq, N, k))
        return fail(CSA2_EINVAL, "csa2_index_topk_merge: N too large for this k");
    if (nq > 0 && !top_idx) return fail(CSA2_EINVAL, "csa2_index_topk_merge: null top_idx");
    const size_t need = csa2_index_topk_workspace_bytes(nq, N, k);
    if (nq > 0 && need > 0 && (!workspace || ws_bytes < need))
        return fail(CSA2_EWORKSPACE, "csa2_index_topk_merge: workspace needs %zu bytes", need);
    (void)hipGetLastError();
    csa2::launch_index_topk_merge(N, nq, k, top_idx, workspace, stream);
    return launched("csa2_index_topk_merge");
}

size_t csa2_index_topk_pool_workspace_bytes(int32_t nq, int64_t N, int32_t k, int32_t pool_k) {
    if (nq <= 0 || N < 1 || N > kMaxN || k < 1 || k > CSA2_MAX_TOPK || pool_k < 1 || pool_k > CSA2_MAX_TOPK) return 0;
    if (!csa2::index_topk_fits(nq, N, k)) return 0;
    return csa2::index_topk_pool_workspace_bytes(nq, N, k, pool_k);
}

int csa2_index_topk_merge_pool(int64_t N, int32_t nq, int32_t k, int32_t* top_idx, const float* block_scores,
                               int32_t pool_k, int32_t* cand_blocks, void* workspace, size_t ws_bytes,
                               hipStream_t stream) {
    const char* who = "csa2_index_topk_merge_pool";
    if (nq < 0) return fail(CSA2_EINVAL, "%s: nq < 0", who);
    if (N < 1 || N > kMaxN) return fail(CSA2_EINVAL, "%s: N must be in [1, 2^31-1]", who);
    if (k < 1 || k > CSA2_MAX_TOPK) return fail(CSA2_EINVAL, "%s: k must be in [1, %d]", who, CSA2_MAX_TOPK);
    if (pool_k < 1 || pool_k > CSA2_MAX_TOPK)
        return fail(CSA2_EINVAL, "%s: pool_k must be in [1, %d]", who, CSA2_MAX_TOPK);
    if (!csa2::index_topk_fits(nq, N, k)) return fail(CSA2_EINVAL, "%s: N too large for this k", who);
    if (nq > 0 && (!top_idx || !block_scores || !cand_blocks)) return fail(CSA2_EINVAL, "%s: null pointer", who);
    const size_t need = csa2_index_topk_pool_workspace_bytes(nq, N, k, pool_k);
    if (nq > 0 && need > 0 && (!workspace || ws_bytes < need))
        return fail(CSA2_EWORKSPACE, "%s: workspace needs %zu bytes", who, need);
    (void)hipGetLastError();
    csa2::launch_index_topk_merge_pool(N, nq, k, top_idx, block_scores, pool_k, cand_blocks, workspace, stream);
    return launched(who);
}

size_t csa2_index_prefill_topk_workspace_bytes(int32_t nq, int64_t N, int32_t k) {
    if (nq <= 0 || N < 1 || N > kMaxN || k < 1 || k > CSA2_MAX_TOPK) return 0;
    if (!csa2::prefill_topk_fits(nq, N, k)) return 0;
    return csa2::prefill_topk_workspace_bytes(nq, N, k);
}

static int prefill_topk_impl(const char* who, const uint16_t* q_idx, const float* w, const void* kc, bool kfp4,
                             int64_t N, int32_t nq, int32_t q_per_seq, const int32_t* n_visible, int32_t k,
                             int32_t* top_idx, float* scores, void* workspace, size_t ws_bytes, hipStream_t stream) {
    int rc = check_index_common(who, q_idx, w, kc, N, nq, q_per_seq);
    if (rc) return rc;
    if (q_per_seq % 8 != 0) return fail(CSA2_EINVAL, "%s: q_per_seq must be a multiple of 8", who);
    if (k < 1 || k > 512) return fail(CSA2_EINVAL, "%s: k must be in [1, 512]", who);
    if (!csa2::prefill_topk_fits(nq, N, k))
        return fail(CSA2_EINVAL, "%s: N too large for this k (use csa2_index_full and csa2_topk)", who);
    if (nq > 0 && !top_idx) return fail(CSA2_EINVAL, "%s: null top_idx", who);
    const size_t need = csa2_index_prefill_topk_workspace_bytes(nq, N, k);
    if (nq > 0 && need > 0 && (!workspace || ws_bytes < need))
        return fail(CSA2_EWORKSPACE, "%s: workspace needs %zu bytes", who, need);
    (void)hipGetLastError();
    csa2::launch_index_prefill_topk(q_idx, w, kc, kfp4, N, nq, q_per_seq, n_visible, k, top_idx, scores, workspace,
                                    stream);
    return launched(who);
}

int csa2_index_prefill_topk(const uint16_t* q_idx, const float* w, const uint16_t* k_idx, int64_t N, int32_t nq,
                            int32_t q_per_seq, const int32_t* n_visible, int32_t k, int32_t* top_idx, float* scores,
                            void* workspace, size_t ws_bytes, hipStream_t stream) {
    return prefill_topk_impl("csa2_index_prefill_topk", q_idx, w, k_idx, false, N, nq, q_per_seq, n_visible, k, top_idx,
                             scores, workspace, ws_bytes, stream);
}

int csa2_index_prefill_topk_fp4k(const uint16_t* q_idx, const float* w, const uint8_t* k_fp4, int64_t N, int32_t nq,
                                 int32_t q_per_seq, const int32_t* n_visible, int32_t k, int32_t* top_idx,
                                 float* scores, void* workspace, size_t ws_bytes, hipStream_t stream) {
    return prefill_topk_impl("csa2_index_prefill_topk_fp4k", q_idx, w, k_fp4, true, N, nq, q_per_seq, n_visible, k,
                             top_idx, scores, workspace, ws_bytes, stream);
}

int csa2_index_full_fp4qk(const uint8_t* q_fp4, const float* w, const uint8_t* k_fp4, int64_t N, int32_t nq,
                          int32_t q_per_seq, const int32_t* n_visible, float* scores, int32_t block_size,
                          float* block_scores, hipStream_t stream) {
    return index_full_impl("csa2_index_full_fp4qk", reinterpret_cast<const uint16_t*>(q_fp4), w, k_fp4, true, N, nq,
                           q_per_seq, n_visible, scores, block_size, block_scores, stream, true);
}

int csa2_index_reindex_fp4qk(const uint8_t* q_fp4, const float* w, const uint8_t* k_fp4, int64_t N, int32_t nq,
                             int32_t q_per_seq, const int32_t* n_visible, const int32_t* cand_blocks, int32_t nb,
                             int32_t block_size, float* pool_scores, int32_t* pool_ids, hipStream_t stream) {
    return index_reindex_impl("csa2_index_reindex_fp4qk", reinterpret_cast<const uint16_t*>(q_fp4), w, k_fp4, true, N,
                              nq, q_per_seq, n_visible, cand_blocks, nb, block_size, pool_scores, pool_ids, stream,
                              true);
}

int csa2_index_topk_fp4qk(const uint8_t* q_fp4, const float* w, const uint8_t* k_fp4, int64_t N, int32_t nq,
                          const int32_t* n_visible, int32_t k, int32_t* top_idx, int32_t block_size,
                          float* block_scores, float* scores, void* workspace, size_t ws_bytes, hipStream_t stream) {
    return index_topk_impl("csa2_index_topk_fp4qk", true, reinterpret_cast<const uint16_t*>(q_fp4), w, k_fp4, true, N,
                           nq, n_visible, k, top_idx, block_size, block_scores, scores, workspace, ws_bytes, stream,
                           true);
}

int csa2_index_topk_select_fp4qk(const uint8_t* q_fp4, const float* w, const uint8_t* k_fp4, int64_t N, int32_t nq,
                                 const int32_t* n_visible, int32_t k, int32_t* top_idx, int32_t block_size,
                                 float* block_scores, float* scores, void* workspace, size_t ws_bytes,
                                 hipStream_t stream) {
    return index_topk_impl("csa2_index_topk_select_fp4qk", false, reinterpret_cast<const uint16_t*>(q_fp4), w, k_fp4,
                           true, N, nq, n_visible, k, top_idx, block_size, block_scores, scores, workspace, ws_bytes,
                           stream, true);
}

int csa2_index_prefill_topk_fp4qk(const uint8_t* q_fp4, const float* w, const uint8_t* k_fp4, int64_t N, int32_t nq,
                                  int32_t q_per_seq, const int32_t* n_visible, int32_t k, int32_t* top_idx,
                                  float* scores, void* workspace, size_t ws_bytes, hipStream_t stream) {
    const char* who = "csa2_index_prefill_topk_fp4qk";
    int rc = check_index_common(who, reinterpret_cast<const uint16_t*>(q_fp4), w, k_fp4, N, nq, q_per_seq);
    if (rc) return rc;
    if (q_per_seq % 8 != 0) return fail(CSA2_EINVAL, "%s: q_per_seq must be a multiple of 8", who);
    if (k < 1 || k > 512) return fail(CSA2_EINVAL, "%s: k must be in [1, 512]", who);
    if (!csa2::prefill_topk_fits(nq, N, k))
        return fail(CSA2_EINVAL, "%s: N too large for this k (use csa2_index_full_fp4qk and csa2_topk)", who);
    if (nq > 0 && !top_idx) return fail(CSA2_EINVAL, "%s: null top_idx", who);
    const size_t need = csa2_index_prefill_topk_workspace_bytes(nq, N, k);
    if (nq > 0 && need > 0 && (!workspace || ws_bytes < need))
        return fail(CSA2_EWORKSPACE, "%s: workspace needs %zu bytes", who, need);
    (void)hipGetLastError();
    csa2::launch_index_prefill_topk_fp4qk(q_fp4, w, k_fp4, N, nq, q_per_seq, n_visible, k, top_idx, scores, workspace,
                                          stream);
    return launched(who);
}

size_t csa2_index_reindex_topk_workspace_bytes(int32_t nq, int32_t nb, int32_t k) {
    if (nq <= 0 || nb < 1 || nb > 65536 || k < 1 || k > CSA2_MAX_TOPK) return 0;
    return csa2::reindex_topk_workspace_bytes(nq, nb, k);
}

static int reindex_topk_impl(const char* who, const uint16_t* q_idx, const float* w, const void* kc, bool kfp4,
                             int64_t N, int32_t nq, int32_t q_per_seq, const int32_t* n_visible,
                             const int32_t* cand_blocks, int32_t nb, int32_t k, int32_t* top_idx, float* pool_scores,
                             void* workspace, size_t ws_bytes, hipStream_t stream, bool qfp4 = false) {
    int rc = check_index_common(who, q_idx, w, kc, N, nq, q_per_seq);
    if (rc) return rc;
    if (nb < 1 || nb > 65536) return fail(CSA2_EINVAL, "%s: nb must be in [1, 65536]", who);
    if (k < 1 || k > CSA2_MAX_TOPK) return fail(CSA2_EINVAL, "%s: k must be in [1, %d]", who, CSA2_MAX_TOPK);
    if (!csa2::reindex_topk_fits(nq, nb, k)) return fail(CSA2_EINVAL, "%s: pool too large for this k", who);
    if (nq > 0 && (!cand_blocks || !top_idx)) return fail(CSA2_EINVAL, "%s: null pointer", who);
    const size_t need = csa2_index_reindex_topk_workspace_bytes(nq, nb, k);
    if (nq > 0 && need > 0 && (!workspace || ws_bytes < need))
        return fail(CSA2_EWORKSPACE, "%s: workspace needs %zu bytes", who, need);
    (void)hipGetLastError();
    csa2::launch_index_reindex_topk(q_idx, w, kc, kfp4, N, nq, q_per_seq, n_visible, cand_blocks, nb, k, top_idx,
                                    pool_scores, workspace, stream, qfp4);
    return launched(who);
}

int csa2_index_reindex_topk(const uint16_t* q_idx, const float* w, const uint16_t* k_idx, int64_t N, int32_t nq,
                            int32_t q_per_seq, const int32_t* n_visible, const int32_t* cand_blocks, int32_t nb,
                            int32_t k, int32_t* top_idx, float* pool_scores, void* workspace, size_t ws_bytes,
                            hipStream_t stream) {
    return reindex_topk_impl("csa2_index_reindex_topk", q_idx, w, k_idx, false, N, nq, q_per_seq, n_visible,
                             cand_blocks, nb, k, top_idx, pool_scores, workspace, ws_bytes, stream);
}

int csa2_index_reindex_topk_fp4k(const uint16_t* q_idx, const float* w, const uint8_t* k_fp4, int64_t N, int32_t nq,
                                 int32_t q_per_seq, const int32_t* n_visible, const int32_t* cand_blocks, int32_t nb,
                                 int32_t k, int32_t* top_idx, float* pool_scores, void* workspace, size_t ws_bytes,
                                 hipStream_t stream) {
    return reindex_topk_impl("csa2_index_reindex_topk_fp4k", q_idx, w, k_fp4, true, N, nq, q_per_seq, n_visible,
                             cand_blocks, nb, k, top_idx, pool_scores, workspace, ws_bytes, stream);
}

int csa2_index_reindex_topk_fp4qk(const uint8_t* q_fp4, const float* w, const uint8_t* k_fp4, int64_t N, int32_t nq,
                                  int32_t q_per_seq, const int32_t* n_visible, const int32_t* cand_blocks, int32_t nb,
                                  int32_t k, int32_t* top_idx, float* pool_scores, void* workspace, size_t ws_bytes,
                                  hipStream_t stream) {
    return reindex_topk_impl("csa2_index_reindex_topk_fp4qk", reinterpret_cast<const uint16_t*>(q_fp4), w, k_fp4,
                             true, N, nq, q_per_seq, n_visible, cand_blocks, nb, k, top_idx, pool_scores, workspace,
                             ws_bytes, stream, true);
}

int kidx_fp4_pack(const uint16_t* x_bf16, int64_t n, uint8_t* out, hipStream_t stream) {
    if (n < 0) return fail(CSA2_EINVAL, "kidx_fp4_pack: n < 0");
    if (n > 0 && (!x_bf16 || !out)) return fail(CSA2_EINVAL, "kidx_fp4_pack: null pointer");
    (void)hipGetLastError();
    csa2::launch_kidx_fp4_pack(x_bf16, n, out, stream);
    return launched("kidx_fp4_pack");
}

size_t csa2_topk_workspace_bytes(int32_t rows, int64_t ncols, int32_t k) {
    if (rows <= 0 || ncols <= 0 || k < 1 || k > CSA2_MAX_TOPK) return 0;
    return csa2::topk_workspace_bytes(rows, ncols, k);
}

int csa2_topk(const float* scores, int32_t rows, int64_t ncols, int64_t ld, const int32_t* row_len, int32_t k,
              const int32_t* id_map, int32_t* out_idx, void* workspace, size_t ws_bytes, hipStream_t stream) {
    if (rows < 0) return fail(CSA2_EINVAL, "csa2_topk: rows < 0");
    if (ncols < 1 || ncols > kMaxN) return fail(CSA2_EINVAL, "csa2_topk: ncols must be in [1, 2^31-1]");
    if (ld < ncols) return fail(CSA2_EINVAL, "csa2_topk: ld < ncols");
    if (k < 1 || k > CSA2_MAX_TOPK) return fail(CSA2_EINVAL, "csa2_topk: k must be in [1, %d]", CSA2_MAX_TOPK);
    if (rows > 0 && (!scores || !out_idx)) return fail(CSA2_EINVAL, "csa2_topk: null pointer");
    const size_t need = csa2_topk_workspace_bytes(rows, ncols, k);
    if (rows > 0 && need > 0 && (!workspace || ws_bytes < need))
        return fail(CSA2_EWORKSPACE, "csa2_topk: workspace needs %zu bytes", need);
    (void)hipGetLastError();
    csa2::launch_topk(scores, rows, ncols, ld, row_len, k, id_map, out_idx, workspace, stream);
    return launched("csa2_topk");
}

size_t csa2_sparse_attn_workspace_bytes(int32_t nq, int32_t k) {
    if (nq <= 0 || k < 0 || k > CSA2_MAX_TOPK) return 0;
    return csa2::attn_workspace_bytes(nq, k);
}

static int sparse_attn_impl(const char* fn, const uint16_t* q, const uint8_t* kv, int64_t N, int32_t nq,
                            int32_t q_per_seq, const int32_t* idx, int32_t k, const void* swa, bool swa_fp8, int64_t T,
                            const int32_t* swa_start, const int32_t* swa_len, float softmax_scale, uint16_t* out,
                            float* lse, void* workspace, size_t ws_bytes, hipStream_t stream) {
    if (nq < 0) return fail(CSA2_EINVAL, "%s: nq < 0", fn);
    if (N < 1 || N > kMaxN) return fail(CSA2_EINVAL, "%s: N must be in [1, 2^31-1]", fn);
    if (q_per_seq < 1 || nq % q_per_seq != 0) return fail(CSA2_EINVAL, "%s: q_per_seq must be >= 1 and divide nq", fn);
    if (k < 0 || k > CSA2_MAX_TOPK) return fail(CSA2_EINVAL, "%s: k must be in [0, %d]", fn, CSA2_MAX_TOPK);
    if (nq > 0 && (!q || !kv || !out)) return fail(CSA2_EINVAL, "%s: null pointer", fn);
    if (nq > 0 && k > 0 && !idx) return fail(CSA2_EINVAL, "%s: null idx", fn);
    if (swa && (T < 1 || !swa_start || !swa_len))
        return fail(CSA2_EINVAL, "%s: a window needs T >= 1, swa_start and swa_len", fn);
    if (!(softmax_scale == softmax_scale)) return fail(CSA2_EINVAL, "%s: softmax_scale is NaN", fn);
    const size_t need = csa2_sparse_attn_workspace_bytes(nq, k);
    if (nq > 0 && need > 0 && (!workspace || ws_bytes < need))
        return fail(CSA2_EWORKSPACE, "%s: workspace needs %zu bytes", fn, need);
    (void)hipGetLastError();
    csa2::launch_sparse_attn(q, kv, N, nq, q_per_seq, idx, k, swa, swa_fp8, swa ? T : 0, swa ? swa_start : nullptr,
                             swa ? swa_len : nullptr, softmax_scale, out, lse, workspace, stream);
    return launched(fn);
}

int csa2_sparse_attn(const uint16_t* q, const uint8_t* kv, int64_t N, int32_t nq, int32_t q_per_seq,
                     const int32_t* idx, int32_t k, const uint16_t* swa, int64_t T, const int32_t* swa_start,
                     const int32_t* swa_len, float softmax_scale, uint16_t* out, float* lse, void* workspace,
                     size_t ws_bytes, hipStream_t stream) {
    return sparse_attn_impl("csa2_sparse_attn", q, kv, N, nq, q_per_seq, idx, k, swa, false, T, swa_start, swa_len,
                            softmax_scale, out, lse, workspace, ws_bytes, stream);
}

int csa2_sparse_attn_fp8w(const uint16_t* q, const uint8_t* kv, int64_t N, int32_t nq, int32_t q_per_seq,
                          const int32_t* idx, int32_t k, const uint8_t* swa_fp8, int64_t T, const int32_t* swa_start,
                          const int32_t* swa_len, float softmax_scale, uint16_t* out, float* lse, void* workspace,
                          size_t ws_bytes, hipStream_t stream) {
    return sparse_attn_impl("csa2_sparse_attn_fp8w", q, kv, N, nq, q_per_seq, idx, k, swa_fp8, true, T, swa_start,
                            swa_len, softmax_scale, out, lse, workspace, ws_bytes, stream);
}

int swa_fp8_pack(const uint16_t* x, int64_t n, uint8_t* out, hipStream_t stream) {
    if (n < 0) return fail(CSA2_EINVAL, "swa_fp8_pack: n < 0");
    if (n > 0 && (!x || !out)) return fail(CSA2_EINVAL, "swa_fp8_pack: null pointer");
    (void)hipGetLastError();
    csa2::launch_swa_fp8_pack(x, n, out, stream);
    return launched("swa_fp8_pack");
}

}  // extern "C"
