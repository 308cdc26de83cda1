// Per-row Top-K (titansim blog, CSA2 modes: each Full / Reindex layer keeps its
// Top-512 entries; eogee.com report 3.3: the Full layer keeps the best 2048
// blocks). Exact selection under the order (score desc, column asc).
//
// Scores map to order-preserving 32-bit keys (larger key = larger score, -0
// folded onto +0, -inf and NaN to key 0 = never chosen). A workgroup finds the
// exact k-th largest key T with an MSB radix select over LDS histograms (a
// 12-bit first digit; the few keys of T's bin are then resolved by one wave,
// or by two more digits when the bin is crowded), then emits every key > T
// plus the lowest-column ties == T, in column order -- so the output is
// already ascending.
//
// Long rows are split: stage 1 selects the top-k of each chunk as (key,
// column) candidates; stage 2 selects the row's top-k among the candidates.
// A row's top-k entry is in its chunk's top-k (fewer than k chunk entries can
// beat it), so the two stages give the same set as one pass.
//
// Main path: each thread of a 256- to 1024-thread workgroup holds a
// contiguous run of up to 32 keys (chunks <= 32768 keys, merges <= 16384
// candidates) in registers, so the radix passes read no memory; the chunk
// keys arrive with coalesced loads through LDS. Wave scans use DPP, and the
// ordered emission is one packed block scan of per-thread counts followed by
// an LDS-staged, coalesced write. Every select's first digit starts at the
// highest bit where the segment's keys differ, since score rows and merged
// candidates sit in narrow bands. Shapes beyond those capacities take the
// global-memory path (512 threads, every pass re-reads the scores through
// the caches). Each register-path launch is described by a job (chunk
// select, final merge, group merge); two independent selections whose jobs
// take the same shape share one launch (the hierarchical Full layer's Top-K
// merge and its pool's block selection).
#include <math.h>

#include "device_common.h"
#include "launch.h"
#include "topk_select.h"

namespace csa2 {

namespace {

constexpr int kTkThreads = 512;
constexpr int kTkWaves = kTkThreads / 64;
constexpr int kHistBins = 2048;

using tk::score_key;

struct TkShared {
    uint32_t hist[kHistBins];
    uint32_t wsum[kTkWaves];
    uint32_t wsum2[kTkWaves];
    uint32_t sel_bin;
    uint32_t sel_above;
    uint32_t total;
};

// Exclusive block scan of one value per thread; returns the block total in *total.
CSA2_DEVINL uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < kTkWaves; i++) {
        const uint32_t s = wsum[i];
        before += (i < wave) ? s : 0u;
        tot += s;
    }
    __syncthreads();
    *total = tot;
    return before + x - v;
}

// Key source: element i of the current row/segment.
struct ScoreSrc {
    const float* row;
    int64_t n;
    CSA2_DEVINL uint32_t key(int64_t i) const { return score_key(row[i]); }
};
struct CandSrc {
    const uint32_t* keys;
    CSA2_DEVINL uint32_t key(int64_t i) const { return keys[i]; }
};

// Radix select over n keys: on return *T is the k-th largest key among the
// selectable ones and *need the number of keys == T to take (lowest first);
// *kq = min(k, #selectable). kq == 0 leaves T = 0xFFFFFFFF.
template <class Src>
CSA2_DEVINL void radix_select(const Src& src, int64_t n, int32_t k, TkShared& sh, uint32_t* T, uint32_t* need,
                              uint32_t* kq) {
    const int tid = threadIdx.x;
    for (int i = tid; i < kHistBins; i += kTkThreads) sh.hist[i] = 0;
    __syncthreads();
    uint32_t cnt = 0;
    uint32_t last_bin = 0xFFFFFFFFu, run = 0;
    for (int64_t i = tid; i < n; i += kTkThreads) {
        const uint32_t key = src.key(i);
        if (key) {
            cnt++;
            const uint32_t bin = key >> 21;
            if (bin == last_bin) {
                run++;
            } else {
                if (run) atomicAdd(&sh.hist[last_bin], run);
                last_bin = bin;
                run = 1;
            }
        }
    }
    if (run) atomicAdd(&sh.hist[last_bin], run);
    uint32_t total;
    block_excl_scan(cnt, sh.wsum, &total);
    const uint32_t kk = total < (uint32_t)k ? total : (uint32_t)k;
    *kq = kk;
    if (kk == 0) {
        *T = 0xFFFFFFFFu;
        *need = 0;
        return;
    }
    uint32_t prefix = 0, rem = kk;
    const int shifts[3] = {21, 10, 0};
    const int bits[3] = {11, 11, 10};
    for (int p = 0; p < 3; p++) {
        const int sh_ = shifts[p];
        const uint32_t nbins = 1u << bits[p];
        if (p > 0) {
            for (int i = tid; i < kHistBins; i += kTkThreads) sh.hist[i] = 0;
            __syncthreads();
            const int hi_shift = sh_ + bits[p];
            last_bin = 0xFFFFFFFFu;
            run = 0;
            for (int64_t i = tid; i < n; i += kTkThreads) {
                const uint32_t key = src.key(i);
                if (key && (key >> hi_shift) == prefix) {
                    const uint32_t bin = (key >> sh_) & (nbins - 1);
                    if (bin == last_bin) {
                        run++;
                    } else {
                        if (run) atomicAdd(&sh.hist[last_bin], run);
                        last_bin = bin;
                        run = 1;
                    }
                }
            }
            if (run) atomicAdd(&sh.hist[last_bin], run);
        }
        __syncthreads();
        // Scan bins from the top: thread t owns bins nbins-1-4t .. nbins-4-4t.
        uint32_t c4[4], loc = 0;
        const int per = (int)(nbins / kTkThreads);  // 4 or 2
#pragma unroll
        for (int j = 0; j < 4; j++) {
            c4[j] = (j < per) ? sh.hist[nbins - 1 - (tid * per + j)] : 0u;
            loc += c4[j];
        }
        uint32_t tot2;
        uint32_t above = block_excl_scan(loc, sh.wsum2, &tot2);
        if (above < rem && rem <= above + loc) {
            for (int j = 0; j < per; j++) {
                if (above + c4[j] >= rem) {
                    sh.sel_bin = nbins - 1 - (tid * per + j);
                    sh.sel_above = above;
                    break;
                }
                above += c4[j];
            }
        }
        __syncthreads();
        prefix = (prefix << bits[p]) | sh.sel_bin;
        rem -= sh.sel_above;
        __syncthreads();
    }
    *T = prefix;
    *need = rem;
}

// Emits the selected elements of [0, n) in index order via `emit(slot, i, key)`;
// returns kq (number emitted). Each thread owns a contiguous index range.
template <class Src, class Emit>
CSA2_DEVINL uint32_t select_and_emit(const Src& src, int64_t n, int32_t k, TkShared& sh, Emit emit) {
    uint32_t T, need, kq;
    radix_select(src, n, k, sh, &T, &need, &kq);
    if (kq == 0) return 0;
    const int tid = threadIdx.x;
    const int64_t per = (n + kTkThreads - 1) / kTkThreads;
    const int64_t i0 = (int64_t)tid * per;
    const int64_t i1 = (i0 + per < n) ? i0 + per : n;
    uint32_t gt = 0, eq = 0;
    for (int64_t i = i0; i < i1; i++) {
        const uint32_t key = src.key(i);
        gt += key > T;
        eq += key == T;
    }
    uint32_t tot;
    const uint32_t eq_before = block_excl_scan(eq, sh.wsum, &tot);
    uint32_t take = need > eq_before ? need - eq_before : 0u;
    take = take < eq ? take : eq;
    uint32_t slot = block_excl_scan(gt + take, sh.wsum2, &tot);
    for (int64_t i = i0; i < i1; i++) {
        const uint32_t key = src.key(i);
        if (key > T || (key == T && take > 0)) {
            if (key == T) take--;
            emit(slot, i, key);
            slot++;
        }
    }
    return kq;
}

// Stage 1 (or the only stage): one workgroup per (row, chunk).
__global__ __launch_bounds__(kTkThreads) void topk_chunk_kernel(const float* __restrict__ scores, int64_t ncols,
                                                                int64_t ld, const int32_t* __restrict__ row_len,
                                                                int32_t k, int32_t nchunks, int64_t chunk_len,
                                                                const int32_t* __restrict__ id_map,
                                                                int32_t* __restrict__ out_idx,
                                                                uint32_t* __restrict__ cand_key,
                                                                int32_t* __restrict__ cand_col) {
    __shared__ TkShared sh;
    const int64_t row = blockIdx.x / nchunks;
    const int64_t chunk = blockIdx.x % nchunks;
    int64_t len = row_len ? (int64_t)row_len[row] : ncols;
    len = len < ncols ? len : ncols;
    len = len > 0 ? len : 0;
    const int64_t c0 = chunk * chunk_len;
    int64_t n = len - c0;
    n = n < chunk_len ? n : chunk_len;
    n = n > 0 ? n : 0;
    ScoreSrc src{scores + row * ld + c0, n};
    if (nchunks == 1) {
        int32_t* out = out_idx + row * k;
        const int32_t* map = id_map ? id_map + row * ld : nullptr;
        const uint32_t kq = select_and_emit(src, n, k, sh, [&](uint32_t slot, int64_t i, uint32_t) {
            out[slot] = map ? map[i] : (int32_t)i;
        });
        for (int64_t t = (int64_t)kq + threadIdx.x; t < k; t += kTkThreads) out[t] = -1;
    } else {
        uint32_t* ck = cand_key + (row * nchunks + chunk) * k;
        int32_t* cc = cand_col + (row * nchunks + chunk) * k;
        const uint32_t kq = select_and_emit(src, n, k, sh, [&](uint32_t slot, int64_t i, uint32_t key) {
            ck[slot] = key;
            cc[slot] = (int32_t)(c0 + i);
        });
        for (int64_t t = (int64_t)kq + threadIdx.x; t < k; t += kTkThreads) {
            ck[t] = 0u;
            cc[t] = -1;
        }
    }
}

// Stage 2: one workgroup per row over its nchunks * k candidates (in column order).
__global__ __launch_bounds__(kTkThreads) void topk_merge_kernel(int64_t ld, int32_t k, int32_t nchunks,
                                                                const int32_t* __restrict__ id_map,
                                                                const uint32_t* __restrict__ cand_key,
                                                                const int32_t* __restrict__ cand_col,
                                                                int32_t* __restrict__ out_idx) {
    __shared__ TkShared sh;
    const int64_t row = blockIdx.x;
    const int64_t n = (int64_t)nchunks * k;
    const uint32_t* ck = cand_key + row * n;
    const int32_t* cc = cand_col + row * n;
    int32_t* out = out_idx + row * k;
    const int32_t* map = id_map ? id_map + row * ld : nullptr;
    CandSrc src{ck};
    const uint32_t kq = select_and_emit(src, n, k, sh, [&](uint32_t slot, int64_t i, uint32_t) {
        const int32_t col = cc[i];
        out[slot] = map ? map[col] : col;
    });
    for (int64_t t = (int64_t)kq + threadIdx.x; t < k; t += kTkThreads) out[t] = -1;
}

// ------------------------------------------------------------- register path

using tk::RegTk;
using tk::reg_select_emit;
using tk::kRegMaxKpt;
using tk::kRegMaxKeys;
using tk::kRegMaxCand;

// Loads KPT consecutive scores of this thread (positions tid*KPT..) as keys;
// positions >= n give key 0.
template <int KPT>
CSA2_DEVINL void load_keys(const float* src, int n, uint32_t (&key)[KPT]) {
    const int p0 = threadIdx.x * KPT;
    if ((KPT % 4) == 0 && (reinterpret_cast<uintptr_t>(src) & 15u) == 0 && p0 + KPT <= n) {
        const float4* v = reinterpret_cast<const float4*>(src + p0);
#pragma unroll
        for (int u = 0; u < KPT / 4; u++) {
            const float4 f = v[u];
            key[4 * u + 0] = score_key(f.x);
            key[4 * u + 1] = score_key(f.y);
            key[4 * u + 2] = score_key(f.z);
            key[4 * u + 3] = score_key(f.w);
        }
    } else {
#pragma unroll
        for (int u = 0; u < KPT; u++) key[u] = (p0 + u < n) ? score_key(src[p0 + u]) : 0u;
    }
}

// The same keys with coalesced loads: thread t loads float4 number j*NT + t
// (positions 4(j*NT + t) .. +3, 16-byte lanes along the row) and the keys go
// through LDS in two halves to come back as each thread's run of KPT
// consecutive positions. stage holds NT*KPT/2 words; a barrier follows.
template <int NT, int KPT>
CSA2_DEVINL void load_keys_coalesced(const float* src, int n, uint32_t (&key)[KPT], uint32_t* stage) {
    static_assert(KPT % 8 == 0, "two halves of whole float4 loads per thread");
    constexpr int kJ = KPT / 4;            // float4 loads per thread
    constexpr int kHalf = NT * KPT / 2;    // positions per half
    const int tid = threadIdx.x;
    const bool vec = (reinterpret_cast<uintptr_t>(src) & 15u) == 0;
    uint4 v[kJ];
#pragma unroll
    for (int j = 0; j < kJ; j++) {
        const int p = 4 * (j * NT + tid);
        float4 f;
        if (vec && p + 4 <= n) {
            f = *reinterpret_cast<const float4*>(src + p);
        } else {
            f.x = p + 0 < n ? src[p + 0] : -INFINITY;
            f.y = p + 1 < n ? src[p + 1] : -INFINITY;
            f.z = p + 2 < n ? src[p + 2] : -INFINITY;
            f.w = p + 3 < n ? src[p + 3] : -INFINITY;
        }
        v[j] = make_uint4(score_key(f.x), score_key(f.y), score_key(f.z), score_key(f.w));
    }
#pragma unroll
    for (int h = 0; h < 2; h++) {
#pragma unroll
        for (int j = h * kJ / 2; j < (h + 1) * kJ / 2; j++)
            *reinterpret_cast<uint4*>(stage + 4 * (j * NT + tid) - h * kHalf) = v[j];
        lds_barrier();
        if (tid / (NT / 2) == h) {
            const uint32_t* run = stage + (tid - h * (NT / 2)) * KPT;
#pragma unroll
            for (int u = 0; u < KPT; u += 4) {
                const uint4 w = *reinterpret_cast<const uint4*>(run + u);
                key[u] = w.x;
                key[u + 1] = w.y;
                key[u + 2] = w.z;
                key[u + 3] = w.w;
            }
        }
        lds_barrier();
    }
}

// One selection of a register-path launch, as plain values: the kernels below
// take it by value, and the paired kernel takes two and tells them apart by
// workgroup index.
enum : int32_t {
    kJobChunk = 0,  // Top-k of each (row, chunk) of a float score matrix
    kJobMerge = 1,  // Top-k of each row's nchunks x k candidates -> final ids
    kJobGroup = 2,  // Top-k of each group of cpg chunks' candidates -> candidates
};
struct TkJob {
    int32_t mode = kJobChunk;
    int32_t nblocks = 0;              // workgroups of the job
    const float* scores = nullptr;    // kJobChunk: rows x ld scores
    int64_t ncols = 0, ld = 0;
    const int32_t* row_len = nullptr;
    int64_t chunk_len = 0;
    const int32_t* id_map = nullptr;  // final ids are mapped through id_map[row * ld + col]
    const uint32_t* ck_in = nullptr;  // merges: candidate keys and columns in
    const int32_t* cc_in = nullptr;
    int32_t nchunks = 1;              // chunks per row (of the scores, or of the input candidates)
    int32_t cpg = 1;                  // kJobGroup: input chunks per group
    int32_t k = 0;
    int32_t* out_idx = nullptr;       // final ids [rows][k]
    uint32_t* ck_out = nullptr;       // candidates out (kJobChunk with nchunks > 1, kJobGroup)
    int32_t* cc_out = nullptr;
};

// LDS of a register-path workgroup: the selection's state, which first stages
// half of a chunk's keys when they are loaded coalesced.
template <int NT, int KPT>
constexpr size_t reg_smem_bytes() {
    constexpr size_t stage = (KPT % 8 == 0) ? (size_t)NT * KPT / 2 * sizeof(uint32_t) : 0;
    return sizeof(RegTk<NT>) > stage ? sizeof(RegTk<NT>) : stage;
}

// kJobChunk, workgroup `bid` = (row, chunk): the chunk's keys in registers.
template <int NT, int KPT>
CSA2_DEVINL void reg_chunk_body(const TkJob& j, int64_t bid, uint8_t* smem) {
    RegTk<NT>& sh = *reinterpret_cast<RegTk<NT>*>(smem);
    const int tid = threadIdx.x;
    const int64_t row = bid / j.nchunks;
    const int64_t chunk = bid % j.nchunks;
    int64_t len = j.row_len ? (int64_t)j.row_len[row] : j.ncols;
    len = len < j.ncols ? len : j.ncols;
    len = len > 0 ? len : 0;
    const int64_t c0 = chunk * j.chunk_len;
    int64_t nn = len - c0;
    nn = nn < j.chunk_len ? nn : j.chunk_len;
    const int n = nn > 0 ? (int)nn : 0;
    const int32_t k = j.k;
    uint32_t key[KPT];
    if constexpr (KPT % 8 == 0)
        load_keys_coalesced<NT, KPT>(j.scores + row * j.ld + c0, n, key, reinterpret_cast<uint32_t*>(smem));
    else
        load_keys<KPT>(j.scores + row * j.ld + c0, n, key);
    const int p0 = tid * KPT;
    uint32_t emitted;
    if (j.nchunks == 1) {
        int32_t* out = j.out_idx + row * k;
        const int32_t* map = j.id_map ? j.id_map + row * j.ld : nullptr;
        emitted = reg_select_emit<NT, KPT, true>(
            key, (uint32_t)k, sh, [&](int u) { return (int32_t)(c0 + p0 + u); },
            [&](uint32_t slot, uint32_t, int32_t col) { out[slot] = map ? map[col] : col; });
        for (int t = (int)emitted + tid; t < k; t += NT) out[t] = -1;
    } else {
        uint32_t* ck = j.ck_out + (row * j.nchunks + chunk) * k;
        int32_t* cc = j.cc_out + (row * j.nchunks + chunk) * k;
        emitted = reg_select_emit<NT, KPT, true>(
            key, (uint32_t)k, sh, [&](int u) { return (int32_t)(c0 + p0 + u); },
            [&](uint32_t slot, uint32_t kv, int32_t col) {
                ck[slot] = kv;
                cc[slot] = col;
            });
        for (int t = (int)emitted + tid; t < k; t += NT) {
            ck[t] = 0u;
            cc[t] = -1;
        }
    }
}

// Loads candidates [base, base + n) as this thread's KPT consecutive (key,
// column) pairs; positions >= n give key 0.
template <int KPT>
CSA2_DEVINL void load_cands(const uint32_t* ckr, const int32_t* ccr, int n, uint32_t (&key)[KPT],
                            int32_t (&col)[KPT]) {
    const int p0 = threadIdx.x * KPT;
    const bool aligned = ((reinterpret_cast<uintptr_t>(ckr) | reinterpret_cast<uintptr_t>(ccr)) & 15u) == 0;
    if ((KPT % 4) == 0 && aligned && p0 + KPT <= n) {
#pragma unroll
        for (int u = 0; u < KPT / 4; u++) {
            const uint4 kv4 = reinterpret_cast<const uint4*>(ckr + p0)[u];
            const int4 cv4 = reinterpret_cast<const int4*>(ccr + p0)[u];
            key[4 * u + 0] = kv4.x;
            key[4 * u + 1] = kv4.y;
            key[4 * u + 2] = kv4.z;
            key[4 * u + 3] = kv4.w;
            col[4 * u + 0] = cv4.x;
            col[4 * u + 1] = cv4.y;
            col[4 * u + 2] = cv4.z;
            col[4 * u + 3] = cv4.w;
        }
    } else {
#pragma unroll
        for (int u = 0; u < KPT; u++) {
            key[u] = (p0 + u < n) ? ckr[p0 + u] : 0u;
            col[u] = (p0 + u < n) ? ccr[p0 + u] : -1;
        }
    }
}

// kJobMerge, workgroup `bid` = row: the row's nchunks * k candidates, which
// are in column order (chunk by chunk, each chunk's selection ascending;
// unused slots hold key 0).
template <int NT, int KPT>
CSA2_DEVINL void reg_merge_body(const TkJob& j, int64_t bid, uint8_t* smem) {
    RegTk<NT>& sh = *reinterpret_cast<RegTk<NT>*>(smem);
    const int tid = threadIdx.x;
    const int64_t row = bid;
    const int32_t k = j.k;
    const int n = j.nchunks * k;
    uint32_t key[KPT];
    int32_t col[KPT];
    load_cands<KPT>(j.ck_in + row * (int64_t)n, j.cc_in + row * (int64_t)n, n, key, col);
    int32_t* out = j.out_idx + row * k;
    const int32_t* map = j.id_map ? j.id_map + row * j.ld : nullptr;
    const uint32_t emitted = reg_select_emit<NT, KPT, true>(
        key, (uint32_t)k, sh, [&](int u) { return col[u]; },
        [&](uint32_t slot, uint32_t, int32_t c) { out[slot] = map ? map[c] : c; });
    for (int t = (int)emitted + tid; t < k; t += NT) out[t] = -1;
}

// kJobGroup, workgroup `bid` = (row, g): the top-k of chunks [g*cpg,
// min((g+1)*cpg, nchunks)) of the row's candidates, written as k candidates
// of group g (column order kept; unused slots key 0, column -1).
template <int NT, int KPT>
CSA2_DEVINL void reg_group_body(const TkJob& j, int64_t bid, uint8_t* smem) {
    RegTk<NT>& sh = *reinterpret_cast<RegTk<NT>*>(smem);
    const int tid = threadIdx.x;
    const int32_t k = j.k;
    const int ngroups = (j.nchunks + j.cpg - 1) / j.cpg;
    const int64_t row = bid / ngroups;
    const int g = (int)(bid % ngroups);
    const int c_end = (g + 1) * j.cpg < j.nchunks ? (g + 1) * j.cpg : j.nchunks;
    const int n = (c_end - g * j.cpg) * k;
    const int64_t base = (row * j.nchunks + (int64_t)g * j.cpg) * k;
    uint32_t key[KPT];
    int32_t col[KPT];
    load_cands<KPT>(j.ck_in + base, j.cc_in + base, n, key, col);
    uint32_t* ok = j.ck_out + (row * ngroups + g) * (int64_t)k;
    int32_t* oc = j.cc_out + (row * ngroups + g) * (int64_t)k;
    const uint32_t emitted = reg_select_emit<NT, KPT, true>(
        key, (uint32_t)k, sh, [&](int u) { return col[u]; },
        [&](uint32_t slot, uint32_t kv, int32_t c) {
            ok[slot] = kv;
            oc[slot] = c;
        });
    for (int t = (int)emitted + tid; t < k; t += NT) {
        ok[t] = 0u;
        oc[t] = -1;
    }
}

template <int NT, int KPT>
__global__ __launch_bounds__(NT) void topk_reg_chunk_kernel(TkJob j) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[reg_smem_bytes<NT, KPT>()];
    reg_chunk_body<NT, KPT>(j, blockIdx.x, smem);
}
template <int NT, int KPT>
__global__ __launch_bounds__(NT) void topk_reg_merge_kernel(TkJob j) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[sizeof(RegTk<NT>)];
    reg_merge_body<NT, KPT>(j, blockIdx.x, smem);
}
template <int NT, int KPT>
__global__ __launch_bounds__(NT) void topk_reg_group_merge_kernel(TkJob j) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[sizeof(RegTk<NT>)];
    reg_group_body<NT, KPT>(j, blockIdx.x, smem);
}

// Any job on 1024 threads with one inlined selection: the mode only decides
// where the keys come from and where the selected ones go, so the select code
// (the bulk of a kernel's instructions) is not repeated per mode.
template <int KPT>
CSA2_DEVINL void reg_any_body(const TkJob& j, int64_t bid, uint8_t* smem) {
    constexpr int NT = 1024;
    RegTk<NT>& sh = *reinterpret_cast<RegTk<NT>*>(smem);
    const int tid = threadIdx.x;
    const int32_t k = j.k;
    uint32_t key[KPT];
    int32_t col[KPT];
    int32_t* out = nullptr;         // final ids (else candidates to ok / oc)
    const int32_t* map = nullptr;
    uint32_t* ok = nullptr;
    int32_t* oc = nullptr;
    if (j.mode == kJobChunk) {
        const int64_t row = bid / j.nchunks, chunk = bid % j.nchunks;
        int64_t len = j.row_len ? (int64_t)j.row_len[row] : j.ncols;
        len = len < j.ncols ? len : j.ncols;
        len = len > 0 ? len : 0;
        const int64_t c0 = chunk * j.chunk_len;
        int64_t nn = len - c0;
        nn = nn < j.chunk_len ? nn : j.chunk_len;
        const int n = nn > 0 ? (int)nn : 0;
        if constexpr (KPT % 8 == 0)
            load_keys_coalesced<NT, KPT>(j.scores + row * j.ld + c0, n, key, reinterpret_cast<uint32_t*>(smem));
        else
            load_keys<KPT>(j.scores + row * j.ld + c0, n, key);
#pragma unroll
        for (int u = 0; u < KPT; u++) col[u] = (int32_t)(c0 + tid * KPT + u);
        if (j.nchunks == 1) {
            out = j.out_idx + row * k;
            map = j.id_map ? j.id_map + row * j.ld : nullptr;
        } else {
            ok = j.ck_out + (row * j.nchunks + chunk) * k;
            oc = j.cc_out + (row * j.nchunks + chunk) * k;
        }
    } else if (j.mode == kJobMerge) {
        const int n = j.nchunks * k;
        load_cands<KPT>(j.ck_in + bid * (int64_t)n, j.cc_in + bid * (int64_t)n, n, key, col);
        out = j.out_idx + bid * k;
        map = j.id_map ? j.id_map + bid * j.ld : nullptr;
    } else {
        const int ngroups = (j.nchunks + j.cpg - 1) / j.cpg;
        const int64_t row = bid / ngroups;
        const int g = (int)(bid % ngroups);
        const int c_end = (g + 1) * j.cpg < j.nchunks ? (g + 1) * j.cpg : j.nchunks;
        const int64_t base = (row * j.nchunks + (int64_t)g * j.cpg) * k;
        load_cands<KPT>(j.ck_in + base, j.cc_in + base, (c_end - g * j.cpg) * k, key, col);
        ok = j.ck_out + (row * ngroups + g) * (int64_t)k;
        oc = j.cc_out + (row * ngroups + g) * (int64_t)k;
    }
    const uint32_t emitted = reg_select_emit<NT, KPT, true>(
        key, (uint32_t)k, sh, [&](int u) { return col[u]; },
        [&](uint32_t slot, uint32_t kv, int32_t c) {
            if (out) {
                out[slot] = map ? map[c] : c;
            } else {
                ok[slot] = kv;
                oc[slot] = c;
            }
        });
    for (int t = (int)emitted + tid; t < k; t += NT) {
        if (out) {
            out[t] = -1;
        } else {
            ok[t] = 0u;
            oc[t] = -1;
        }
    }
}

// Two independent selections in one launch of 1024-thread workgroups:
// workgroups [0, a.nblocks) run job a, the rest job b (each with up to KPT
// keys per thread). Small selections cost little more than a launch, so two
// that do not depend on each other share one.
template <int KPT>
__global__ __launch_bounds__(1024) void topk_pair_kernel(TkJob a, TkJob b) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[reg_smem_bytes<1024, KPT>()];
    const bool first = (int)blockIdx.x < a.nblocks;
    const TkJob j = first ? a : b;
    reg_any_body<KPT>(j, first ? (int64_t)blockIdx.x : (int64_t)blockIdx.x - a.nblocks, smem);
}

// Chunks per row on the register path; 0 = the shape needs the global-memory path.
int32_t topk_reg_chunks(int32_t rows, int64_t ncols, int32_t k) {
    // chunks of <= 16384 keys (16 per thread: two workgroups fit a CU) unless
    // the merge capacity needs the larger ones
    int64_t c = (ncols + kRegMaxKeys / 2 - 1) / (kRegMaxKeys / 2);
    if (c > 1 && c * k > kRegMaxCand) c = (ncols + kRegMaxKeys - 1) / kRegMaxKeys;
    // few rows: split further until the chunks of all rows give 128 workgroups
    // (chunks >= 2048). 128 rather than one per CU: for 32 rows x 32768 block
    // scores, k = 2048, 4 chunks and a merge of 8192 candidates measured
    // 19.4 us against 20.1 us with 8 chunks and 16384 candidates.
    while (rows * c < 128 && ncols / (c * 2) >= 2048 && (c * 2) * k <= kRegMaxCand) c *= 2;
    if (c > 1 && c * k > kRegMaxCand) return 0;
    return (int32_t)c;
}

// Workgroup size and keys per thread for a segment of n keys: 256 threads up
// to 8 keys each, else 1024 threads with the smallest power of two covering n.
struct RegShape {
    int nt, kpt;
};
RegShape reg_shape(int64_t n) {
    if (n <= 256 * 8) {
        int kpt = 1;
        while ((int64_t)kpt * 256 < n) kpt *= 2;
        return {256, kpt};
    }
    int kpt = 1;
    while ((int64_t)kpt * 1024 < n) kpt *= 2;
    return {1024, kpt};
}

// Threads and keys per thread of a job: from its segment size (the chunk
// length, nchunks * k merged candidates, or cpg * k grouped ones), as each
// kernel below is instantiated.
RegShape job_shape(const TkJob& j) {
    if (j.mode == kJobChunk) {
        // 512 threads x 32 keys: measured 23% faster than 1024 x 16 for 4096
        // rows x 65536 scores (two workgroups of 8 waves per CU); with fewer
        // workgroups than CUs, 1024 x 16 is faster (8 rows x 131072 block
        // scores, k = 2048: 26.5 against 28.6 us)
        if (j.chunk_len > 8192 && j.chunk_len <= 16384 && j.nblocks >= 256) return {512, 32};
        RegShape a = reg_shape(j.chunk_len);
        if (a.nt == 1024) a.kpt = a.kpt < 4 ? 4 : a.kpt > 32 ? 32 : a.kpt;
        return a;
    }
    if (j.mode == kJobMerge) {
        RegShape m = reg_shape((int64_t)j.nchunks * j.k);
        if (m.nt == 1024) m.kpt = m.kpt < 4 ? 4 : m.kpt > 16 ? 16 : m.kpt;
        return m;
    }
    const RegShape m = reg_shape((int64_t)j.cpg * j.k);
    if (m.nt == 256) return {256, 8};
    return {1024, m.kpt <= 8 ? 8 : 16};
}

void launch_chunk_job(const TkJob& j, RegShape a, hipStream_t s) {
    const dim3 g((unsigned)j.nblocks);
#define CSA2_CHUNK(NT, KPT) hipLaunchKernelGGL((topk_reg_chunk_kernel<NT, KPT>), g, dim3(NT), 0, s, j)
    if (a.nt == 512) {
        CSA2_CHUNK(512, 32);
    } else if (a.nt == 256) {
        switch (a.kpt) {
            case 1: CSA2_CHUNK(256, 1); break;
            case 2: CSA2_CHUNK(256, 2); break;
            case 4: CSA2_CHUNK(256, 4); break;
            default: CSA2_CHUNK(256, 8); break;
        }
    } else {
        switch (a.kpt) {
            case 4: CSA2_CHUNK(1024, 4); break;
            case 8: CSA2_CHUNK(1024, 8); break;
            case 16: CSA2_CHUNK(1024, 16); break;
            default: CSA2_CHUNK(1024, 32); break;
        }
    }
#undef CSA2_CHUNK
}

void launch_merge_job(const TkJob& j, RegShape m, hipStream_t s) {
    const dim3 g((unsigned)j.nblocks);
#define CSA2_MERGE(NT, KPT) hipLaunchKernelGGL((topk_reg_merge_kernel<NT, KPT>), g, dim3(NT), 0, s, j)
    if (m.nt == 256) {
        switch (m.kpt) {
            case 1: CSA2_MERGE(256, 1); break;
            case 2: CSA2_MERGE(256, 2); break;
            case 4: CSA2_MERGE(256, 4); break;
            default: CSA2_MERGE(256, 8); break;
        }
    } else {
        switch (m.kpt) {
            case 4: CSA2_MERGE(1024, 4); break;
            case 8: CSA2_MERGE(1024, 8); break;
            default: CSA2_MERGE(1024, 16); break;
        }
    }
#undef CSA2_MERGE
}

void launch_group_job(const TkJob& j, RegShape m, hipStream_t s) {
    const dim3 g((unsigned)j.nblocks);
    if (m.nt == 256)
        hipLaunchKernelGGL((topk_reg_group_merge_kernel<256, 8>), g, dim3(256), 0, s, j);
    else if (m.kpt == 8)
        hipLaunchKernelGGL((topk_reg_group_merge_kernel<1024, 8>), g, dim3(1024), 0, s, j);
    else
        hipLaunchKernelGGL((topk_reg_group_merge_kernel<1024, 16>), g, dim3(1024), 0, s, j);
}

void launch_job(const TkJob& j, hipStream_t s) {
    if (j.nblocks == 0) return;
    const RegShape sh = job_shape(j);
    switch (j.mode) {
        case kJobChunk: launch_chunk_job(j, sh, s); break;
        case kJobMerge: launch_merge_job(j, sh, s); break;
        default: launch_group_job(j, sh, s); break;
    }
}

// Two independent jobs: one launch when both take the same 1024-thread shape
// (run with another shape, a selection measured up to 3.6 times slower: a
// 2048-candidate group merge took 22 us at 1024 x 16 against 6 us at
// 256 x 8), else one launch each.
void launch_pair(const TkJob& a, const TkJob& b, hipStream_t s) {
    const RegShape sa = job_shape(a), sb = job_shape(b);
    if (a.nblocks == 0 || b.nblocks == 0 || sa.nt != 1024 || sb.nt != 1024 || sa.kpt != sb.kpt || sa.kpt > 16) {
        launch_job(a, s);
        launch_job(b, s);
        return;
    }
    const dim3 g((unsigned)(a.nblocks + b.nblocks));
    switch (sa.kpt) {
        case 4: hipLaunchKernelGGL(topk_pair_kernel<4>, g, dim3(1024), 0, s, a, b); break;
        case 8: hipLaunchKernelGGL(topk_pair_kernel<8>, g, dim3(1024), 0, s, a, b); break;
        default: hipLaunchKernelGGL(topk_pair_kernel<16>, g, dim3(1024), 0, s, a, b); break;
    }
}

int32_t topk_chunks(int32_t rows, int64_t ncols, int32_t k) {
    if (rows >= 256 || ncols <= 4 * (int64_t)k || ncols <= 8192) return 1;
    int64_t c = 1;
    while (c * 2 * c * 2 <= ncols / k && c < 64) c *= 2;  // about sqrt(ncols / k)
    while (c > 1 && ncols / c < 2 * (int64_t)k) c /= 2;
    return (int32_t)c;
}

TkJob merge_job(int32_t rows, int32_t k, int32_t c, const int32_t* id_map, int64_t ld, const uint32_t* ck,
                const int32_t* cc, int32_t* out_idx) {
    TkJob j;
    j.mode = kJobMerge;
    j.nblocks = rows;
    j.k = k;
    j.nchunks = c;
    j.id_map = id_map;
    j.ld = ld;
    j.ck_in = ck;
    j.cc_in = cc;
    j.out_idx = out_idx;
    return j;
}

// The launches of one register-path selection: one or two levels of jobs.
struct TkPlan {
    int n = 0;
    TkJob lv[2];
};

}  // namespace

// Two-level merges: first-level groups of 2048 candidates where the second
// level still fits the merge capacity (more, smaller workgroups: 20.7 against
// 23.0 us with 8192-candidate groups, and 35.9 us with 16384, at 8 rows x 128
// chunks x 512), else groups of up to 8192 candidates.
static int32_t merge_chunks_per_group(int32_t nchunks, int32_t k) {
    for (const int32_t cand : {2048, kRegMaxCand / 2}) {
        const int32_t cpg = k <= cand ? cand / k : 1;
        if ((int64_t)((nchunks + cpg - 1) / cpg) * k <= kRegMaxCand) return cpg;
    }
    return k <= kRegMaxCand / 2 ? (kRegMaxCand / 2) / k : 1;
}

int32_t topk_merge_groups(int32_t nchunks, int32_t k) {
    if ((int64_t)nchunks * k <= kRegMaxCand) return 1;
    const int32_t cpg = merge_chunks_per_group(nchunks, k);
    return (nchunks + cpg - 1) / cpg;
}

// The merge of rows x nchunks x k candidates (nothing when nchunks <= 1).
static TkPlan plan_merge(int32_t rows, int32_t k, int32_t nchunks, const uint32_t* ck, const int32_t* cc,
                         int32_t* out_idx, uint32_t* ck2, int32_t* cc2) {
    TkPlan p;
    if (rows == 0 || nchunks <= 1) return p;
    const int32_t ng = topk_merge_groups(nchunks, k);
    if (ng == 1) {
        p.lv[p.n++] = merge_job(rows, k, nchunks, nullptr, 0, ck, cc, out_idx);
        return p;
    }
    TkJob g;
    g.mode = kJobGroup;
    g.nblocks = rows * ng;
    g.k = k;
    g.nchunks = nchunks;
    g.cpg = merge_chunks_per_group(nchunks, k);
    g.ck_in = ck;
    g.cc_in = cc;
    g.ck_out = ck2;
    g.cc_out = cc2;
    p.lv[p.n++] = g;
    p.lv[p.n++] = merge_job(rows, k, ng, nullptr, 0, ck2, cc2, out_idx);
    return p;
}

// Top-k over rows x ncols scores on the register path (n = 0: the shape needs
// the global-memory path). ws holds the chunks' candidates.
// c_force > 0 takes that many chunks instead of topk_reg_chunks' count (the
// caller checks the merge capacity and the workspace).
static TkPlan plan_select(const float* scores, int32_t rows, int64_t ncols, int64_t ld, const int32_t* row_len,
                          int32_t k, const int32_t* id_map, int32_t* out_idx, void* ws, int32_t c_force = 0) {
    TkPlan p;
    const int32_t c = c_force > 0 ? c_force : topk_reg_chunks(rows, ncols, k);
    if (c == 0 || rows == 0) return p;
    TkJob j;
    j.mode = kJobChunk;
    j.nblocks = rows * c;
    j.scores = scores;
    j.ncols = ncols;
    j.ld = ld;
    j.row_len = row_len;
    j.chunk_len = (ncols + c - 1) / c;
    j.id_map = id_map;
    j.nchunks = c;
    j.k = k;
    j.out_idx = out_idx;
    if (c > 1) {
        j.ck_out = reinterpret_cast<uint32_t*>(ws);
        j.cc_out = reinterpret_cast<int32_t*>(j.ck_out + (size_t)rows * c * k);
    }
    p.lv[p.n++] = j;
    if (c > 1) p.lv[p.n++] = merge_job(rows, k, c, id_map, ld, j.ck_out, j.cc_out, out_idx);
    return p;
}

int launch_topk_merge(int32_t rows, int32_t k, int32_t nchunks, const uint32_t* ck, const int32_t* cc,
                      int32_t* out_idx, uint32_t* ck2, int32_t* cc2, hipStream_t s) {
    const TkPlan p = plan_merge(rows, k, nchunks, ck, cc, out_idx, ck2, cc2);
    for (int i = 0; i < p.n; i++) launch_job(p.lv[i], s);
    return 0;
}

bool launch_topk_merge_select(int32_t rows_a, int32_t k_a, int32_t nchunks_a, const uint32_t* ck, const int32_t* cc,
                              int32_t* out_a, uint32_t* ck2, int32_t* cc2, const float* scores_b, int32_t rows_b,
                              int64_t ncols_b, int32_t k_b, int32_t* out_b, void* ws_b, hipStream_t s) {
    TkPlan b = plan_select(scores_b, rows_b, ncols_b, ncols_b, nullptr, k_b, nullptr, out_b, ws_b);
    if (rows_b > 0 && b.n == 0) return false;
    const TkPlan a = plan_merge(rows_a, k_a, nchunks_a, ck, cc, out_a, ck2, cc2);
    if (a.n > 0 && b.n > 0) {
        // Fewer, longer chunks of the second selection where that gives its
        // first level the shape of the merge's first level, so the two share
        // a launch (32 x 32768 block maxima, k = 2048: 2 chunks of 16384 beside
        // a 16384-candidate merge). Fewer chunks need no more workspace.
        const RegShape sa = job_shape(a.lv[0]), sb = job_shape(b.lv[0]);
        const int64_t len = (int64_t)1024 * sa.kpt;
        const int32_t c = (int32_t)((ncols_b + len - 1) / len);
        if (sa.nt == 1024 && (sa.nt != sb.nt || sa.kpt != sb.kpt) && c < b.lv[0].nchunks &&
            (c == 1 || (int64_t)c * k_b <= kRegMaxCand)) {
            const TkPlan b2 = plan_select(scores_b, rows_b, ncols_b, ncols_b, nullptr, k_b, nullptr, out_b, ws_b, c);
            const RegShape s2 = job_shape(b2.lv[0]);
            if (s2.nt == sa.nt && s2.kpt == sa.kpt) b = b2;
        }
    }
    const int levels = a.n > b.n ? a.n : b.n;
    for (int i = 0; i < levels; i++) {
        if (i < a.n && i < b.n)
            launch_pair(a.lv[i], b.lv[i], s);
        else
            launch_job(i < a.n ? a.lv[i] : b.lv[i], s);
    }
    return true;
}

size_t topk_workspace_bytes(int32_t rows, int64_t ncols, int32_t k) {
    int32_t c = topk_reg_chunks(rows, ncols, k);
    if (c == 0) c = topk_chunks(rows, ncols, k);
    if (c == 1) return 0;
    return (size_t)rows * c * k * (sizeof(uint32_t) + sizeof(int32_t));
}

int launch_topk(const float* scores, int32_t rows, int64_t ncols, int64_t ld, const int32_t* row_len, int32_t k,
                const int32_t* id_map, int32_t* out_idx, void* ws, hipStream_t s) {
    if (rows == 0) return 0;
    const TkPlan p = plan_select(scores, rows, ncols, ld, row_len, k, id_map, out_idx, ws);
    if (p.n > 0) {
        for (int i = 0; i < p.n; i++) launch_job(p.lv[i], s);
        return 0;
    }
    const int32_t c = topk_chunks(rows, ncols, k);
    const int64_t chunk_len = (ncols + c - 1) / c;
    uint32_t* ck = nullptr;
    int32_t* cc = nullptr;
    if (c > 1) {
        ck = reinterpret_cast<uint32_t*>(ws);
        cc = reinterpret_cast<int32_t*>(ck + (size_t)rows * c * k);
    }
    hipLaunchKernelGGL(topk_chunk_kernel, dim3((unsigned)((int64_t)rows * c)), dim3(kTkThreads), 0, s, scores, ncols,
                       ld, row_len, k, c, chunk_len, id_map, out_idx, ck, cc);
    if (c > 1)
        hipLaunchKernelGGL(topk_merge_kernel, dim3((unsigned)rows), dim3(kTkThreads), 0, s, ld, k, c, id_map, ck, cc,
                           out_idx);
    return 0;
}

}  // namespace csa2
