// Per-row Top-K (titansim blog, CSA2 modes: each Full / Reindex layer keeps its
// Top-512 entries; eogee.com report 3.3: the Full layer keeps the best 2048
// blocks). Exact selection under the order (score desc, column asc).
//
// Scores map to order-preserving 32-bit keys (larger key = larger score, -0
// folded onto +0, -inf and NaN to key 0 = never chosen). A workgroup finds the
// exact k-th largest key T with a 3-pass MSB radix select (11, 11, 10 bits)
// over LDS histograms, then emits every key > T plus the lowest-column ties
// == T, in column order, through a block-wide scan -- so the output is already
// ascending.
//
// Long rows are split: stage 1 selects the top-k of each chunk as (key,
// column) candidates; stage 2 selects the row's top-k among the candidates.
// A row's top-k entry is in its chunk's top-k (fewer than k chunk entries can
// beat it), so the two stages give the same set as one pass.
//
// Main path: a 1024-thread workgroup stages its chunk (<= 32768 keys) or its
// candidates (<= 16384 key/column pairs) in LDS, so every radix pass and the
// compaction read LDS, not memory. The first (most skewed) digit's histogram
// merges equal bins across a wave before the LDS atomic. The compaction gives
// each wave a contiguous range and emits in order with ballot prefix counts.
// Shapes beyond those capacities take the global-memory path (512 threads,
// every pass re-reads the scores through the caches).
#include <math.h>

#include "device_common.h"
#include "launch.h"

namespace csa2 {

namespace {

constexpr int kTkThreads = 512;
constexpr int kTkWaves = kTkThreads / 64;
constexpr int kHistBins = 2048;

CSA2_DEVINL uint32_t score_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (f != f || u == 0xFF800000u) return 0u;
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

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

// ------------------------------------------------------------------ LDS path

constexpr int kLdsThreads = 1024;
constexpr int kLdsWaves = kLdsThreads / 64;
constexpr int kLdsMaxKeys = 32768;  // stage-1 chunk capacity (128 KiB of keys)
constexpr int kLdsMaxCand = 16384;  // merge capacity (keys + columns, 128 KiB)

struct LdsTk {
    uint32_t hist[kHistBins];
    uint32_t wsum[kLdsWaves];
    uint32_t wsum2[kLdsWaves];
    uint32_t wgt[kLdsWaves];
    uint32_t weq[kLdsWaves];
    uint32_t sel_bin, sel_above;
};

CSA2_DEVINL uint32_t lane_prefix(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

CSA2_DEVINL uint32_t block_excl_scan_lds(uint32_t v, uint32_t* wsum, uint32_t* total) {
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
    for (int i = 0; i < kLdsWaves; i++) {
        const uint32_t s = wsum[i];
        before += (i < wave) ? s : 0u;
        tot += s;
    }
    __syncthreads();
    *total = tot;
    return before + x - v;
}

// Adds 1 to hist[bin] for every active lane; lanes of a wave with equal bins
// are merged into one atomic (the top digit of similar scores is shared).
CSA2_DEVINL void hist_add_merged(uint32_t* hist, uint32_t bin, bool act) {
    uint64_t todo = __ballot(act);
    const int lane = threadIdx.x & 63;
    while (todo) {
        const int leader = __ffsll((unsigned long long)todo) - 1;
        const uint32_t b = __shfl(bin, leader);
        const uint64_t same = __ballot(act && bin == b);
        if (lane == leader) atomicAdd(&hist[b], (uint32_t)__popcll(same));
        todo &= ~same;
    }
}

// Finds, from the current histogram, the bin holding the rem-th largest key
// (counting from the top bin): sets sh.sel_bin and sh.sel_above (keys in
// higher bins). nbins is 2048 or 1024.
CSA2_DEVINL void pick_bin(LdsTk& sh, uint32_t nbins, uint32_t rem) {
    const int tid = threadIdx.x;
    const int per = (int)(nbins / kLdsThreads);  // 2 or 1
    uint32_t c2[2] = {0u, 0u}, loc = 0;
#pragma unroll
    for (int jx = 0; jx < 2; jx++) {
        c2[jx] = (jx < per) ? sh.hist[nbins - 1 - (tid * per + jx)] : 0u;
        loc += c2[jx];
    }
    uint32_t tot;
    uint32_t above = block_excl_scan_lds(loc, sh.wsum2, &tot);
    if (above < rem && rem <= above + loc) {
        for (int jx = 0; jx < per; jx++) {
            if (above + c2[jx] >= rem) {
                sh.sel_bin = nbins - 1 - (tid * per + jx);
                sh.sel_above = above;
                break;
            }
            above += c2[jx];
        }
    }
    __syncthreads();
}

// Radix select over n LDS keys whose top-digit histogram and selectable count
// are already in sh.hist / `total`. Returns T and need (see radix_select).
CSA2_DEVINL void lds_select(const uint32_t* keys, int n, uint32_t kk, LdsTk& sh, uint32_t* T, uint32_t* need) {
    const int tid = threadIdx.x;
    uint32_t prefix = 0, rem = kk;
    pick_bin(sh, 2048u, rem);
    prefix = sh.sel_bin;
    rem -= sh.sel_above;
    const int shifts[2] = {10, 0};
    const int bits[2] = {11, 10};
#pragma unroll
    for (int p = 0; p < 2; p++) {
        __syncthreads();
        for (int i = tid; i < kHistBins; i += kLdsThreads) sh.hist[i] = 0;
        __syncthreads();
        const int sh_ = shifts[p], hi_shift = shifts[p] + bits[p];
        const uint32_t mask = (1u << bits[p]) - 1u;
        for (int i = tid; i < n; i += kLdsThreads) {
            const uint32_t key = keys[i];
            if (key && (key >> hi_shift) == prefix) atomicAdd(&sh.hist[(key >> sh_) & mask], 1u);
        }
        __syncthreads();
        pick_bin(sh, 1u << bits[p], rem);
        prefix = (prefix << bits[p]) | sh.sel_bin;
        rem -= sh.sel_above;
    }
    *T = prefix;
    *need = rem;
}

// Ordered emission of the selected positions of keys[0, n): wave w owns a
// contiguous range; emit(slot, i) is called for each selected i, slots in
// ascending i. Returns the number emitted.
template <class Emit>
CSA2_DEVINL uint32_t lds_emit(const uint32_t* keys, int n, uint32_t T, uint32_t need, LdsTk& sh, Emit emit) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int W = (n + kLdsWaves - 1) / kLdsWaves;
    W = (W + 63) & ~63;
    const int b0 = wave * W, b1 = (b0 + W < n) ? b0 + W : n;
    uint32_t gt = 0, eq = 0;
    for (int i = b0 + lane; i < b1; i += 64) {
        const uint32_t key = keys[i];
        gt += key > T;
        eq += key == T;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        gt += __shfl_xor(gt, o);
        eq += __shfl_xor(eq, o);
    }
    if (lane == 0) {
        sh.wgt[wave] = gt;
        sh.weq[wave] = eq;
    }
    __syncthreads();
    uint32_t gt_before = 0, eq_before = 0, total_gt = 0, total_eq = 0;
#pragma unroll
    for (int w = 0; w < kLdsWaves; w++) {
        gt_before += (w < wave) ? sh.wgt[w] : 0u;
        eq_before += (w < wave) ? sh.weq[w] : 0u;
        total_gt += sh.wgt[w];
        total_eq += sh.weq[w];
    }
    uint32_t slot = gt_before + (eq_before < need ? eq_before : need);
    uint32_t eq_run = eq_before;
    for (int base = b0; base < b1; base += 64) {
        const int i = base + lane;
        const uint32_t key = (i < b1) ? keys[i] : 0u;
        const bool isgt = (i < b1) && key > T, iseq = (i < b1) && key == T;
        const uint64_t eqm = __ballot(iseq);
        const bool sel = isgt || (iseq && eq_run + lane_prefix(eqm) < need);
        const uint64_t selm = __ballot(sel);
        if (sel) emit(slot + lane_prefix(selm), i);
        eq_run += (uint32_t)__popcll(eqm);
        slot += (uint32_t)__popcll(selm);
    }
    return total_gt + (total_eq < need ? total_eq : need);
}

// Stage 1 (or the only stage) on LDS: one 1024-thread workgroup per (row, chunk).
__global__ __launch_bounds__(kLdsThreads) void topk_lds_chunk_kernel(
    const float* __restrict__ scores, int64_t ncols, int64_t ld, const int32_t* __restrict__ row_len, int32_t k,
    int32_t nchunks, int64_t chunk_len, const int32_t* __restrict__ id_map, int32_t* __restrict__ out_idx,
    uint32_t* __restrict__ cand_key, int32_t* __restrict__ cand_col) {
    __shared__ uint32_t keys[kLdsMaxKeys];
    __shared__ LdsTk sh;
    const int tid = threadIdx.x;
    const int64_t row = blockIdx.x / nchunks;
    const int64_t chunk = blockIdx.x % nchunks;
    int64_t len = row_len ? (int64_t)row_len[row] : ncols;
    len = len < ncols ? len : ncols;
    len = len > 0 ? len : 0;
    const int64_t c0 = chunk * chunk_len;
    int64_t nn = len - c0;
    nn = nn < chunk_len ? nn : chunk_len;
    const int n = nn > 0 ? (int)nn : 0;
    for (int i = tid; i < kHistBins; i += kLdsThreads) sh.hist[i] = 0;
    __syncthreads();
    const float* src = scores + row * ld + c0;
    // Stage the chunk: 8 independent loads in flight per thread, then the
    // top-digit histogram from LDS (its merge loop would otherwise serialize
    // the loads).
    for (int i0 = 0; i0 < n; i0 += 8 * kLdsThreads) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; u++) {
            const int i = i0 + u * kLdsThreads + tid;
            v[u] = (i < n) ? src[i] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < 8; u++) {
            const int i = i0 + u * kLdsThreads + tid;
            if (i < n) keys[i] = score_key(v[u]);
        }
    }
    __syncthreads();
    uint32_t cnt = 0;
    for (int i = tid; i < n; i += kLdsThreads) {
        const uint32_t key = keys[i];
        cnt += key != 0u;
        if (key) atomicAdd(&sh.hist[key >> 21], 1u);
    }
    uint32_t total;
    block_excl_scan_lds(cnt, sh.wsum, &total);  // also orders the key stores above
    const uint32_t kk = total < (uint32_t)k ? total : (uint32_t)k;
    uint32_t emitted = 0;
    if (kk > 0) {
        uint32_t T, need;
        lds_select(keys, n, kk, sh, &T, &need);
        if (nchunks == 1) {
            int32_t* out = out_idx + row * k;
            const int32_t* map = id_map ? id_map + row * ld : nullptr;
            emitted = lds_emit(keys, n, T, need, sh, [&](uint32_t slot, int i) {
                out[slot] = map ? map[c0 + i] : (int32_t)(c0 + i);
            });
        } else {
            uint32_t* ck = cand_key + (row * nchunks + chunk) * k;
            int32_t* cc = cand_col + (row * nchunks + chunk) * k;
            emitted = lds_emit(keys, n, T, need, sh, [&](uint32_t slot, int i) {
                ck[slot] = keys[i];
                cc[slot] = (int32_t)(c0 + i);
            });
        }
    }
    if (nchunks == 1) {
        int32_t* out = out_idx + row * k;
        for (int t = (int)emitted + tid; t < k; t += kLdsThreads) out[t] = -1;
    } else {
        uint32_t* ck = cand_key + (row * nchunks + chunk) * k;
        int32_t* cc = cand_col + (row * nchunks + chunk) * k;
        for (int t = (int)emitted + tid; t < k; t += kLdsThreads) {
            ck[t] = 0u;
            cc[t] = -1;
        }
    }
}

// Stage 2 on LDS: one workgroup per row over its nchunks * k candidates.
__global__ __launch_bounds__(kLdsThreads) void topk_lds_merge_kernel(int64_t ld, int32_t k, int32_t nchunks,
                                                                      const int32_t* __restrict__ id_map,
                                                                      const uint32_t* __restrict__ cand_key,
                                                                      const int32_t* __restrict__ cand_col,
                                                                      int32_t* __restrict__ out_idx) {
    __shared__ uint32_t keys[kLdsMaxCand];
    __shared__ int32_t cols[kLdsMaxCand];
    __shared__ LdsTk sh;
    const int tid = threadIdx.x;
    const int64_t row = blockIdx.x;
    const int n = nchunks * k;
    for (int i = tid; i < kHistBins; i += kLdsThreads) sh.hist[i] = 0;
    __syncthreads();
    const uint32_t* ckr = cand_key + row * n;
    const int32_t* ccr = cand_col + row * n;
    for (int i0 = 0; i0 < n; i0 += 4 * kLdsThreads) {
        uint32_t kv_[4];
        int32_t cv[4];
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const int i = i0 + u * kLdsThreads + tid;
            kv_[u] = (i < n) ? ckr[i] : 0u;
            cv[u] = (i < n) ? ccr[i] : -1;
        }
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const int i = i0 + u * kLdsThreads + tid;
            if (i < n) {
                keys[i] = kv_[u];
                cols[i] = cv[u];
            }
        }
    }
    __syncthreads();
    uint32_t cnt = 0;
    for (int i = tid; i < n; i += kLdsThreads) {
        const uint32_t key = keys[i];
        cnt += key != 0u;
        if (key) atomicAdd(&sh.hist[key >> 21], 1u);
    }
    uint32_t total;
    block_excl_scan_lds(cnt, sh.wsum, &total);
    const uint32_t kk = total < (uint32_t)k ? total : (uint32_t)k;
    int32_t* out = out_idx + row * k;
    uint32_t emitted = 0;
    if (kk > 0) {
        uint32_t T, need;
        lds_select(keys, n, kk, sh, &T, &need);
        const int32_t* map = id_map ? id_map + row * ld : nullptr;
        emitted = lds_emit(keys, n, T, need, sh, [&](uint32_t slot, int i) {
            const int32_t col = cols[i];
            out[slot] = map ? map[col] : col;
        });
    }
    for (int t = (int)emitted + tid; t < k; t += kLdsThreads) out[t] = -1;
}

// Chunks per row on the LDS path; 0 = the shape needs the global-memory path.
int32_t topk_lds_chunks(int32_t rows, int64_t ncols, int32_t k) {
    int64_t c = (ncols + kLdsMaxKeys - 1) / kLdsMaxKeys;
    // few rows: split further so more workgroups share the row (chunks >= 4096)
    while (rows * c < 128 && ncols / (c * 2) >= 4096 && (c * 2) * k <= kLdsMaxCand) c *= 2;
    if (c > 1 && c * k > kLdsMaxCand) return 0;
    return (int32_t)c;
}

int32_t topk_chunks(int32_t rows, int64_t ncols, int32_t k) {
    if (rows >= 256 || ncols <= 4 * (int64_t)k || ncols <= 8192) return 1;
    int64_t c = 1;
    while (c * 2 * c * 2 <= ncols / k && c < 64) c *= 2;  // about sqrt(ncols / k)
    while (c > 1 && ncols / c < 2 * (int64_t)k) c /= 2;
    return (int32_t)c;
}

}  // namespace

size_t topk_workspace_bytes(int32_t rows, int64_t ncols, int32_t k) {
    int32_t c = topk_lds_chunks(rows, ncols, k);
    if (c == 0) c = topk_chunks(rows, ncols, k);
    if (c == 1) return 0;
    return (size_t)rows * c * k * (sizeof(uint32_t) + sizeof(int32_t));
}

int launch_topk(const float* scores, int32_t rows, int64_t ncols, int64_t ld, const int32_t* row_len, int32_t k,
                const int32_t* id_map, int32_t* out_idx, void* ws, hipStream_t s) {
    if (rows == 0) return 0;
    const int32_t cl = topk_lds_chunks(rows, ncols, k);
    const int32_t c = cl ? cl : topk_chunks(rows, ncols, k);
    const int64_t chunk_len = (ncols + c - 1) / c;
    uint32_t* ck = nullptr;
    int32_t* cc = nullptr;
    if (c > 1) {
        ck = reinterpret_cast<uint32_t*>(ws);
        cc = reinterpret_cast<int32_t*>(ck + (size_t)rows * c * k);
    }
    if (cl) {
        hipLaunchKernelGGL(topk_lds_chunk_kernel, dim3((unsigned)((int64_t)rows * c)), dim3(kLdsThreads), 0, s, scores,
                           ncols, ld, row_len, k, c, chunk_len, id_map, out_idx, ck, cc);
        if (c > 1)
            hipLaunchKernelGGL(topk_lds_merge_kernel, dim3((unsigned)rows), dim3(kLdsThreads), 0, s, ld, k, c, id_map,
                               ck, cc, out_idx);
        return 0;
    }
    hipLaunchKernelGGL(topk_chunk_kernel, dim3((unsigned)((int64_t)rows * c)), dim3(kTkThreads), 0, s, scores, ncols,
                       ld, row_len, k, c, chunk_len, id_map, out_idx, ck, cc);
    if (c > 1)
        hipLaunchKernelGGL(topk_merge_kernel, dim3((unsigned)rows), dim3(kTkThreads), 0, s, ld, k, c, id_map, ck, cc,
                           out_idx);
    return 0;
}

}  // namespace csa2
