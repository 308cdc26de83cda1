// Indexer scoring: score(q, i) = sum_h w[q][h] * max(q_idx[q][h] . k_idx[i], 0)
// over 32 heads x 128 dims (eogee.com report on DeepSeek-V4.1-Flash, 3.2 and
// 3.3; nxbn.cn walkthrough 3.3 for the 32 x 128 geometry), plus the 8-position
// block maximum of the hierarchical indexer (eogee.com report 3.3).
//
// The head contraction runs on 32x32x16 bf16 MFMA: M = the 32 heads of one
// query, N = 32 entries, K = 128 channels in 8 steps. Each lane of the result
// holds 16 heads of one entry; the ReLU-weighted head sum runs in fp32 on the
// lane, then one cross-half exchange adds the other 16 heads.
//
// The indexer K is either bf16 [N][128] or FP4 entries [N][68] (128 E2M1
// codes + one binary32 scale s, the storage precision implied by the pages'
// byte accounting). FP4 codes decode exactly to bf16 and feed the same MFMA;
// s multiplies the entry's head sum once (ReLU(s x) = s ReLU(x), s >= 0).
//
// Three kernels:
//  * index_stream_kernel -- one query per workgroup slice; each wave streams
//    32-entry tiles of the indexer K straight from HBM into MFMA operand
//    registers (2 tiles in flight). Bound by HBM (256 B per entry per query).
//    Serves decode (a sequence per query) and the Reindex pool gather.
//  * index_topk_kernel -- the same streaming score for a chunk of a row, kept
//    in LDS and reduced to the chunk's top-k candidates (decode Full layers,
//    and Reindex layers over their pool); a merge finishes the row.
//  * index_prefill_kernel -- many queries over one sequence: a workgroup holds
//    8 queries' operands in registers and stages 64-entry K tiles in LDS, so
//    each K byte read from L2 feeds 8 queries. Bound by MFMA.
#include <math.h>

#include "device_common.h"
#include "launch.h"
#include "topk_select.h"

namespace csa2 {

namespace {

constexpr int kStreamThreads = 256;
constexpr int kStreamWaves = kStreamThreads / 64;

template <bool kFp4>
struct StreamTile;
template <>
struct StreamTile<false> {
    bf16x8 b[8];
    int64_t ent;
    bool valid;
};
template <>
struct StreamTile<true> {
    uint32_t code[8];  // 64 channels of the entry, 8 per dword
    float scale;
    int64_t ent;
    bool valid;
};

constexpr int kKRec = 68;  // bytes per FP4 indexer-K entry

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Eight E2M1 codes (channel 2b in bits 8b..8b+3, 2b+1 above) -> their exact
// bf16 values, in channel order.
CSA2_DEVINL bf16x8 fp4x8_to_bf16(uint32_t w) {
    const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0);
    const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1);
    const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2);
    const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3);
    return as_bf16x8(make_uint4(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                                __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)));
}

// Row of the accumulator held in register r by a lane of half `half` (32x32 layout).
CSA2_DEVINL int acc_row(int r, int half) { return (r >> 2) * 8 + half * 4 + (r & 3); }

// Per-lane state of the streaming kernels: the query's A operand and head
// weights. A operand: head = lane % 32; step j covers channels 16j + 8*half
// .. +8 (bf16 K), or 64*half + 8j .. +8 for FP4 K so that a lane's 8 steps
// read 32 contiguous code bytes of its entry (the same re-ordering on both
// operands leaves the dot product unchanged).
template <bool kFp4>
struct StreamQuery {
    bf16x8 a[8];
    float wr[16];
    CSA2_DEVINL void load(const uint16_t* q_idx, const float* w, int64_t q, int half, int col_in_tile) {
        const uint16_t* qrow = q_idx + (q * kIdxHeads + col_in_tile) * kIdxDim;
#pragma unroll
        for (int j = 0; j < 8; j++)
            a[j] = as_bf16x8(reinterpret_cast<const uint4*>(qrow)[kFp4 ? 8 * half + j : 2 * j + half]);
#pragma unroll
        for (int r = 0; r < 16; r++) wr[r] = w[q * kIdxHeads + acc_row(r, half)];
    }
};

// Loads the K data of entry `ent` of one sequence (kseq: bf16 [N][128] or FP4
// [N][68]) for this lane's half. Plain (cache-allocating) loads: a tile reads
// 32 B of each of 32 rows per instruction, and the other 7 instructions of the
// same wave consume the rest of those lines, so the lines must stay in cache
// between them. An invalid entry reads entry 0 (its score is discarded).
template <bool kFp4>
CSA2_DEVINL void stream_load(const void* kseq, int64_t ent, bool valid, int half, StreamTile<kFp4>& st) {
    st.ent = ent;
    st.valid = valid;
    if constexpr (kFp4) {
        // 68-byte entries are only 4-byte aligned: dword loads
        const uint8_t* e = static_cast<const uint8_t*>(kseq) + (valid ? ent : 0) * kKRec;
        const uint32_t* src = reinterpret_cast<const uint32_t*>(e + 32 * half);
#pragma unroll
        for (int j = 0; j < 8; j++) st.code[j] = src[j];
        st.scale = *reinterpret_cast<const float*>(e + 64);
    } else {
        const uint4* src =
            reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(kseq) + (valid ? ent : 0) * kIdxDim) + half;
#pragma unroll
        for (int j = 0; j < 8; j++) st.b[j] = as_bf16x8(src[2 * j]);
    }
}

// Score of the tile's entry in lanes 0..31 (lanes 32..63 hold a partial sum):
// the 32-head contraction, ReLU, weights, head sum; -inf for invalid entries.
template <bool kFp4>
CSA2_DEVINL float stream_score(const StreamQuery<kFp4>& Q, const StreamTile<kFp4>& st) {
    f32x16 acc = {};
#pragma unroll
    for (int j = 0; j < 8; j++) {
        if constexpr (kFp4)
            acc = mfma32x32x16(Q.a[j], fp4x8_to_bf16(st.code[j]), acc);
        else
            acc = mfma32x32x16(Q.a[j], st.b[j], acc);
    }
    float s = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; r++) s = fmaf(Q.wr[r], relu_bits(acc[r]), s);
    s += from_upper_half(s);  // lanes 0..31 hold the sum over all 32 heads
    if constexpr (kFp4) s *= st.scale;
    return st.valid ? s : -INFINITY;
}

template <bool kReindex, bool kFp4>
__global__ __launch_bounds__(kStreamThreads) void index_stream_kernel(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w, const void* __restrict__ k_idx, int64_t N,
    int32_t q_per_seq, const int32_t* __restrict__ n_visible, const int32_t* __restrict__ cand_blocks, int32_t nb,
    float* __restrict__ scores, float* __restrict__ block_scores, int32_t* __restrict__ pool_ids, int64_t ncols,
    int64_t ntiles, int32_t wgs_per_q, int32_t tiles_per_wg) {
    const int64_t q = blockIdx.x / wgs_per_q;
    const int64_t chunk = blockIdx.x % wgs_per_q;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int half = lane >> 5, col_in_tile = lane & 31;
    const int64_t seq = q / q_per_seq;
    int64_t nv = n_visible ? (int64_t)n_visible[q] : N;
    nv = nv < N ? nv : N;

    StreamQuery<kFp4> Q;
    Q.load(q_idx, w, q, half, col_in_tile);
    const void* kseq = kFp4 ? static_cast<const void*>(static_cast<const uint8_t*>(k_idx) + seq * N * kKRec)
                            : static_cast<const void*>(static_cast<const uint16_t*>(k_idx) + seq * N * kIdxDim);
    const int64_t t_begin = chunk * tiles_per_wg;
    const int64_t t_end = (t_begin + tiles_per_wg < ntiles) ? t_begin + tiles_per_wg : ntiles;
    const int64_t nblk = (N + 7) >> 3;

    auto load = [&](int64_t t, StreamTile<kFp4>& st) {
        const int64_t col = t * 32 + col_in_tile;
        if (kReindex) {
            const int32_t blk = (col < ncols) ? cand_blocks[q * nb + (col >> 3)] : -1;
            const int64_t ent = (int64_t)blk * 8 + (col & 7);
            stream_load<kFp4>(kseq, ent, blk >= 0 && ent < nv, half, st);
        } else {
            stream_load<kFp4>(kseq, col, col < nv, half, st);
        }
    };

    auto finish = [&](int64_t t, const StreamTile<kFp4>& st) {
        const float s = stream_score<kFp4>(Q, st);
        const int64_t col = t * 32 + col_in_tile;
        if (half == 0 && col < ncols) scores[q * ncols + col] = s;
        if (kReindex) {
            if (pool_ids && half == 0 && col < ncols) pool_ids[q * ncols + col] = st.valid ? (int32_t)st.ent : -1;
        } else if (block_scores) {
            const float m = max8_lanes(s);
            if (half == 0 && (lane & 7) == 0 && col < ncols) block_scores[q * nblk + (col >> 3)] = m;
        }
    };

    int64_t t = t_begin + wave;
    if (t >= t_end) return;
    StreamTile<kFp4> s0, s1;
    load(t, s0);
    while (true) {
        const int64_t t1 = t + kStreamWaves;
        if (t1 < t_end) load(t1, s1);
        finish(t, s0);
        if (t1 >= t_end) break;
        const int64_t t2 = t1 + kStreamWaves;
        if (t2 < t_end) load(t2, s0);
        finish(t1, s1);
        if (t2 >= t_end) break;
        t = t2;
    }
}

// Full-mode scoring fused with the per-query Top-K (the selection the pages'
// DeepSelect kernel makes, eogee.com report 3.5; Top-512 per query, titansim
// blog): a workgroup scores a chunk of kFtChunk entries of one query exactly
// as index_stream_kernel does, keeps the scores in LDS instead of writing
// them out, and selects the chunk's top-k as (key, entry) candidates; the
// Top-K merge then combines a query's chunks. A query's top-k entry is in its
// chunk's top-k, so the result equals Top-K over the full score row. With one
// chunk per query the workgroup writes the final indices itself; otherwise
// the Top-K merge kernels combine the chunks' candidates (a separate launch:
// making the last workgroup of a query merge in place needs device-scope
// fences, whose L2 write-back and invalidate cost the streaming workgroups
// more than the launch, measured 106 -> 159 us at 64 x 32768).
// Optional outputs: 8-position block maxima (the hierarchical pool's input)
// and the scores themselves (a debug path for parity checks).
//
// kRe: the same for a Reindex layer (eogee.com report 3.3: scoring restricted
// to the candidate pool) -- the row is the pool, position j*8 + t holding
// entry cand_blocks[q][j]*8 + t of sequence q / q_per_seq, and the candidates
// carry entry ids; with ascending cand_blocks the result is the Top-K of
// csa2_index_reindex's pool row mapped through its pool ids.
template <bool kFp4, bool kRe, int kFtThreads, int kFtChunk>
__global__ __launch_bounds__(kFtThreads) void index_topk_kernel(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w, const void* __restrict__ k_idx, int64_t N,
    int32_t q_per_seq, const int32_t* __restrict__ n_visible, const int32_t* __restrict__ cand_blocks, int32_t nb,
    int32_t k, int32_t nchunks, int32_t* __restrict__ out_idx, uint32_t* __restrict__ cand_key,
    int32_t* __restrict__ cand_col, float* __restrict__ block_scores, float* __restrict__ scores_dbg) {
    constexpr int kFtWaves = kFtThreads / 64;
    constexpr int kFtKpt = kFtChunk / kFtThreads;  // keys per thread
    static_assert(kFtKpt >= 4 && kFtKpt % 4 == 0, "keys are read from LDS as float4");
    __shared__ __attribute__((aligned(16))) float sc[kFtChunk];
    __shared__ tk::RegTk<kFtThreads> sh;
    // Reindex: the chunk's pool block ids (-1 past the pool)
    __shared__ int32_t cblk[kRe ? kFtChunk / 8 : 1];
    const int64_t q = blockIdx.x / nchunks;
    const int chunk = blockIdx.x % nchunks;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int half = lane >> 5, col_in_tile = lane & 31;
    int64_t nv = n_visible ? (int64_t)n_visible[q] : N;
    nv = nv < N ? nv : N;
    const int64_t ncols = kRe ? (int64_t)nb * 8 : N;  // row length: entries or pool positions
    const int64_t c0 = (int64_t)chunk * kFtChunk;
    const int n = (int)((ncols - c0) < kFtChunk ? (ncols - c0) : kFtChunk);  // positions of this chunk
    const int ntile = (n + 31) >> 5;
    const int64_t nblk = (N + 7) >> 3;
    if constexpr (kRe) {
        for (int i = tid; i < kFtChunk / 8; i += kFtThreads) {
            const int64_t b = c0 / 8 + i;
            cblk[i] = b < nb ? cand_blocks[q * nb + b] : -1;
        }
        lds_barrier();
    }

    StreamQuery<kFp4> Q;
    Q.load(q_idx, w, q, half, col_in_tile);
    const int64_t seq = kRe ? q / q_per_seq : q;
    const void* kseq = kFp4 ? static_cast<const void*>(static_cast<const uint8_t*>(k_idx) + seq * N * kKRec)
                            : static_cast<const void*>(static_cast<const uint16_t*>(k_idx) + seq * N * kIdxDim);
    // entry id at position p of the chunk (Reindex), p < n
    auto pool_entry = [&](int p) { return (int64_t)cblk[p >> 3] * 8 + (p & 7); };
    auto load = [&](int t, StreamTile<kFp4>& st) {
        const int p = t * 32 + col_in_tile;
        if constexpr (kRe) {
            const int32_t blk = p < n ? cblk[p >> 3] : -1;
            const int64_t ent = (int64_t)blk * 8 + (p & 7);
            stream_load<kFp4>(kseq, ent, blk >= 0 && ent < nv, half, st);
        } else {
            const int64_t col = c0 + p;
            stream_load<kFp4>(kseq, col, col < nv, half, st);
        }
    };
    auto finish = [&](int t, const StreamTile<kFp4>& st) {
        const float s = stream_score<kFp4>(Q, st);
        const int p = t * 32 + col_in_tile;
        if (half == 0) sc[p] = s;
        if (scores_dbg && half == 0 && p < n) scores_dbg[q * ncols + c0 + p] = s;
        if (!kRe && block_scores) {
            const float m = max8_lanes(s);
            if (half == 0 && (lane & 7) == 0 && p < n) block_scores[q * nblk + ((c0 + p) >> 3)] = m;
        }
    };
    int t = wave;
    if (t < ntile) {
        StreamTile<kFp4> s0, s1;
        load(t, s0);
        while (true) {
            const int t1 = t + kFtWaves;
            if (t1 < ntile) load(t1, s1);
            finish(t, s0);
            if (t1 >= ntile) break;
            const int t2 = t1 + kFtWaves;
            if (t2 < ntile) load(t2, s0);
            finish(t1, s1);
            if (t2 >= ntile) break;
            t = t2;
        }
    }
    lds_barrier();

    // the chunk's keys, kFtKpt consecutive positions per thread
    uint32_t key[kFtKpt];
    const int p0 = tid * kFtKpt;
#pragma unroll
    for (int u = 0; u < kFtKpt; u += 4) {
        const float4 f = *reinterpret_cast<const float4*>(&sc[p0 + u]);
        key[u + 0] = (p0 + u + 0 < n) ? tk::score_key(f.x) : 0u;
        key[u + 1] = (p0 + u + 1 < n) ? tk::score_key(f.y) : 0u;
        key[u + 2] = (p0 + u + 2 < n) ? tk::score_key(f.z) : 0u;
        key[u + 3] = (p0 + u + 3 < n) ? tk::score_key(f.w) : 0u;
    }
    // a selected key's payload: its entry id
    auto ent_of = [&](int u) { return (int32_t)(kRe ? pool_entry(p0 + u) : c0 + p0 + u); };
    if (nchunks == 1) {
        int32_t* out = out_idx + q * k;
        const uint32_t emitted = tk::reg_select_emit<kFtThreads, kFtKpt, true>(
            key, (uint32_t)k, sh, ent_of, [&](uint32_t slot, uint32_t, int32_t col) { out[slot] = col; });
        for (int i = (int)emitted + tid; i < k; i += kFtThreads) out[i] = -1;
    } else {
        uint32_t* ck = cand_key + (q * nchunks + chunk) * (int64_t)k;
        int32_t* cc = cand_col + (q * nchunks + chunk) * (int64_t)k;
        const uint32_t emitted = tk::reg_select_emit<kFtThreads, kFtKpt, true>(
            key, (uint32_t)k, sh, ent_of,
            [&](uint32_t slot, uint32_t kv, int32_t col) {
                ck[slot] = kv;
                cc[slot] = col;
            });
        for (int i = (int)emitted + tid; i < k; i += kFtThreads) {
            ck[i] = 0u;
            cc[i] = -1;
        }
    }
}

constexpr int kPfQueries = 8;          // queries per workgroup (2 per wave)
constexpr int kPfSub = 64;             // entries per LDS tile
constexpr int kPfRow = 256 + 16;       // padded LDS row bytes
constexpr int kPfChunk = 4096;         // entries per workgroup

// Registers of one prefill tile load: bf16 K 4 units of 16 bytes per thread;
// FP4 K 16 code bytes and the entry scale per thread.
template <bool kFp4>
struct PfPre;
template <>
struct PfPre<false> {
    uint4 v[4];
};
template <>
struct PfPre<true> {
    uint4 v;
    float scale;
};

template <bool kFp4, bool kBlk>
__global__ __launch_bounds__(256, 2) void index_prefill_kernel(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w, const void* __restrict__ k_idx, int64_t N,
    int32_t q_per_seq, const int32_t* __restrict__ n_visible, float* __restrict__ scores,
    float* __restrict__ block_scores, int32_t nchunks) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][kPfSub * kPfRow];
    __shared__ float kscale[2][kPfSub];  // FP4 K: the entries' scales
    const int b = blockIdx.x;
    int chunk, qg;
    if ((nchunks & 7) == 0) {
        // Consecutive workgroups land on different XCDs (round-robin); give each
        // XCD a fixed slice of entry chunks so its L2 keeps serving the same K.
        const int per = nchunks >> 3;
        chunk = (b & 7) * per + (b >> 3) % per;
        qg = b / nchunks;
    } else {
        chunk = b % nchunks;
        qg = b / nchunks;
    }
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int half = lane >> 5, col_in_tile = lane & 31;
    const int64_t qa = (int64_t)qg * kPfQueries + 2 * wave, qb = qa + 1;
    const int64_t seq = ((int64_t)qg * kPfQueries) / q_per_seq;
    int64_t nva = n_visible ? (int64_t)n_visible[qa] : N, nvb = n_visible ? (int64_t)n_visible[qb] : N;
    nva = nva < N ? nva : N;
    nvb = nvb < N ? nvb : N;

    bf16x8 aa[8], ab[8];
    {
        const uint4* sa = reinterpret_cast<const uint4*>(q_idx + (qa * kIdxHeads + col_in_tile) * kIdxDim) + half;
        const uint4* sb = reinterpret_cast<const uint4*>(q_idx + (qb * kIdxHeads + col_in_tile) * kIdxDim) + half;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            aa[j] = as_bf16x8(sa[2 * j]);
            ab[j] = as_bf16x8(sb[2 * j]);
        }
    }
    float wa[16], wb[16];
#pragma unroll
    for (int r = 0; r < 16; r++) {
        wa[r] = w[qa * kIdxHeads + acc_row(r, half)];
        wb[r] = w[qb * kIdxHeads + acc_row(r, half)];
    }

    const uint16_t* kseq = static_cast<const uint16_t*>(k_idx) + (kFp4 ? 0 : seq * N * kIdxDim);
    const uint8_t* kfseq = static_cast<const uint8_t*>(k_idx) + (kFp4 ? seq * N * kKRec : 0);
    const int64_t e_begin = (int64_t)chunk * kPfChunk;
    const int64_t e_end = (e_begin + kPfChunk < N) ? e_begin + kPfChunk : N;
    const int nsub = (int)((e_end - e_begin + kPfSub - 1) / kPfSub);
    const int64_t nblk = (N + 7) >> 3;

    // Tile loads into registers. bf16 K: 4 16-byte units per thread of the
    // 64 x 256 B tile. FP4 K: thread (entry tid/4, quarter tid%4) takes 16 code
    // bytes (32 channels) and the entry's scale.
    using Pre = PfPre<kFp4>;
    auto gload = [&](int st) {
        Pre p;
        if constexpr (kFp4) {
            const int row = tid >> 2, qq = tid & 3;
            int64_t e = e_begin + (int64_t)st * kPfSub + row;
            e = e < N ? e : 0;
            const uint32_t* src = reinterpret_cast<const uint32_t*>(kfseq + e * kKRec) + 4 * qq;
            p.v = make_uint4(src[0], src[1], src[2], src[3]);
            p.scale = *reinterpret_cast<const float*>(kfseq + e * kKRec + 64);
        } else {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int u = i * 256 + tid;  // 16-byte unit within the 64 x 256 B tile
                const int row = u >> 4, c16 = u & 15;
                int64_t e = e_begin + (int64_t)st * kPfSub + row;
                e = e < N ? e : 0;
                p.v[i] = reinterpret_cast<const uint4*>(kseq + e * kIdxDim)[c16];
            }
        }
        return p;
    };
    auto lstore = [&](int buf, const Pre& p) {
        if constexpr (kFp4) {
            const int row = tid >> 2, qq = tid & 3;
            uint8_t* dst = &lds[buf][row * kPfRow + qq * 64];
            const uint32_t c[4] = {p.v.x, p.v.y, p.v.z, p.v.w};
#pragma unroll
            for (int i = 0; i < 4; i++) *reinterpret_cast<bf16x8*>(dst + 16 * i) = fp4x8_to_bf16(c[i]);
            if (qq == 0) kscale[buf][row] = p.scale;
        } else {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int u = i * 256 + tid;
                const int row = u >> 4, c16 = u & 15;
                *reinterpret_cast<uint4*>(&lds[buf][row * kPfRow + c16 * 16]) = p.v[i];
            }
        }
    };
    // ReLU-weighted head sum of one query's 32 x 32 block (times the entry's
    // scale for FP4 K); valid in lanes 0..31.
    // ReLU-weighted head sums of both queries' 32 x 32 blocks, one query per
    // half-wave: each lane sums its 16 heads of each query, and one half-wave
    // swap hands lanes 0..31 both halves of query a and lanes 32..63 both
    // halves of query b (times the entry's scale for FP4 K).
    const int64_t nv_mine = half ? nvb : nva;
    auto head_sums = [&](const f32x16& acca, const f32x16& accb, int64_t col, float esc) {
        float sa = 0.0f, sb = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; r++) {
            sa = fmaf(wa[r], relu_bits(acca[r]), sa);
            sb = fmaf(wb[r], relu_bits(accb[r]), sb);
        }
        const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(sa), __float_as_uint(sb), false, false);
        float s = __uint_as_float(x[0]) + __uint_as_float(x[1]);
        if constexpr (kFp4) s *= esc;
        return col < nv_mine ? s : -INFINITY;
    };
    const int64_t q_mine = half ? qb : qa;
    auto store = [&](float s, float m, int64_t col) {
        if (col < N) {
            scores[q_mine * N + col] = s;
            if (kBlk && (lane & 7) == 0) block_scores[q_mine * nblk + (col >> 3)] = m;
        }
    };
    // One group = 32 entries (rows h2*32.. of an LDS tile) for both queries:
    // 8 fragment reads, 16 MFMAs. The epilogue of the previous group runs in
    // the same straight-line block so the scheduler can put its VALU work in
    // the shadow of these MFMAs. The group's entry scale (FP4 K) is read here,
    // while its tile is still in LDS, and travels with the accumulators.
    auto group = [&](int buf, int h2, f32x16& acca, f32x16& accb, float& esc, const f32x16& pa, const f32x16& pb,
                     float pesc, int64_t pcol, float (&out)[2]) {
        const uint8_t* rowp = lds[buf] + (h2 * 32 + col_in_tile) * kPfRow + half * 16;
        bf16x8 bj[8];
#pragma unroll
        for (int j = 0; j < 8; j++) bj[j] = as_bf16x8(*reinterpret_cast<const uint4*>(rowp + j * 32));
        if constexpr (kFp4) esc = kscale[buf][h2 * 32 + col_in_tile];
        acca = f32x16{};
        accb = f32x16{};
#pragma unroll
        for (int j = 0; j < 8; j++) {
            acca = mfma32x32x16(aa[j], bj[j], acca);
            accb = mfma32x32x16(ab[j], bj[j], accb);
        }
        out[0] = head_sums(pa, pb, pcol, pesc);
        out[1] = kBlk ? max8_lanes(out[0]) : 0.0f;  // block maxima only when asked for
        __builtin_amdgcn_sched_group_barrier(0x100, kFp4 ? 9 : 8, 0);  // fragment reads first
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
#pragma unroll
        for (int i = 0; i < 16; i++) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
        }
    };

    const int64_t tile_base = e_begin;
    lstore(0, gload(0));
    lds_barrier();
    f32x16 pa, pb, ca, cb;
    float pesc = 1.0f, cesc = 1.0f;
    float out[2];
    {
        const f32x16 z = {};
        group(0, 0, pa, pb, pesc, z, z, 1.0f, N, out);  // no previous group: its results are discarded
    }
    for (int st = 0; st < nsub; st++) {
        const bool more = st + 1 < nsub;
        // the last iteration re-reads tile 0 (in bounds) and discards it
        const Pre nxt = gload(more ? st + 1 : 0);
        const int64_t col0 = tile_base + (int64_t)st * kPfSub + col_in_tile;
        group(st & 1, 1, ca, cb, cesc, pa, pb, pesc, col0, out);
        store(out[0], out[1], col0);
        if (more) lstore((st + 1) & 1, nxt);
        lds_barrier();
        // After the last tile this reads the stale buffer; those results are never stored.
        group((st + 1) & 1, 0, pa, pb, pesc, ca, cb, cesc, col0 + 32, out);
        store(out[0], out[1], col0 + 32);
    }
}

}  // namespace

int launch_index_full(const uint16_t* q_idx, const float* w, const void* k, bool kfp4, int64_t N, int32_t nq,
                      int32_t q_per_seq, const int32_t* n_visible, float* scores, int32_t block_size,
                      float* block_scores, hipStream_t s) {
    if (nq == 0) return 0;
    float* bs = block_size > 0 ? block_scores : nullptr;
    if (q_per_seq % kPfQueries == 0) {
        const int32_t nchunks = (int32_t)((N + kPfChunk - 1) / kPfChunk);
        const int64_t grid = (int64_t)(nq / kPfQueries) * nchunks;
#define CSA2_PF(FP4, BLK)                                                                                  \
    hipLaunchKernelGGL((index_prefill_kernel<FP4, BLK>), dim3((unsigned)grid), dim3(256), 0, s, q_idx, w, k, N, \
                       q_per_seq, n_visible, scores, bs, nchunks)
        if (kfp4) {
            if (bs) CSA2_PF(true, true); else CSA2_PF(true, false);
        } else {
            if (bs) CSA2_PF(false, true); else CSA2_PF(false, false);
        }
#undef CSA2_PF
        return 0;
    }
    const int64_t ntiles = (N + 31) / 32;
    const int64_t total = ntiles * nq;
    int64_t tpw = (total + 2047) / 2048;
    tpw = ((tpw + kStreamWaves - 1) / kStreamWaves) * kStreamWaves;
    if (tpw < kStreamWaves) tpw = kStreamWaves;
    const int64_t wgs_per_q = (ntiles + tpw - 1) / tpw;
    const dim3 grid((unsigned)(wgs_per_q * nq));
    if (kfp4)
        hipLaunchKernelGGL((index_stream_kernel<false, true>), grid, dim3(kStreamThreads), 0, s, q_idx, w, k, N,
                           q_per_seq, n_visible, (const int32_t*)nullptr, 0, scores, bs, (int32_t*)nullptr, N, ntiles,
                           (int32_t)wgs_per_q, (int32_t)tpw);
    else
        hipLaunchKernelGGL((index_stream_kernel<false, false>), grid, dim3(kStreamThreads), 0, s, q_idx, w, k, N,
                           q_per_seq, n_visible, (const int32_t*)nullptr, 0, scores, bs, (int32_t*)nullptr, N, ntiles,
                           (int32_t)wgs_per_q, (int32_t)tpw);
    return 0;
}

// Entries per fused workgroup: 8192, or 4096 when 8192 would leave fewer than
// 512 workgroups; 256 threads for bf16 keys, 512 for FP4 keys (compute-
// heavier per byte). Measured select + merge (64 x 32K / 32 x 256K / 8 x 1M,
// us): bf16 with 256 threads 105 / 397 / 404 against 106 / 415 / 423 with
// 512 threads and 8192 entries; FP4 at 64 x 32K 43 with (512, 4096), 48 with
// (256, 4096), 47 with (512, 8192).
int64_t index_topk_chunk_len(int32_t nq, int64_t N) { return (int64_t)nq * ((N + 8191) / 8192) < 512 ? 4096 : 8192; }
int32_t index_topk_chunks(int32_t nq, int64_t N) {
    const int64_t c = index_topk_chunk_len(nq, N);
    return (int32_t)((N + c - 1) / c);
}

// The merge takes at most two levels of <= 16384 candidates per row.
static bool chunks_fit(int32_t c, int32_t k) { return c <= 1 || (int64_t)topk_merge_groups(c, k) * k <= 16384; }

// Reindex rows are short (nb * 8 pool positions, 16384 for the pages' 2048
// blocks) and few: the smallest chunk of 1024 .. 8192 positions holding at
// least 2k of them that keeps the grid within 512 workgroups (small batches
// still spread over the GPU) and the candidates within the merge.
int64_t reindex_topk_chunk_len(int32_t nq, int64_t ncols, int32_t k) {
    int64_t len = 1024;
    while (len < 8192 && len < 2 * (int64_t)k) len *= 2;
    while (len < 8192 && (int64_t)nq * ((ncols + len - 1) / len) > 512) len *= 2;
    while (len < 8192 && !chunks_fit((int32_t)((ncols + len - 1) / len), k)) len *= 2;
    return len;
}
int32_t reindex_topk_chunks(int32_t nq, int32_t nb, int32_t k) {
    const int64_t nc = (int64_t)nb * 8;
    const int64_t len = reindex_topk_chunk_len(nq, nc, k);
    return (int32_t)((nc + len - 1) / len);
}
static size_t chunks_workspace_bytes(int32_t nq, int32_t c, int32_t k) {
    if (c <= 1) return 0;
    const int32_t g = topk_merge_groups(c, k);
    return (size_t)nq * k * ((size_t)c + (g > 1 ? (size_t)g : 0)) * (sizeof(uint32_t) + sizeof(int32_t));
}
bool index_topk_fits(int32_t nq, int64_t N, int32_t k) { return chunks_fit(index_topk_chunks(nq, N), k); }
size_t index_topk_workspace_bytes(int32_t nq, int64_t N, int32_t k) {
    return chunks_workspace_bytes(nq, index_topk_chunks(nq, N), k);
}
bool reindex_topk_fits(int32_t nq, int32_t nb, int32_t k) { return chunks_fit(reindex_topk_chunks(nq, nb, k), k); }
size_t reindex_topk_workspace_bytes(int32_t nq, int32_t nb, int32_t k) {
    return chunks_workspace_bytes(nq, reindex_topk_chunks(nq, nb, k), k);
}

// Workspace layout of the fused call: rows x c x k candidate keys, then their
// entry ids, then (two-level merge only) rows x g x k of each.
struct FtWs {
    uint32_t* ck = nullptr;
    int32_t* cc = nullptr;
    uint32_t* ck2 = nullptr;
    int32_t* cc2 = nullptr;
    int32_t c = 1;
};
FtWs ft_ws_chunks(void* ws, int32_t nq, int32_t c, int32_t topk) {
    FtWs r;
    r.c = c;
    if (r.c > 1) {
        r.ck = reinterpret_cast<uint32_t*>(ws);
        r.cc = reinterpret_cast<int32_t*>(r.ck + (size_t)nq * r.c * topk);
        const int32_t g = topk_merge_groups(r.c, topk);
        if (g > 1) {
            r.ck2 = reinterpret_cast<uint32_t*>(r.cc + (size_t)nq * r.c * topk);
            r.cc2 = reinterpret_cast<int32_t*>(r.ck2 + (size_t)nq * g * topk);
        }
    }
    return r;
}
FtWs ft_ws(void* ws, int32_t nq, int64_t N, int32_t topk) { return ft_ws_chunks(ws, nq, index_topk_chunks(nq, N), topk); }

int launch_index_topk(const uint16_t* q_idx, const float* w, const void* k, bool kfp4, int64_t N, int32_t nq,
                      const int32_t* n_visible, int32_t topk, int32_t* out_idx, float* block_scores,
                      float* scores_dbg, void* ws, hipStream_t s) {
    if (nq == 0) return 0;
    const FtWs f = ft_ws(ws, nq, N, topk);
    const bool small = index_topk_chunk_len(nq, N) == 4096;
    const dim3 grid((unsigned)((int64_t)nq * f.c));
#define CSA2_FT(FP4, NT, CH)                                                                                   \
    hipLaunchKernelGGL((index_topk_kernel<FP4, false, NT, CH>), grid, dim3(NT), 0, s, q_idx, w, k, N, 1, n_visible, \
                       nullptr, 0, topk, f.c, out_idx, f.ck, f.cc, block_scores, scores_dbg)
    if (kfp4) {
        if (small) CSA2_FT(true, 512, 4096); else CSA2_FT(true, 512, 8192);
    } else {
        if (small) CSA2_FT(false, 256, 4096); else CSA2_FT(false, 256, 8192);
    }
#undef CSA2_FT
    return 0;
}

int launch_index_topk_merge(int64_t N, int32_t nq, int32_t topk, int32_t* out_idx, void* ws, hipStream_t s) {
    if (nq == 0) return 0;
    const FtWs f = ft_ws(ws, nq, N, topk);
    if (f.c > 1) launch_topk_merge(nq, topk, f.c, f.ck, f.cc, out_idx, f.ck2, f.cc2, s);
    return 0;
}

// Reindex scoring fused with the Top-K: the chunk kernel in Reindex mode
// (256 threads for either key format), then the merge of the chunks'
// candidates when a row has more than one chunk.
int launch_index_reindex_topk(const uint16_t* q_idx, const float* w, const void* k, bool kfp4, int64_t N, int32_t nq,
                              int32_t q_per_seq, const int32_t* n_visible, const int32_t* cand_blocks, int32_t nb,
                              int32_t topk, int32_t* out_idx, float* pool_scores, void* ws, hipStream_t s) {
    if (nq == 0) return 0;
    const FtWs f = ft_ws_chunks(ws, nq, reindex_topk_chunks(nq, nb, topk), topk);
    const int64_t len = reindex_topk_chunk_len(nq, (int64_t)nb * 8, topk);
    const dim3 grid((unsigned)((int64_t)nq * f.c));
#define CSA2_RT(FP4, CH)                                                                                         \
    hipLaunchKernelGGL((index_topk_kernel<FP4, true, 256, CH>), grid, dim3(256), 0, s, q_idx, w, k, N, q_per_seq, \
                       n_visible, cand_blocks, nb, topk, f.c, out_idx, f.ck, f.cc, nullptr, pool_scores)
#define CSA2_RT_LEN(FP4)                   \
    switch (len) {                         \
        case 1024: CSA2_RT(FP4, 1024); break; \
        case 2048: CSA2_RT(FP4, 2048); break; \
        case 4096: CSA2_RT(FP4, 4096); break; \
        default: CSA2_RT(FP4, 8192); break;   \
    }
    if (kfp4) {
        CSA2_RT_LEN(true)
    } else {
        CSA2_RT_LEN(false)
    }
#undef CSA2_RT_LEN
#undef CSA2_RT
    if (f.c > 1) launch_topk_merge(nq, topk, f.c, f.ck, f.cc, out_idx, f.ck2, f.cc2, s);
    return 0;
}

int launch_index_reindex(const uint16_t* q_idx, const float* w, const void* k, bool kfp4, int64_t N, int32_t nq,
                         int32_t q_per_seq, const int32_t* n_visible, const int32_t* cand_blocks, int32_t nb,
                         float* pool_scores, int32_t* pool_ids, hipStream_t s) {
    if (nq == 0) return 0;
    const int64_t ncols = (int64_t)nb * 8;
    const int64_t ntiles = (ncols + 31) / 32;
    const int64_t total = ntiles * nq;
    int64_t tpw = (total + 2047) / 2048;
    tpw = ((tpw + kStreamWaves - 1) / kStreamWaves) * kStreamWaves;
    if (tpw < kStreamWaves) tpw = kStreamWaves;
    const int64_t wgs_per_q = (ntiles + tpw - 1) / tpw;
    const dim3 grid((unsigned)(wgs_per_q * nq));
    if (kfp4)
        hipLaunchKernelGGL((index_stream_kernel<true, true>), grid, dim3(kStreamThreads), 0, s, q_idx, w, k, N,
                           q_per_seq, n_visible, cand_blocks, nb, pool_scores, (float*)nullptr, pool_ids, ncols,
                           ntiles, (int32_t)wgs_per_q, (int32_t)tpw);
    else
        hipLaunchKernelGGL((index_stream_kernel<true, false>), grid, dim3(kStreamThreads), 0, s, q_idx, w, k, N,
                           q_per_seq, n_visible, cand_blocks, nb, pool_scores, (float*)nullptr, pool_ids, ncols,
                           ntiles, (int32_t)wgs_per_q, (int32_t)tpw);
    return 0;
}

}  // namespace csa2
