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
// The indexer K is either bf16 [N][128] or FP4 entries [N][68] in the OCP
// MXFP4 format (128 E2M1 codes + one E8M0 scale per 32 channels, the storage
// precision implied by the pages' byte accounting). The gfx950 scaled
// FP4 -> bf16 conversion applies a block's power-of-two scale itself, so the
// decoded key E2M1 * 2^(b-127) is exact in bf16 (for scale bytes 2..252, the
// range whose decoded values are normal numbers) and feeds the same MFMA.
//
// Three kernels:
//  * index_stream_kernel -- one query per workgroup slice; each wave streams
//    32-entry tiles of the indexer K straight from HBM into MFMA operand
//    registers (2 tiles in flight). Bound by HBM (256 B per entry per query).
//    Serves decode (a sequence per query) and the Reindex pool gather.
//  * index_topk_kernel -- the same score for a chunk of a row, kept in LDS
//    and reduced to the chunk's top-k candidates (decode Full layers, and
//    Reindex layers over their pool); a merge finishes the row. Its tiles are
//    read in whole 128-byte lines with non-temporal loads (a streaming read
//    of this kind reaches about 6.9 TB/s on MI355X against about 6 TB/s for
//    plain loads) and reach the MFMA operand layout through a small per-wave
//    LDS stage.
//  * index_prefill_kernel -- many queries over one sequence: a workgroup holds
//    8 queries' operands in registers and stages 64-entry K tiles in LDS, so
//    each K byte read from L2 feeds 8 queries. Bound by MFMA.
#include <math.h>

#include <algorithm>
#include <type_traits>
#include <mutex>

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
    uint32_t scales;   // the entry's 4 E8M0 block scales
    int64_t ent;
    bool valid;
};

constexpr int kKRec = kKidxRecord;  // bytes per FP4 indexer-K entry

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Eight E2M1 codes (channel 2b in bits 8b..8b+3, 2b+1 above) times the power
// of two `x` -> their bf16 values, in channel order (exact while they are
// normal bf16 numbers).
CSA2_DEVINL bf16x8 fp4x8_to_bf16(uint32_t w, float x) {
    const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, x, 0);
    const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, x, 1);
    const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, x, 2);
    const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, x, 3);
    return as_bf16x8(make_uint4(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                                __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)));
}

// E8M0 byte `sel` of four packed scale bytes -> its value 2^(b-127) as a float
// (the byte becomes the binary32 exponent field).
CSA2_DEVINL float e8m0_byte(uint32_t four, int sel) { return __uint_as_float(((four >> (8 * sel)) & 0xFFu) << 23); }

// Row of the accumulator held in register r by a lane of half `half` (32x32 layout).
CSA2_DEVINL int acc_row(int r, int half) { return (r >> 2) * 8 + half * 4 + (r & 3); }

typedef int i32x8 __attribute__((ext_vector_type(8)));

// 32x32x64 MXFP4 x MXFP4 MFMA (gfx950 scaled f8f6f4, both operands E2M1): lane
// l holds row / column l % 32 and 32 consecutive channels of one scale block,
// whose E8M0 byte `sa` / `sb` it supplies; the result layout is that of the
// 32x32 bf16 MFMA. Each product is exact and accumulates in fp32.
CSA2_DEVINL f32x16 mfma32x32x64_fp4(uint4 a, uint4 b, uint32_t sa, uint32_t sb, f32x16 c) {
    const i32x8 av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
    const i32x8 bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 4, 4, 0, (int)sa, 0, (int)sb);
}

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
        st.scales = *reinterpret_cast<const uint32_t*>(e + kIdxDim / 2);
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
CSA2_DEVINL float stream_score(const StreamQuery<kFp4>& Q, const StreamTile<kFp4>& st, int half) {
    f32x16 acc = {};
    float x0 = 1.0f, x1 = 1.0f;  // FP4: scales of the lane's blocks 2*half and 2*half+1
    if constexpr (kFp4) {
        x0 = e8m0_byte(st.scales, 2 * half);
        x1 = e8m0_byte(st.scales, 2 * half + 1);
    }
#pragma unroll
    for (int j = 0; j < 8; j++) {
        if constexpr (kFp4)
            acc = mfma32x32x16(Q.a[j], fp4x8_to_bf16(st.code[j], j < 4 ? x0 : x1), acc);
        else
            acc = mfma32x32x16(Q.a[j], st.b[j], acc);
    }
    float s = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; r++) s = fmaf(Q.wr[r], relu_bits(acc[r]), s);
    s += from_upper_half(s);  // lanes 0..31 hold the sum over all 32 heads
    return st.valid ? s : -INFINITY;
}

// MXFP4 indexer Q (one 68-byte entry per head, the K entry format) with FP4 K:
// K-step s of lane (head / entry lane % 32, half) contracts scale block
// 2*half + s, i.e. the code dwords 4s .. 4s+3 of the 8 a K lane already holds
// (stream_load, line_operands4) against the same block of the query head, on
// the scaled FP4 MFMA: two 32x32x64 instructions, no decode.
struct StreamQuery4 {
    uint4 a4[2];
    uint32_t s4[2];
    float wr[16];
    CSA2_DEVINL void load(const uint16_t* q_idx, const float* w, int64_t q, int half, int col_in_tile) {
        const uint8_t* e = reinterpret_cast<const uint8_t*>(q_idx) + (q * kIdxHeads + col_in_tile) * kKRec;
        const uint32_t sc = *reinterpret_cast<const uint32_t*>(e + kIdxDim / 2);
#pragma unroll
        for (int st = 0; st < 2; st++) {
            const uint32_t* c = reinterpret_cast<const uint32_t*>(e + 16 * (2 * half + st));
            a4[st] = make_uint4(c[0], c[1], c[2], c[3]);
            s4[st] = (sc >> (8 * (2 * half + st))) & 0xFFu;
        }
#pragma unroll
        for (int r = 0; r < 16; r++) wr[r] = w[q * kIdxHeads + acc_row(r, half)];
    }
};
CSA2_DEVINL float stream_score4(const StreamQuery4& Q, const StreamTile<true>& st, int half) {
    f32x16 acc = mfma32x32x64_fp4(Q.a4[0], make_uint4(st.code[0], st.code[1], st.code[2], st.code[3]), Q.s4[0],
                                  (st.scales >> (16 * half)) & 0xFFu, f32x16{});
    acc = mfma32x32x64_fp4(Q.a4[1], make_uint4(st.code[4], st.code[5], st.code[6], st.code[7]), Q.s4[1],
                           (st.scales >> (16 * half + 8)) & 0xFFu, acc);
    float s = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; r++) s = fmaf(Q.wr[r], relu_bits(acc[r]), s);
    s += from_upper_half(s);
    return st.valid ? s : -INFINITY;
}
// The query state and score of the decode kernels for each operand format.
template <bool kFp4, bool kQ4>
using StreamQ = std::conditional_t<kQ4, StreamQuery4, StreamQuery<kFp4>>;
template <bool kFp4, bool kQ4>
CSA2_DEVINL float score_tile(const StreamQ<kFp4, kQ4>& Q, const StreamTile<kFp4>& st, int half) {
    if constexpr (kQ4)
        return stream_score4(Q, st, half);
    else
        return stream_score<kFp4>(Q, st, half);
}

// bf16 Full rows, line-ordered: a wave's 32-entry tile is 8 KiB of
// consecutive entries. Instruction j reads line j >> 2 (bytes 128 (j >> 2) ..
// +128) of entries 8 (j & 3) .. +8, one whole 128-byte line per 8 lanes, with
// non-temporal loads: each line is read once, by one instruction, so nothing
// has to stay cached for a later one (a plain streaming read reaches less
// bandwidth than a non-temporal one on this part).
// Buffer resource word 3 for the gfx9-family raw loads (32-bit data format),
// and the cache-policy operand that marks a load non-temporal (the nt bit).
constexpr int kRsrcFlags = 0x00020000;
constexpr int kCpolNt = 2;
struct LineTile {
    u32x4 v[8];
};
// rs: buffer resource over the chunk's valid entries (reads past them return
// zeros; their scores are discarded); off0: the tile's byte offset in it.
CSA2_DEVINL void line_load(__amdgpu_buffer_rsrc_t rs, int off0, int lane, LineTile& lt) {
    const int lo = (lane >> 3) * (kIdxDim * 2) + 16 * (lane & 7);
#pragma unroll
    for (int j = 0; j < 8; j++)
        lt.v[j] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, lo + 128 * (j >> 2), off0 + 2048 * (j & 3), kCpolNt));
}
// Reindex rows: the tile's 32 pool positions are 4 blocks of 8 consecutive
// entries (cb: their block ids, -1 for an empty slot); instruction j reads
// line j >> 2 of block j & 3's 8 entries, so every line is again read whole
// by one instruction. rs covers the sequence; an empty slot's offset lies past
// it and reads zeros.
CSA2_DEVINL void line_load_blocks(__amdgpu_buffer_rsrc_t rs, const int32_t* cb, int lane, LineTile& lt) {
    const int lo = (lane >> 3) * (kIdxDim * 2) + 16 * (lane & 7);
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const int blk = __builtin_amdgcn_readfirstlane(cb[j & 3]);
        const int so = blk >= 0 ? blk * (8 * kIdxDim * 2) : 0x7FFFF000;
        lt.v[j] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, lo + 128 * (j >> 2), so, kCpolNt));
    }
}
// The tile's operands in MFMA layout (lane (n, half) takes 16-byte unit
// 2j + half of entry n at step j), through a wave-private 4 KiB LDS stage, one
// line of the 32 entries at a time. Stage slot of 16-byte unit u (0..7) of
// entry e: row e >> 1, group 8 (e & 1) + (u ^ ((e >> 1) & 7)) of 16 -- writes
// (16 lanes: 2 entries x 8 units) and reads (16 lanes: 16 entries, one unit)
// both touch 16 distinct groups, so neither has bank conflicts. LDS
// operations of one wave complete in order, so the stage needs no barrier:
// the wave barriers only keep the compiler from moving accesses across.
CSA2_DEVINL void line_operands(const LineTile& lt, uint8_t* stage, int lane, bf16x8 (&b)[8]) {
    const int e_in = lane >> 3, u = lane & 7, n = lane & 31, half = lane >> 5;
#pragma unroll
    for (int r = 0; r < 2; r++) {
#pragma unroll
        for (int jj = 0; jj < 4; jj++) {
            const int e = 8 * jj + e_in;
            *reinterpret_cast<u32x4*>(stage + 256 * (e >> 1) + 16 * (8 * (e & 1) + (u ^ ((e >> 1) & 7)))) =
                lt.v[4 * r + jj];
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int s2 = 0; s2 < 4; s2++) {
            const int uu = 2 * s2 + half;
            b[4 * r + s2] = as_bf16x8(
                *reinterpret_cast<const u32x4*>(stage + 256 * (n >> 1) + 16 * (8 * (n & 1) + (uu ^ ((n >> 1) & 7)))));
        }
        __builtin_amdgcn_wave_barrier();
    }
}
CSA2_DEVINL float line_score(const StreamQuery<false>& Q, const bf16x8 (&b)[8], bool valid) {
    f32x16 acc = {};
#pragma unroll
    for (int j = 0; j < 8; j++) acc = mfma32x32x16(Q.a[j], b[j], acc);
    float s = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; r++) s = fmaf(Q.wr[r], relu_bits(acc[r]), s);
    s += from_upper_half(s);
    return valid ? s : -INFINITY;
}

// FP4 Full rows, line-ordered: a 32-entry tile is 2176 consecutive bytes (17
// lines, line-aligned when the sequence length is a multiple of 32), read as
// 136 16-byte units by 3 non-temporal instructions (the third on 8 lanes; the
// other lanes' offsets lie past the resource and read nothing).
struct LineTile4 {
    u32x4 v[3];
};
CSA2_DEVINL void line_load4(__amdgpu_buffer_rsrc_t rs, int off0, int lane, LineTile4& lt) {
#pragma unroll
    for (int i = 0; i < 3; i++) {
        const int vo = (i < 2 || lane < 8) ? 16 * (lane + 64 * i) : 0x40000000;
        lt.v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, vo, off0, kCpolNt));
    }
}
// The tile through a wave-private 3 KiB LDS stage into the per-entry layout
// of stream_load: lane (n, half) takes code dwords 8 half .. +8 and the scale
// dword of entry n (4-byte aligned reads at 68-byte strides).
CSA2_DEVINL void line_operands4(const LineTile4& lt, uint8_t* stage, int lane, StreamTile<true>& st) {
#pragma unroll
    for (int i = 0; i < 3; i++) *reinterpret_cast<u32x4*>(stage + 16 * (lane + 64 * i)) = lt.v[i];
    __builtin_amdgcn_wave_barrier();
    const uint8_t* e = stage + kKRec * (lane & 31);
    const uint32_t* c = reinterpret_cast<const uint32_t*>(e + 32 * (lane >> 5));
#pragma unroll
    for (int j = 0; j < 8; j++) st.code[j] = c[j];
    st.scales = *reinterpret_cast<const uint32_t*>(e + kIdxDim / 2);
    __builtin_amdgcn_wave_barrier();
}

template <bool kReindex, bool kFp4, bool kQ4 = false>
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

    StreamQ<kFp4, kQ4> Q;
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
        const float s = score_tile<kFp4, kQ4>(Q, st, half);
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
template <bool kFp4, bool kRe, int kFtThreads, int kFtChunk, bool kQ4 = false>
__global__ __launch_bounds__(kFtThreads, kFtThreads == 256 && !kRe ? 3 : 1) void index_topk_kernel(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w, const void* __restrict__ k_idx, int64_t N,
    int32_t q_per_seq, const int32_t* __restrict__ n_visible, const int32_t* __restrict__ cand_blocks, int32_t nb,
    int32_t k, int32_t nchunks, int32_t* __restrict__ out_idx, uint32_t* __restrict__ cand_key,
    int32_t* __restrict__ cand_col, float* __restrict__ block_scores, float* __restrict__ scores_dbg) {
    constexpr int kFtWaves = kFtThreads / 64;
    constexpr int kFtKpt = kFtChunk / kFtThreads;  // keys per thread
    static_assert(kFtKpt >= 4 && kFtKpt % 4 == 0, "keys are read from LDS as float4");
    // The chunk's scores, then (once every thread holds its keys in registers)
    // the selection's state in the same bytes: 32 KiB instead of 59 KiB at
    // 8192 entries, so twice as many workgroups stream K on a CU.
    constexpr size_t kScBytes = sizeof(float) * kFtChunk;
    constexpr size_t kSmem = kScBytes > sizeof(tk::RegTk<kFtThreads>) ? kScBytes : sizeof(tk::RegTk<kFtThreads>);
    __shared__ __attribute__((aligned(16))) uint8_t smem[kSmem];
    float* sc = reinterpret_cast<float*>(smem);
    tk::RegTk<kFtThreads>& sh = *reinterpret_cast<tk::RegTk<kFtThreads>*>(smem);
    // Reindex: the chunk's pool block ids (-1 past the pool)
    __shared__ int32_t cblk[kRe ? kFtChunk / 8 : 1];
    // line-ordered tiles (bf16 rows, FP4 Full rows): each wave's LDS stage
    constexpr bool kLine = !(kRe && kFp4);
    __shared__ __attribute__((aligned(16))) uint8_t stage[kLine ? kFtWaves : 1][kLine ? (kFp4 ? 3072 : 4096) : 16];
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

    static_assert(!kQ4 || kFp4, "MXFP4 Q pairs with MXFP4 K");
    StreamQ<kFp4, kQ4> Q;
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
        const float s = score_tile<kFp4, kQ4>(Q, st, half);
        const int p = t * 32 + col_in_tile;
        if (half == 0) sc[p] = s;
        if (scores_dbg && half == 0 && p < n) scores_dbg[q * ncols + c0 + p] = s;
        if (!kRe && block_scores) {
            const float m = max8_lanes(s);
            if (half == 0 && (lane & 7) == 0 && p < n) block_scores[q * nblk + ((c0 + p) >> 3)] = m;
        }
    };
    int t = wave;
    if constexpr (kLine && kFp4) {
        if ((N & 31) == 0) {
            // whole 32-entry tiles (the row is a multiple of 32): the chunk's
            // entries as one buffer resource, every tile read in whole lines
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint8_t*>(static_cast<const uint8_t*>(kseq) + c0 * kKRec), (short)0, n * kKRec, kRsrcFlags);
            auto lfinish = [&](int tt, const LineTile4& lt) {
                StreamTile<true> st;
                line_operands4(lt, stage[wave], lane, st);
                const int p = tt * 32 + col_in_tile;
                st.valid = c0 + p < nv;
                const float s = score_tile<true, kQ4>(Q, st, half);
                if (half == 0) sc[p] = s;
                if (scores_dbg && half == 0 && p < n) scores_dbg[q * ncols + c0 + p] = s;
                if (block_scores) {
                    const float m = max8_lanes(s);
                    if (half == 0 && (lane & 7) == 0 && p < n) block_scores[q * nblk + ((c0 + p) >> 3)] = m;
                }
            };
            if (t < ntile) {
                LineTile4 l0, l1;
                line_load4(rs, t * 32 * kKRec, lane, l0);
                while (true) {
                    const int t1 = t + kFtWaves;
                    if (t1 < ntile) line_load4(rs, t1 * 32 * kKRec, lane, l1);
                    lfinish(t, l0);
                    if (t1 >= ntile) break;
                    const int t2 = t1 + kFtWaves;
                    if (t2 < ntile) line_load4(rs, t2 * 32 * kKRec, lane, l0);
                    lfinish(t1, l1);
                    if (t2 >= ntile) break;
                    t = t2;
                }
            }
            t = ntile;  // done: the per-entry path below runs no tile
        }
    }
    if constexpr (kLine && !kFp4) {
        // Full: the chunk's entries below nv; Reindex: the whole sequence (its
        // byte offsets must fit an int: N < 2^23, else the per-entry path runs)
        if (!kRe || N < (int64_t(1) << 23)) {
            const int64_t nvalid = nv - c0 < 0 ? 0 : (nv - c0 < kFtChunk ? nv - c0 : kFtChunk);
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint16_t*>(static_cast<const uint16_t*>(kseq) + (kRe ? 0 : c0) * kIdxDim), (short)0,
                (int)((kRe ? N : nvalid) * kIdxDim * 2), kRsrcFlags);
            auto lload = [&](int tt, LineTile& lt) {
                if constexpr (kRe)
                    line_load_blocks(rs, &cblk[tt * 4], lane, lt);
                else
                    line_load(rs, tt * 8192, lane, lt);
            };
            auto lfinish = [&](int tt, const LineTile& lt) {
                bf16x8 b[8];
                line_operands(lt, stage[wave], lane, b);
                const int p = tt * 32 + col_in_tile;
                bool valid;
                if constexpr (kRe) {
                    const int32_t blk = p < n ? cblk[p >> 3] : -1;
                    valid = blk >= 0 && (int64_t)blk * 8 + (p & 7) < nv;
                } else {
                    valid = c0 + p < nv;
                }
                const float s = line_score(Q, b, valid);
                if (half == 0) sc[p] = s;
                if (scores_dbg && half == 0 && p < n) scores_dbg[q * ncols + c0 + p] = s;
                if (!kRe && block_scores) {
                    const float m = max8_lanes(s);
                    if (half == 0 && (lane & 7) == 0 && p < n) block_scores[q * nblk + ((c0 + p) >> 3)] = m;
                }
            };
            if (t < ntile) {
                LineTile l0, l1;
                lload(t, l0);
                while (true) {
                    const int t1 = t + kFtWaves;
                    if (t1 < ntile) lload(t1, l1);
                    lfinish(t, l0);
                    if (t1 >= ntile) break;
                    const int t2 = t1 + kFtWaves;
                    if (t2 < ntile) lload(t2, l0);
                    lfinish(t1, l1);
                    if (t2 >= ntile) break;
                    t = t2;
                }
            }
            t = ntile;  // done: the per-entry path below runs no tile
        }
    }
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
    lds_barrier();  // the score buffer becomes the selection's state
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
constexpr int kPfChunk = 4096;         // entries per workgroup (scores written out)
constexpr int kPfSelK = 512;           // largest k of the fused prefill selection
constexpr int kPfBuf = 960;            // candidate slots per query (a multiple of 64; 2 workgroups fit a CU)
constexpr int kPfBufQ4 = 896;          // the same for the MXFP4 Q x K variant (3 workgroups fit a CU)
constexpr int kPfLow = kPfSelK + 128;  // buffers at or below this are left alone in a round
constexpr int kPfSlack = 64;           // a round's compaction may keep up to k + kPfSlack (<= kPfLow)
static_assert(kPfSelK + kPfSlack <= kPfLow, "a compacted buffer must stay out of the next round");
static_assert(kPfBufQ4 - 64 > kPfLow && kPfBufQ4 % 64 == 0, "room for a tile after a compaction");
constexpr int64_t kPfMaxChunk = 65536; // entry offsets within a chunk fit 16 bits

// Registers of one prefill tile load: bf16 K 4 units of 16 bytes per thread;
// FP4 K 16 code bytes (one 32-channel block) and that block's scale per thread.
template <bool kFp4>
struct PfPre;
template <>
struct PfPre<false> {
    uint4 v[4];
};
template <>
struct PfPre<true> {
    uint4 v;
    float x;  // the block's E8M0 scale as a float
};

// kQ4 (MXFP4 Q and K): thread (entry tid/4, block tid%4) copies the block's 16
// code bytes and its scale byte unchanged; nothing is decoded.
struct PfPreQ4 {
    uint4 v;
    uint32_t sb;  // the block's E8M0 scale byte
};
constexpr int kPfRowQ4 = 80;  // LDS row of a raw MXFP4 entry: 64 code bytes, 4 scales, 12 pad

// kSel: scoring fused with the per-query Top-k (k <= kPfSelK; the DeepSelect
// selection eogee.com report 3.5 names, for the prefill chunk): no score row
// is written. Each wave owns its 2 queries' candidate buffers in LDS (keys and
// 16-bit entry offsets within the chunk) and sees their entries in ascending
// order. A query's threshold T is a score that at least k buffered entries
// reach; an entry can only enter the query's Top-k if its score beats T (an
// equal or lower score arrives after k buffered ones that rank above it).
// Passing entries are appended; the buffers are compacted (tk::wave_keep_topk)
// only at tile boundaries, all waves in the same round (the waves meet at
// every tile's barrier, so one wave compacting alone would stall the other
// three). A round's compaction keeps every entry at or above a new T that
// between k and k + kPfSlack of them reach: the radix search stops there
// instead of resolving the exact k-th key. A random row of n entries appends
// about k (1 + ln(n / k)) entries, so rounds are few. At the end an exact
// compaction leaves each query's k best, which go out in entry order: final
// indices when the row is one chunk, else (key, entry) candidates that the
// Top-K merge combines. `scores`, when given, still receives the score row (a
// checking aid).
// kQ4: the indexer Q is MXFP4 too (one 68-byte entry per head, the K entry
// format; eogee.com report 3.4: the indexer Q/K already ran in FP4), and the
// contraction runs on the scaled FP4 MFMA straight from the stored codes:
// 4 MFMAs of 32x32x64 per 32-entry group where bf16 operands take 16 of
// 32x32x16, and the K tile is copied to LDS undecoded (80-byte rows).
template <bool kFp4, bool kBlk, bool kSel, bool kQ4 = false>
__global__ __launch_bounds__(256, 2) void index_prefill_kernel(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w, const void* __restrict__ k_idx, int64_t N,
    int32_t q_per_seq, const int32_t* __restrict__ n_visible, float* __restrict__ scores,
    float* __restrict__ block_scores, int32_t nchunks, int64_t chunk_len, int32_t k, int32_t* __restrict__ out_idx,
    uint32_t* __restrict__ cand_key, int32_t* __restrict__ cand_col) {
    // candidate slots per query: the MXFP4 variant's smaller tiles and buffers
    // (53 KB with the selection) leave room for a third workgroup per CU
    constexpr int kBuf = kQ4 ? kPfBufQ4 : kPfBuf;
    constexpr int kHigh = kBuf - 64;  // compact before a tile's 64 entries could overflow
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][kPfSub * (kQ4 ? kPfRowQ4 : kPfRow)];
    // kSel: candidate keys and entry offsets of the workgroup's 8 queries, and
    // each wave's "a buffer is nearly full" flag per tile parity
    __shared__ uint32_t bkey[kSel ? kPfQueries : 1][kSel ? kBuf : 1];
    __shared__ uint16_t bid[kSel ? kPfQueries : 1][kSel ? kBuf : 1];
    __shared__ __attribute__((aligned(16))) uint32_t full_flag[2][4];
    const int b = blockIdx.x;
    int chunk, qg;
    if (!kSel && (nchunks & 7) == 0) {
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

    static_assert(!kQ4 || kFp4, "MXFP4 Q pairs with MXFP4 K");
    bf16x8 aa[8], ab[8];
    // kQ4: K-step s uses scale block 2s + half of head col_in_tile: 16 code
    // bytes (dword loads: entries are 4-byte aligned) and the block's scale
    uint4 qa4[2], qb4[2];
    uint32_t qas[2], qbs[2];
    if constexpr (kQ4) {
        const uint8_t* q8 = reinterpret_cast<const uint8_t*>(q_idx);
        const uint8_t* ea = q8 + (qa * kIdxHeads + col_in_tile) * kKRec;
        const uint8_t* eb = q8 + (qb * kIdxHeads + col_in_tile) * kKRec;
        const uint32_t sca = *reinterpret_cast<const uint32_t*>(ea + kIdxDim / 2);
        const uint32_t scb = *reinterpret_cast<const uint32_t*>(eb + kIdxDim / 2);
#pragma unroll
        for (int st = 0; st < 2; st++) {
            const int blk = 2 * st + half;
            const uint32_t* ca = reinterpret_cast<const uint32_t*>(ea + 16 * blk);
            const uint32_t* cb = reinterpret_cast<const uint32_t*>(eb + 16 * blk);
            qa4[st] = make_uint4(ca[0], ca[1], ca[2], ca[3]);
            qb4[st] = make_uint4(cb[0], cb[1], cb[2], cb[3]);
            qas[st] = (sca >> (8 * blk)) & 0xFFu;
            qbs[st] = (scb >> (8 * blk)) & 0xFFu;
        }
    } else {
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
    const int64_t e_begin = (int64_t)chunk * chunk_len;
    int64_t e_end = (e_begin + chunk_len < N) ? e_begin + chunk_len : N;
    // Entries no query of the workgroup sees need no products: the selection
    // skips them; a written score row gets -inf there from plain stores after
    // the tile loop (whole tiles past the largest visible length).
    int64_t e_fill = e_end;  // first entry of the -inf fill
    if (kSel || scores) {
        int64_t nvmax = 0;
        for (int i = 0; i < kPfQueries; i++)
            nvmax = max(nvmax, n_visible ? (int64_t)n_visible[(int64_t)qg * kPfQueries + i] : N);
        if (kSel && !scores) {
            e_end = e_end < nvmax ? e_end : nvmax;
        } else if (!kSel) {
            const int64_t t_end = e_begin + (nvmax > e_begin ? (nvmax - e_begin + kPfSub - 1) / kPfSub * kPfSub : 0);
            e_fill = t_end < e_end ? t_end : e_end;
        }
    }
    const int64_t e_tiles = kSel ? e_end : e_fill;  // entries the tile loop scores
    const int nsub = e_tiles > e_begin ? (int)((e_tiles - e_begin + kPfSub - 1) / kPfSub) : 0;
    const int64_t nblk = (N + 7) >> 3;

    // Tile loads into registers. bf16 K: 4 16-byte units per thread of the
    // 64 x 256 B tile. FP4 K: thread (entry tid/4, quarter tid%4) takes 16 code
    // bytes (32 channels, one scale block) and that block's scale.
    using Pre = std::conditional_t<kQ4, PfPreQ4, PfPre<kFp4>>;
    // The tile's first entry is uniform: a scalar base plus 32-bit lane offsets,
    // and rows past the sequence re-read its last entry (their scores are
    // never kept).
    auto gload = [&](int st) {
        Pre p;
        const int64_t t0 = e_begin + (int64_t)st * kPfSub;
        const int lim = (int)(N - 1 - t0 < kPfSub - 1 ? N - 1 - t0 : kPfSub - 1);
        if constexpr (kQ4) {
            const int row = tid >> 2, qq = tid & 3;
            const uint8_t* e = kfseq + t0 * kKRec + (uint32_t)((row < lim ? row : lim) * kKRec);
            const uint32_t* src = reinterpret_cast<const uint32_t*>(e) + 4 * qq;
            p.v = make_uint4(src[0], src[1], src[2], src[3]);
            p.sb = e[kIdxDim / 2 + qq];
        } else if constexpr (kFp4) {
            const int row = tid >> 2, qq = tid & 3;
            const uint8_t* e = kfseq + t0 * kKRec + (uint32_t)((row < lim ? row : lim) * kKRec);
            const uint32_t* src = reinterpret_cast<const uint32_t*>(e) + 4 * qq;
            p.v = make_uint4(src[0], src[1], src[2], src[3]);
            p.x = __uint_as_float((uint32_t)e[kIdxDim / 2 + qq] << 23);
        } else {
            const uint4* tb = reinterpret_cast<const uint4*>(kseq + t0 * kIdxDim);
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int u = i * 256 + tid;  // 16-byte unit within the 64 x 256 B tile
                const int row = u >> 4, c16 = u & 15;
                p.v[i] = tb[(uint32_t)((row < lim ? row : lim) * 16 + c16)];
            }
        }
        return p;
    };
    auto lstore = [&](int buf, const Pre& p) {
        if constexpr (kQ4) {
            const int row = tid >> 2, qq = tid & 3;
            *reinterpret_cast<uint4*>(&lds[buf][row * kPfRowQ4 + 16 * qq]) = p.v;
            lds[buf][row * kPfRowQ4 + kIdxDim / 2 + qq] = (uint8_t)p.sb;
        } else if constexpr (kFp4) {
            const int row = tid >> 2, qq = tid & 3;
            uint8_t* dst = &lds[buf][row * kPfRow + qq * 64];
            const uint32_t c[4] = {p.v.x, p.v.y, p.v.z, p.v.w};
#pragma unroll
            for (int i = 0; i < 4; i++) *reinterpret_cast<bf16x8*>(dst + 16 * i) = fp4x8_to_bf16(c[i], p.x);
        } else {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int u = i * 256 + tid;
                const int row = u >> 4, c16 = u & 15;
                *reinterpret_cast<uint4*>(&lds[buf][row * kPfRow + c16 * 16]) = p.v[i];
            }
        }
    };
    // ReLU-weighted head sums of both queries' 32 x 32 blocks, one query per
    // half-wave: each lane sums its 16 heads of each query, and one half-wave
    // swap hands lanes 0..31 both halves of query a and lanes 32..63 both
    // halves of query b.
    // entry positions fit 32 bits (N < 2^31)
    const int32_t nv_mine = (int32_t)(half ? nvb : nva);
    const int32_t n32 = (int32_t)N;
    auto head_sums = [&](const f32x16& acca, const f32x16& accb, int32_t col) {
        float sa = 0.0f, sb = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; r++) {
            sa = fmaf(wa[r], relu_bits(acca[r]), sa);
            sb = fmaf(wb[r], relu_bits(accb[r]), sb);
        }
        const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(sa), __float_as_uint(sb), false, false);
        const float s = __uint_as_float(x[0]) + __uint_as_float(x[1]);
        return col < nv_mine ? s : -INFINITY;
    };
    const int64_t q_mine = half ? qb : qa;
    float* srow = scores ? scores + q_mine * N : nullptr;  // this half-wave's score row
    float* brow = kBlk ? block_scores + q_mine * nblk : nullptr;
    // kSel state of the wave's two queries (wave-uniform): buffered candidates
    // and the score an entry must beat, as a float (-inf: any valid score).
    // key(s) > key(t) <=> s > t for every score s (NaN and -inf never pass),
    // so the common case -- no lane passes once the threshold has settled --
    // costs one compare and one branch per 32 entries.
    uint32_t na = 0, nb = 0;
    float ta = -INFINITY, tb = -INFINITY;
    const int slot_a = 2 * wave, slot_b = 2 * wave + 1;
    auto store = [&](float s, float m, int32_t col) {
        if constexpr (kSel) {
            if (srow && col < n32) srow[(uint32_t)col] = s;
            const bool pass = s > (half ? tb : ta);
            const uint64_t bal = __ballot(pass);
            if (bal == 0) return;
            const uint32_t ml = (uint32_t)bal, mh = (uint32_t)(bal >> 32);
            // rank among the passing lanes of this half-wave (lanes 0..31: query a)
            const uint32_t rank = __builtin_amdgcn_mbcnt_hi(half ? mh : 0u, __builtin_amdgcn_mbcnt_lo(half ? 0u : ml, 0u));
            if (pass) {
                const uint32_t pos = (half ? nb : na) + rank;
                bkey[half ? slot_b : slot_a][pos] = tk::score_key(s);
                bid[half ? slot_b : slot_a][pos] = (uint16_t)(col - (int32_t)e_begin);
            }
            na += (uint32_t)__builtin_popcount(ml);
            nb += (uint32_t)__builtin_popcount(mh);
        } else if (col < n32) {
            // written once and read by a later call: streamed past the caches
            // that hold K (measured 2% faster than plain stores at 4096 x 65536)
            __builtin_nontemporal_store(s, srow + (uint32_t)col);
            if (kBlk && (lane & 7) == 0) __builtin_nontemporal_store(m, brow + ((uint32_t)col >> 3));
        }
    };
    // One group = 32 entries (rows h2*32.. of an LDS tile) for both queries:
    // 8 fragment reads, 16 MFMAs. The epilogue of the previous group runs in
    // the same straight-line block so the scheduler can put its VALU work in
    // the shadow of these MFMAs.
    auto group = [&](int buf, int h2, f32x16& acca, f32x16& accb, const f32x16& pa, const f32x16& pb, int32_t pcol,
                     float (&out)[2]) {
        if constexpr (kQ4) {
            __builtin_amdgcn_s_setprio(1);
            // entry h2*32 + col_in_tile: scale blocks 2s + half for K-steps s = 0, 1
            const uint8_t* rowp = lds[buf] + (h2 * 32 + col_in_tile) * kPfRowQ4;
            const uint4 b0 = *reinterpret_cast<const uint4*>(rowp + 16 * half);
            const uint4 b1 = *reinterpret_cast<const uint4*>(rowp + 16 * (2 + half));
            const uint32_t sc = *reinterpret_cast<const uint32_t*>(rowp + kIdxDim / 2);
            const uint32_t s0 = (sc >> (8 * half)) & 0xFFu, s1 = (sc >> (8 * (2 + half))) & 0xFFu;
            acca = mfma32x32x64_fp4(qa4[0], b0, qas[0], s0, f32x16{});
            accb = mfma32x32x64_fp4(qb4[0], b0, qbs[0], s0, f32x16{});
            acca = mfma32x32x64_fp4(qa4[1], b1, qas[1], s1, acca);
            accb = mfma32x32x64_fp4(qb4[1], b1, qbs[1], s1, accb);
            out[0] = head_sums(pa, pb, pcol);
            out[1] = kBlk ? max8_lanes(out[0]) : 0.0f;
            __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);  // fragment reads first
#pragma unroll
            for (int i = 0; i < 4; i++) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);
            }
            __builtin_amdgcn_s_setprio(0);
            return;
        }
        // the wave issuing its MFMAs goes first on the SIMD
        __builtin_amdgcn_s_setprio(1);
        const uint8_t* rowp = lds[buf] + (h2 * 32 + col_in_tile) * kPfRow + half * 16;
        bf16x8 bj[8];
#pragma unroll
        for (int j = 0; j < 8; j++) bj[j] = as_bf16x8(*reinterpret_cast<const uint4*>(rowp + j * 32));
        acca = f32x16{};
        accb = f32x16{};
#pragma unroll
        for (int j = 0; j < 8; j++) {
            acca = mfma32x32x16(aa[j], bj[j], acca);
            accb = mfma32x32x16(ab[j], bj[j], accb);
        }
        out[0] = head_sums(pa, pb, pcol);
        out[1] = kBlk ? max8_lanes(out[0]) : 0.0f;  // block maxima only when asked for
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // fragment reads first
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
#pragma unroll
        for (int i = 0; i < 16; i++) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
        }
        __builtin_amdgcn_s_setprio(0);
    };

    const int64_t tile_base = e_begin;
    lstore(0, gload(0));
    lds_barrier();
    f32x16 pa, pb, ca, cb;
    float out[2];
    {
        const f32x16 z = {};
        group(0, 0, pa, pb, z, z, n32, out);  // no previous group: its results are discarded
    }
    for (int st = 0; st < nsub; st++) {
        const bool more = st + 1 < nsub;
        // the last iteration re-reads tile 0 (in bounds) and discards it
        const Pre nxt = gload(more ? st + 1 : 0);
        const int32_t col0 = (int32_t)tile_base + st * kPfSub + col_in_tile;
        group(st & 1, 1, ca, cb, pa, pb, col0, out);
        store(out[0], out[1], col0);
        if (more) lstore((st + 1) & 1, nxt);
        if constexpr (kSel) {
            // 64 more entries per query arrive before the next barrier
            if (lane == 0) full_flag[st & 1][wave] = (uint32_t)(max(na, nb) > (uint32_t)kHigh);
        }
        lds_barrier();
        // After the last tile this reads the stale buffer; those results are never stored.
        group((st + 1) & 1, 0, pa, pb, ca, cb, col0 + 32, out);
        if constexpr (kSel) {
            // read after the group's fragment reads are issued, so the wait is theirs
            const uint4 f = *reinterpret_cast<const uint4*>(full_flag[st & 1]);
            if (f.x | f.y | f.z | f.w) {
                // a compaction round: every wave compacts its fuller buffers
                if (na > (uint32_t)kPfLow)
                    ta = tk::key_score(
                        tk::wave_keep_topk<kBuf>(bkey[slot_a], bid[slot_a], na, (uint32_t)k, (uint32_t)kPfSlack, na));
                if (nb > (uint32_t)kPfLow)
                    tb = tk::key_score(
                        tk::wave_keep_topk<kBuf>(bkey[slot_b], bid[slot_b], nb, (uint32_t)k, (uint32_t)kPfSlack, nb));
            }
        }
        store(out[0], out[1], col0 + 32);
    }
    if (!kSel && e_fill < e_end) {
        // -inf past the tiles scored (every entry there is invisible to all
        // of the workgroup's queries), and their blocks' maxima; e_fill is
        // then a multiple of the tile, so no block straddles it
        for (int i = 0; i < kPfQueries; i++) {
            const int64_t q = (int64_t)qg * kPfQueries + i;
            for (int64_t c = e_fill + tid; c < e_end; c += 256) __builtin_nontemporal_store(-INFINITY, scores + q * N + c);
            if constexpr (kBlk)
                for (int64_t b = (e_fill >> 3) + tid; b < ((e_end + 7) >> 3); b += 256)
                    __builtin_nontemporal_store(-INFINITY, block_scores + q * nblk + b);
        }
    }
    if constexpr (kSel) {
        // each query's k best, in entry order
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const int slot = h ? slot_b : slot_a;
            uint32_t n = h ? nb : na;
            if (n > (uint32_t)k) tk::wave_keep_topk<kBuf>(bkey[slot], bid[slot], n, (uint32_t)k, 0u, n);  // exact: n = k
            const int64_t q = h ? qb : qa;
            if (nchunks == 1) {
                for (int i = lane; i < k; i += 64) out_idx[q * k + i] = i < (int)n ? (int32_t)(e_begin + bid[slot][i]) : -1;
            } else {
                const int64_t base = (q * nchunks + chunk) * (int64_t)k;
                for (int i = lane; i < k; i += 64) {
                    cand_key[base + i] = i < (int)n ? bkey[slot][i] : 0u;
                    cand_col[base + i] = i < (int)n ? (int32_t)(e_begin + bid[slot][i]) : -1;
                }
            }
        }
    }
}

}  // namespace

int launch_index_full(const uint16_t* q_idx, const float* w, const void* k, bool kfp4, int64_t N, int32_t nq,
                      int32_t q_per_seq, const int32_t* n_visible, float* scores, int32_t block_size,
                      float* block_scores, hipStream_t s, bool qfp4) {
    if (nq == 0) return 0;
    float* bs = block_size > 0 ? block_scores : nullptr;
    if (qfp4 && q_per_seq % kPfQueries == 0)
        return launch_index_full_fp4qk(reinterpret_cast<const uint8_t*>(q_idx), w, static_cast<const uint8_t*>(k), N,
                                       nq, q_per_seq, n_visible, scores, block_size, block_scores, s);
    if (q_per_seq % kPfQueries == 0) {
        const int32_t nchunks = (int32_t)((N + kPfChunk - 1) / kPfChunk);
        const int64_t grid = (int64_t)(nq / kPfQueries) * nchunks;
#define CSA2_PF(FP4, BLK)                                                                                     \
    hipLaunchKernelGGL((index_prefill_kernel<FP4, BLK, false>), dim3((unsigned)grid), dim3(256), 0, s, q_idx, w, k, \
                       N, q_per_seq, n_visible, scores, bs, nchunks, (int64_t)kPfChunk, 0, (int32_t*)nullptr,       \
                       (uint32_t*)nullptr, (int32_t*)nullptr)
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
    if (qfp4)
        hipLaunchKernelGGL((index_stream_kernel<false, true, true>), grid, dim3(kStreamThreads), 0, s, q_idx, w, k, N,
                           q_per_seq, n_visible, (const int32_t*)nullptr, 0, scores, bs, (int32_t*)nullptr, N, ntiles,
                           (int32_t)wgs_per_q, (int32_t)tpw);
    else if (kfp4)
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
                      float* scores_dbg, void* ws, hipStream_t s, bool qfp4) {
    if (nq == 0) return 0;
    const FtWs f = ft_ws(ws, nq, N, topk);
    const bool small = index_topk_chunk_len(nq, N) == 4096;
    const dim3 grid((unsigned)((int64_t)nq * f.c));
#define CSA2_FT(FP4, NT, CH, Q4)                                                                               \
    hipLaunchKernelGGL((index_topk_kernel<FP4, false, NT, CH, Q4>), grid, dim3(NT), 0, s, q_idx, w, k, N, 1,       \
                       n_visible, nullptr, 0, topk, f.c, out_idx, f.ck, f.cc, block_scores, scores_dbg)
    if (qfp4) {
        if (small) CSA2_FT(true, 512, 4096, true); else CSA2_FT(true, 512, 8192, true);
    } else if (kfp4) {
        if (small) CSA2_FT(true, 512, 4096, false); else CSA2_FT(true, 512, 8192, false);
    } else {
        if (small) CSA2_FT(false, 256, 4096, false); else CSA2_FT(false, 256, 8192, false);
    }
#undef CSA2_FT
    return 0;
}

// Scratch of csa2_index_topk_noalloc, for callers that cannot allocate: the
// per-chunk candidates of one call live in this file-scope device array, of
// which every GPU the library runs on holds its own copy until the process
// ends. Every selection slot is rewritten by each call, so nothing needs
// clearing; calls that overlap on one GPU share the array and race.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

size_t index_topk_noalloc_capacity() { return kNoAllocScratchBytes; }

// Device address of the current device's copy of `scratch`. In host code the
// array's name is only a stand-in, so the address is looked up once per
// device (with that device current) and kept.
void* index_topk_noalloc_scratch(hipError_t* err) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        *err = e != hipSuccess ? e : hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
            return nullptr;
        }
        addr[dev] = p;
    }
    *err = hipSuccess;
    return addr[dev];
}

int launch_index_topk_merge(int64_t N, int32_t nq, int32_t topk, int32_t* out_idx, void* ws, hipStream_t s) {
    if (nq == 0) return 0;
    const FtWs f = ft_ws(ws, nq, N, topk);
    if (f.c > 1) launch_topk_merge(nq, topk, f.c, f.ck, f.cc, out_idx, f.ck2, f.cc2, s);
    return 0;
}

// The hierarchical Full layer's two selections after the scoring launch: the
// Top-k merge of the chunks' candidates and the pool's Top-pool_k blocks over
// the block maxima do not depend on each other, so each level of the two runs
// in one launch (two launches instead of four at 8 x 1M entries).
static size_t align256(size_t b) { return (b + 255) & ~size_t(255); }
size_t index_topk_pool_workspace_bytes(int32_t nq, int64_t N, int32_t k, int32_t pool_k) {
    return align256(index_topk_workspace_bytes(nq, N, k)) + topk_workspace_bytes(nq, (N + 7) / 8, pool_k);
}
int launch_index_topk_merge_pool(int64_t N, int32_t nq, int32_t topk, int32_t* out_idx, const float* block_scores,
                                 int32_t pool_k, int32_t* cand_blocks, void* ws, hipStream_t s) {
    if (nq == 0) return 0;
    const FtWs f = ft_ws(ws, nq, N, topk);
    void* ws_b = ws ? static_cast<void*>(static_cast<uint8_t*>(ws) + align256(index_topk_workspace_bytes(nq, N, topk)))
                    : nullptr;
    const int64_t nblk = (N + 7) / 8;
    if (!launch_topk_merge_select(nq, topk, f.c, f.ck, f.cc, out_idx, f.ck2, f.cc2, block_scores, nq, nblk, pool_k,
                                  cand_blocks, ws_b, s)) {
        launch_index_topk_merge(N, nq, topk, out_idx, ws, s);
        launch_topk(block_scores, nq, nblk, nblk, nullptr, pool_k, nullptr, cand_blocks, ws_b, s);
    }
    return 0;
}

// Reindex scoring fused with the Top-K: the chunk kernel in Reindex mode
// (256 threads for either key format), then the merge of the chunks'
// candidates when a row has more than one chunk.
int launch_index_reindex_topk(const uint16_t* q_idx, const float* w, const void* k, bool kfp4, int64_t N, int32_t nq,
                              int32_t q_per_seq, const int32_t* n_visible, const int32_t* cand_blocks, int32_t nb,
                              int32_t topk, int32_t* out_idx, float* pool_scores, void* ws, hipStream_t s, bool qfp4) {
    if (nq == 0) return 0;
    const FtWs f = ft_ws_chunks(ws, nq, reindex_topk_chunks(nq, nb, topk), topk);
    const int64_t len = reindex_topk_chunk_len(nq, (int64_t)nb * 8, topk);
    const dim3 grid((unsigned)((int64_t)nq * f.c));
#define CSA2_RT(FP4, CH, Q4)                                                                                    \
    hipLaunchKernelGGL((index_topk_kernel<FP4, true, 256, CH, Q4>), grid, dim3(256), 0, s, q_idx, w, k, N,       \
                       q_per_seq, n_visible, cand_blocks, nb, topk, f.c, out_idx, f.ck, f.cc, nullptr, pool_scores)
#define CSA2_RT_LEN(FP4, Q4)                   \
    switch (len) {                             \
        case 1024: CSA2_RT(FP4, 1024, Q4); break; \
        case 2048: CSA2_RT(FP4, 2048, Q4); break; \
        case 4096: CSA2_RT(FP4, 4096, Q4); break; \
        default: CSA2_RT(FP4, 8192, Q4); break;   \
    }
    if (qfp4) {
        CSA2_RT_LEN(true, true)
    } else if (kfp4) {
        CSA2_RT_LEN(true, false)
    } else {
        CSA2_RT_LEN(false, false)
    }
#undef CSA2_RT_LEN
#undef CSA2_RT
    if (f.c > 1) launch_topk_merge(nq, topk, f.c, f.ck, f.cc, out_idx, f.ck2, f.cc2, s);
    return 0;
}

// Fused prefill scoring + Top-K: whole rows of up to 65536 entries per
// workgroup (fewest candidates, fewest compactions), cut into more chunks
// only when the batch would leave fewer than 512 workgroups (chunks of at
// least 4096 entries, multiples of the 64-entry tile).
int64_t prefill_topk_chunk_len(int32_t nq, int64_t N, bool q4) {
    const int64_t groups = nq / kPfQueries > 0 ? nq / kPfQueries : 1;
    int64_t nch = (N + kPfMaxChunk - 1) / kPfMaxChunk;
    // workgroups wanted: 512 (two per CU) for bf16 products; the MXFP4 variant
    // holds three per CU and wants two full rounds of them
    const int64_t wgs = q4 ? 1536 : 512;
    const int64_t want = std::min((wgs + groups - 1) / groups, (N + 4095) / 4096);
    nch = nch > want ? nch : want;
    const int64_t len = (N + nch - 1) / nch;
    return (len + kPfSub - 1) / kPfSub * kPfSub;
}
int32_t prefill_topk_chunks(int32_t nq, int64_t N, bool q4) {
    const int64_t len = prefill_topk_chunk_len(nq, N, q4);
    return (int32_t)((N + len - 1) / len);
}
bool prefill_topk_fits(int32_t nq, int64_t N, int32_t k) {
    return k >= 1 && k <= kPfSelK && chunks_fit(prefill_topk_chunks(nq, N, false), k) &&
           chunks_fit(prefill_topk_chunks(nq, N, true), k);
}
// one workspace size serves both variants
size_t prefill_topk_workspace_bytes(int32_t nq, int64_t N, int32_t k) {
    return std::max(chunks_workspace_bytes(nq, prefill_topk_chunks(nq, N, false), k),
                    chunks_workspace_bytes(nq, prefill_topk_chunks(nq, N, true), k));
}

int launch_index_prefill_topk(const uint16_t* q_idx, const float* w, const void* k, bool kfp4, int64_t N, int32_t nq,
                              int32_t q_per_seq, const int32_t* n_visible, int32_t topk, int32_t* out_idx,
                              float* scores_dbg, void* ws, hipStream_t s) {
    if (nq == 0) return 0;
    const FtWs f = ft_ws_chunks(ws, nq, prefill_topk_chunks(nq, N, false), topk);
    const int64_t len = prefill_topk_chunk_len(nq, N, false);
    const dim3 grid((unsigned)((int64_t)(nq / kPfQueries) * f.c));
    if (kfp4)
        hipLaunchKernelGGL((index_prefill_kernel<true, false, true>), grid, dim3(256), 0, s, q_idx, w, k, N,
                           q_per_seq, n_visible, scores_dbg, (float*)nullptr, f.c, len, topk, out_idx, f.ck, f.cc);
    else
        hipLaunchKernelGGL((index_prefill_kernel<false, false, true>), grid, dim3(256), 0, s, q_idx, w, k, N,
                           q_per_seq, n_visible, scores_dbg, (float*)nullptr, f.c, len, topk, out_idx, f.ck, f.cc);
    if (f.c > 1) launch_topk_merge(nq, topk, f.c, f.ck, f.cc, out_idx, f.ck2, f.cc2, s);
    return 0;
}

int launch_index_full_fp4qk(const uint8_t* q_fp4, const float* w, const uint8_t* k_fp4, int64_t N, int32_t nq,
                            int32_t q_per_seq, const int32_t* n_visible, float* scores, int32_t block_size,
                            float* block_scores, hipStream_t s) {
    if (nq == 0) return 0;
    float* bs = block_size > 0 ? block_scores : nullptr;
    const int32_t nchunks = (int32_t)((N + kPfChunk - 1) / kPfChunk);
    const dim3 grid((unsigned)((int64_t)(nq / kPfQueries) * nchunks));
    const uint16_t* q = reinterpret_cast<const uint16_t*>(q_fp4);  // the kernel reads it as bytes
    if (bs)
        hipLaunchKernelGGL((index_prefill_kernel<true, true, false, true>), grid, dim3(256), 0, s, q, w, k_fp4, N,
                           q_per_seq, n_visible, scores, bs, nchunks, (int64_t)kPfChunk, 0, (int32_t*)nullptr,
                           (uint32_t*)nullptr, (int32_t*)nullptr);
    else
        hipLaunchKernelGGL((index_prefill_kernel<true, false, false, true>), grid, dim3(256), 0, s, q, w, k_fp4, N,
                           q_per_seq, n_visible, scores, bs, nchunks, (int64_t)kPfChunk, 0, (int32_t*)nullptr,
                           (uint32_t*)nullptr, (int32_t*)nullptr);
    return 0;
}

int launch_index_prefill_topk_fp4qk(const uint8_t* q_fp4, const float* w, const uint8_t* k_fp4, int64_t N,
                                    int32_t nq, int32_t q_per_seq, const int32_t* n_visible, int32_t topk,
                                    int32_t* out_idx, float* scores_dbg, void* ws, hipStream_t s) {
    if (nq == 0) return 0;
    const FtWs f = ft_ws_chunks(ws, nq, prefill_topk_chunks(nq, N, true), topk);
    const int64_t len = prefill_topk_chunk_len(nq, N, true);
    const dim3 grid((unsigned)((int64_t)(nq / kPfQueries) * f.c));
    hipLaunchKernelGGL((index_prefill_kernel<true, false, true, true>), grid, dim3(256), 0, s,
                       reinterpret_cast<const uint16_t*>(q_fp4), w, k_fp4, N, q_per_seq, n_visible, scores_dbg,
                       (float*)nullptr, f.c, len, topk, out_idx, f.ck, f.cc);
    if (f.c > 1) launch_topk_merge(nq, topk, f.c, f.ck, f.cc, out_idx, f.ck2, f.cc2, s);
    return 0;
}

int launch_index_reindex(const uint16_t* q_idx, const float* w, const void* k, bool kfp4, int64_t N, int32_t nq,
                         int32_t q_per_seq, const int32_t* n_visible, const int32_t* cand_blocks, int32_t nb,
                         float* pool_scores, int32_t* pool_ids, hipStream_t s, bool qfp4) {
    if (nq == 0) return 0;
    const int64_t ncols = (int64_t)nb * 8;
    const int64_t ntiles = (ncols + 31) / 32;
    const int64_t total = ntiles * nq;
    int64_t tpw = (total + 2047) / 2048;
    tpw = ((tpw + kStreamWaves - 1) / kStreamWaves) * kStreamWaves;
    if (tpw < kStreamWaves) tpw = kStreamWaves;
    const int64_t wgs_per_q = (ntiles + tpw - 1) / tpw;
    const dim3 grid((unsigned)(wgs_per_q * nq));
    if (qfp4)
        hipLaunchKernelGGL((index_stream_kernel<true, true, true>), grid, dim3(kStreamThreads), 0, s, q_idx, w, k, N,
                           q_per_seq, n_visible, cand_blocks, nb, pool_scores, (float*)nullptr, pool_ids, ncols,
                           ntiles, (int32_t)wgs_per_q, (int32_t)tpw);
    else if (kfp4)
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
