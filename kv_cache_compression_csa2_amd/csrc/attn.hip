// Sparse MQA attention over the selected FP4 main-KV entries plus the layer's
// sliding-window KV (eogee.com report on DeepSeek-V4.1-Flash, 3.2: a query
// attends only to its Top-K entries and its layer's SWA KV, 64 query heads of
// dim 512 share one KV head; 3.4: the FP4 cache is dequantized before the
// attention math, so no FP4 matrix instruction is needed).
//
// Workgroup = one query (all 64 heads) x a run of 32-key tiles; 4 waves, wave w
// owns heads 16w..16w+15. Per tile:
//   1. the workgroup gathers 32 keys (288-byte records, or bf16 window rows),
//      decodes E2M1 x E4M3 to bf16 (exact) and stores the tile once in LDS,
//      key-major. The decode uses the gfx950 scaled FP4 conversion with the
//      scale's power of two, then one multiply by the scale's significand;
//   2. each wave computes S^T = K . Q^T (16x16x32 bf16 MFMA, its Q slice held
//      in registers) and runs the online softmax in the exp2 domain;
//   3. O^T += V^T . P^T: V^T comes from the same key-major tile through the LDS
//      transpose read, P^T straight from the S^T accumulator registers.
// LDS is double-buffered (one barrier per tile) and the next tile's records are
// loaded into registers while the current tile is computed.
//
// LDS row layout: physical 16-byte unit u of a key row holds logical dims
// 8*L(u) .. 8*L(u)+7 with L(u) = 4*(u % 16) + u / 16, so a lane that decodes 32
// consecutive dims writes 4 units 16 apart and 16 lanes of a row write 256
// contiguous bytes. The logits MFMA visits the 16 keys of a half-tile in the
// order perm16(i) = 2i mod 16 + i/8, which keeps the transpose reads free of
// bank conflicts with 1040-byte rows. Both are pure re-orderings of the
// contraction index: Q is loaded in the same dim order, and O is written back
// in logical order.
//
// The running max is refreshed only when it grows by more than 2^8, so the
// 128-register O^T rescale is rare; exp2 arguments stay <= 8.
// Few queries cannot fill the GPU, so a query's tiles may be split across
// workgroups that write partial (O, max, sum) to the workspace; a second
// kernel merges them.
#include <math.h>

#include "device_common.h"
#include "launch.h"

namespace csa2 {

namespace {

constexpr int kTile = 32;                 // keys per tile
constexpr int kRowB = kDim * 2 + 16;      // bytes per LDS key row (16-byte pad)
constexpr int kTileB = kTile * kRowB;     // 33,280 bytes
constexpr int kAttThreads = 256;
constexpr float kRescaleSlack = 8.0f;     // log2 units

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

CSA2_DEVINL int unit_logical(int u) { return 4 * (u & 15) + (u >> 4); }
CSA2_DEVINL int perm16(int i) { return ((2 * i) & 15) + (i >> 3); }

// Two FP4 channels (byte SEL of w) times the scale -> packed bf16 pair. The
// conversion applies only the scale's exponent (a power of two); `mant` is the
// scale divided by that power of two. Both products are exact.
template <int SEL>
CSA2_DEVINL uint32_t deq_pair(uint32_t w, float pow2, float mant) {
    const f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, pow2, SEL);
    return __builtin_amdgcn_perm(__float_as_uint(v[1] * mant), __float_as_uint(v[0] * mant), 0x07060302u);
}

CSA2_DEVINL uint4 deq_unit(uint32_t w, float pow2, float mant) {
    return make_uint4(deq_pair<0>(w, pow2, mant), deq_pair<1>(w, pow2, mant), deq_pair<2>(w, pow2, mant),
                      deq_pair<3>(w, pow2, mant));
}

template <int SEL>
CSA2_DEVINL void split_scale(uint32_t sbytes, float& pow2, float& mant) {
    const float S = __builtin_amdgcn_cvt_f32_fp8((int)sbytes, SEL);  // OCP E4M3 -> f32, exact
    const uint32_t b = __float_as_uint(S);
    pow2 = __uint_as_float(b & 0x7F800000u);
    mant = (S == 0.0f) ? S : __uint_as_float((b & 0x807FFFFFu) | 0x3F800000u);
}

CSA2_DEVINL bf16x8 as_bf16x8_2(i16x4 lo, i16x4 hi) {
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v);
}

}  // namespace

// Tiles per query: the index slots plus the largest window; the number of
// workgroups sharing a query depends only on (nq, k) so the workspace size can
// be computed before launch.
static inline int attn_total_tiles(int32_t k) { return (k + kTile - 1) / kTile + kMaxWindow / kTile; }

static inline int attn_splits(int32_t nq, int32_t k) {
    const int tiles = attn_total_tiles(k);
    // Workgroups per query: more splits fill the GPU at small batch but add
    // partial (O, max, sum) traffic and merge work. Measured on MI355X for
    // Top-512 + 128 window (20 tiles): best at 10 / 7 / 4 / 2 / 2 / 1 splits
    // for 8 / 16-32 / 64 / 128 / 256 / 512 queries.
    int want = nq >= 512 ? 1 : nq >= 128 ? 2 : nq >= 64 ? 4 : nq >= 16 ? 7 : 10;
    if (want > tiles) want = tiles;
    const int per = (tiles + want - 1) / want;
    return (tiles + per - 1) / per;
}

namespace {

struct RawRec {
    uint4 codes[2];   // 16 code bytes of each of the thread's two rows
    uint32_t sc[2];   // 2 scale bytes of each row
};

__global__ __launch_bounds__(kAttThreads, 2) void sparse_attn_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ kv, int64_t N, int32_t q_per_seq,
    const int32_t* __restrict__ idx, int32_t k, const uint16_t* __restrict__ swa, int64_t T,
    const int32_t* __restrict__ swa_start, const int32_t* __restrict__ swa_len, float scale_log2,
    uint16_t* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_o, float* __restrict__ part_ml,
    int32_t nsplit, int32_t tiles_per_split) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kTileB];
    __shared__ uint32_t key_ok[2][kTile];

    const int64_t qi = blockIdx.x / nsplit;
    const int split = blockIdx.x % nsplit;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int j = lane & 15, G = lane >> 4;
    const int head = wave * 16 + j;
    const int64_t seq = qi / q_per_seq;
    const int main_tiles = (k + kTile - 1) / kTile;
    const int slen = (swa && swa_len) ? swa_len[qi] : 0;
    const int sst = (swa && swa_start) ? swa_start[qi] : 0;
    const int total_tiles = main_tiles + kMaxWindow / kTile;
    const int t_begin = split * tiles_per_split;
    int t_end = t_begin + tiles_per_split;
    t_end = t_end < total_tiles ? t_end : total_tiles;

    f32x4 o[32];
#pragma unroll
    for (int m = 0; m < 32; m++) o[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.0f;

    const uint8_t* kv_seq = kv + seq * N * kRecord;
    const uint16_t* swa_seq = swa ? swa + seq * T * kDim : nullptr;
    const int32_t* idx_q = idx + qi * (int64_t)k;

    // gather role: rows r0 and r0 + 16 of a tile, 32-dim chunk c
    const int r0 = tid >> 4, c = tid & 15;

    auto row_ids = [&](int t, int32_t* id) {
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const int slot = t * kTile + r0 + 16 * h;
            int32_t v = slot < k ? idx_q[slot] : -1;
            id[h] = (v >= 0 && v < N) ? v : -1;
        }
    };
    auto load_raw = [&](const int32_t* id, RawRec& rw) {
#pragma unroll
        for (int h = 0; h < 2; h++) {
            if (id[h] >= 0) {
                const uint8_t* rec = kv_seq + (int64_t)id[h] * kRecord;
                rw.codes[h] = *reinterpret_cast<const uint4*>(rec + 16 * c);
                rw.sc[h] = *reinterpret_cast<const uint16_t*>(rec + kCodeBytes + 2 * c);
            } else {
                rw.codes[h] = make_uint4(0u, 0u, 0u, 0u);
                rw.sc[h] = 0u;
            }
        }
    };
    auto write_main = [&](int buf, const RawRec& rw, const int32_t* id) {
        uint8_t* base = lds + buf * kTileB;
#pragma unroll
        for (int h = 0; h < 2; h++) {
            uint8_t* row = base + (r0 + 16 * h) * kRowB + 16 * c;
            float p0, m0, p1, m1;
            split_scale<0>(rw.sc[h], p0, m0);
            split_scale<1>(rw.sc[h], p1, m1);
            *reinterpret_cast<uint4*>(row + 0 * 256) = deq_unit(rw.codes[h].x, p0, m0);
            *reinterpret_cast<uint4*>(row + 1 * 256) = deq_unit(rw.codes[h].y, p0, m0);
            *reinterpret_cast<uint4*>(row + 2 * 256) = deq_unit(rw.codes[h].z, p1, m1);
            *reinterpret_cast<uint4*>(row + 3 * 256) = deq_unit(rw.codes[h].w, p1, m1);
            if (c == 0) key_ok[buf][r0 + 16 * h] = id[h] >= 0 ? 1u : 0u;
        }
    };
    auto write_window = [&](int buf, int wbase) {
        uint8_t* base = lds + buf * kTileB;
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const int r = wbase + r0 + 16 * h;
            const bool ok = r < slen && sst + r >= 0 && sst + r < T;
            uint4 u[4];
            if (ok) {
                const uint4* src = reinterpret_cast<const uint4*>(swa_seq + (int64_t)(sst + r) * kDim) + 4 * c;
#pragma unroll
                for (int jj = 0; jj < 4; jj++) u[jj] = src[jj];
            } else {
#pragma unroll
                for (int jj = 0; jj < 4; jj++) u[jj] = make_uint4(0u, 0u, 0u, 0u);
            }
            uint8_t* row = base + (r0 + 16 * h) * kRowB + 16 * c;
#pragma unroll
            for (int jj = 0; jj < 4; jj++) *reinterpret_cast<uint4*>(row + jj * 256) = u[jj];
            if (c == 0) key_ok[buf][r0 + 16 * h] = ok ? 1u : 0u;
        }
    };

    // Records are loaded two tiles ahead of their decode: slot A holds even
    // tiles (relative to t_begin), slot B odd ones; their ids are read one tile
    // earlier still.
    int32_t id_a[2] = {-1, -1}, id_b[2] = {-1, -1}, id_n[2] = {-1, -1};
    RawRec raw_a, raw_b;
    auto prefetchable = [&](int t) { return t < t_end && t < main_tiles; };
    if (prefetchable(t_begin)) {
        row_ids(t_begin, id_a);
        load_raw(id_a, raw_a);
    }
    if (prefetchable(t_begin + 1)) {
        row_ids(t_begin + 1, id_b);
        load_raw(id_b, raw_b);
    }
    if (prefetchable(t_begin + 2)) row_ids(t_begin + 2, id_n);
    // Q after the index and record loads: memory counters retire in order, so
    // loads issued first are the ones the first decode can wait for alone.
    // Q^T operand of k-step s: head `head`, the logical dims of physical unit 4s + G.
    bf16x8 qf[16];
    {
        const uint16_t* qh = q + (qi * kHeads + head) * kDim;
#pragma unroll
        for (int s = 0; s < 16; s++)
            qf[s] = as_bf16x8(*reinterpret_cast<const uint4*>(qh + 8 * unit_logical(4 * s + G)));
    }

    const int pr_a = perm16(j), pr_t = perm16(4 * G + (j >> 2));
    auto tile = [&](int t, RawRec& rw, int32_t (&id)[2]) -> bool {
        const int buf = (t - t_begin) & 1;
        const bool is_main = t < main_tiles;
        const int wbase = (t - main_tiles) * kTile;
        if (!is_main && wbase >= slen) return false;  // no window keys left (uniform)

        // ---- 1. decode this tile into LDS; refill the slot with tile t + 2 ----
        if (is_main) {
            write_main(buf, rw, id);
            if (prefetchable(t + 2)) {
                id[0] = id_n[0];
                id[1] = id_n[1];
                load_raw(id, rw);
                if (prefetchable(t + 3)) row_ids(t + 3, id_n);
            }
        } else {
            write_window(buf, wbase);
        }
        lds_barrier();

        const uint8_t* base = lds + buf * kTileB;
        // ---- 2. logits S^T[key][head] for this wave's 16 heads ----
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
        {
            const uint8_t* ra = base + pr_a * kRowB + 16 * G;
            const uint8_t* rb = ra + 16 * kRowB;
#pragma unroll
            for (int s = 0; s < 16; s++) {
                const bf16x8 a0 = as_bf16x8(*reinterpret_cast<const uint4*>(ra + 64 * s));
                const bf16x8 a1 = as_bf16x8(*reinterpret_cast<const uint4*>(rb + 64 * s));
                s0 = mfma16x16x32(a0, qf[s], s0);
                s1 = mfma16x16x32(a1, qf[s], s1);
            }
        }
        // lane holds logical keys 4G + r of each half-tile, i.e. LDS rows perm16(4G + r)
        float x[8];
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int row = perm16(4 * G + r);
            x[r] = key_ok[buf][row] ? s0[r] * scale_log2 : -INFINITY;
            x[4 + r] = key_ok[buf][16 + row] ? s1[r] * scale_log2 : -INFINITY;
        }
        float tmax = x[0];
#pragma unroll
        for (int i = 1; i < 8; i++) tmax = fmaxf(tmax, x[i]);
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const float m_new = fmaxf(m_run, tmax);
        const bool grow = m_new > m_run + kRescaleSlack || (m_run == -INFINITY && m_new != -INFINITY);
        if (__any(grow)) {
            const float corr = (m_run == -INFINITY) ? 0.0f : exp2f(m_run - m_new);
            l_run *= corr;
#pragma unroll
            for (int m = 0; m < 32; m++) o[m] *= corr;
            m_run = m_new;
        }
        uint32_t pk[4];
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
            const float p0 = (m_run == -INFINITY) ? 0.0f : exp2f(x[i] - m_run);
            const float p1 = (m_run == -INFINITY) ? 0.0f : exp2f(x[i + 1] - m_run);
            // round to bf16 (nearest even); the denominator sums the rounded values
            const uint32_t b = pack_bf16x2(p0, p1);
            l_run += bf16_bits_to_float(b & 0xFFFFu) + bf16_bits_to_float(b >> 16);
            pk[i >> 1] = b;
        }
        const bf16x8 pf = as_bf16x8(make_uint4(pk[0], pk[1], pk[2], pk[3]));

        // ---- 3. O^T[dim][head] += V^T[dim][keys] . P^T[keys][head] ----
        {
            const uint8_t* v0 = base + pr_t * kRowB + 8 * (j & 3);
            const uint8_t* v1 = v0 + 16 * kRowB;
#pragma unroll
            for (int mt = 0; mt < 32; mt++) {
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(v0 + 32 * mt));
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(v1 + 32 * mt));
                o[mt] = mfma16x16x32(as_bf16x8_2(lo, hi), pf, o[mt]);
            }
        }
        return true;
    };
    for (int t = t_begin; t < t_end; t += 2) {
        if (!tile(t, raw_a, id_a)) break;
        if (t + 1 >= t_end || !tile(t + 1, raw_b, id_b)) break;
    }

    // ---- finish: lanes with the same head (G = 0..3) hold different keys' sums ----
    float l_tot = l_run;
    l_tot += __shfl_xor(l_tot, 16);
    l_tot += __shfl_xor(l_tot, 32);
    // lane holds O^T[physical dim 16mt + 4G + r][head]: logical dims
    // 8*L(2mt + G/2) + 4*(G%2) + r, four consecutive ones per mt
    if (nsplit == 1) {
        const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        uint16_t* orow = out + (qi * kHeads + head) * kDim + 4 * (G & 1);
#pragma unroll
        for (int mt = 0; mt < 32; mt++)
            *reinterpret_cast<uint2*>(orow + 8 * unit_logical(2 * mt + (G >> 1))) =
                make_uint2(pack_bf16x2(o[mt][0] * inv, o[mt][1] * inv), pack_bf16x2(o[mt][2] * inv, o[mt][3] * inv));
        if (lse && G == 0)
            lse[qi * kHeads + head] = l_tot > 0.0f ? (m_run + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
    } else {
        const int64_t pidx = qi * nsplit + split;
        float* po = part_o + (pidx * kHeads + head) * kDim + 4 * (G & 1);
#pragma unroll
        for (int mt = 0; mt < 32; mt++)
            *reinterpret_cast<f32x4*>(po + 8 * unit_logical(2 * mt + (G >> 1))) = o[mt];
        if (G == 0) {
            part_ml[(pidx * kHeads + head) * 2 + 0] = l_tot > 0.0f ? m_run : -INFINITY;
            part_ml[(pidx * kHeads + head) * 2 + 1] = l_tot;
        }
    }
}

// Merge of split partials: one workgroup per (query, head), 128 threads x 4 dims.
__global__ __launch_bounds__(128) void attn_merge_kernel(const float* __restrict__ part_o,
                                                         const float* __restrict__ part_ml, int32_t nsplit,
                                                         uint16_t* __restrict__ out, float* __restrict__ lse) {
    const int64_t qh = blockIdx.x;  // qi * 64 + head
    const int64_t qi = qh / kHeads, head = qh % kHeads;
    float M = -INFINITY;
    for (int s = 0; s < nsplit; s++) M = fmaxf(M, part_ml[((qi * nsplit + s) * kHeads + head) * 2]);
    float L = 0.0f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const int d = threadIdx.x * 4;
    for (int s = 0; s < nsplit; s++) {
        const int64_t pidx = (qi * nsplit + s) * kHeads + head;
        const float ms = part_ml[pidx * 2], ls = part_ml[pidx * 2 + 1];
        if (ms == -INFINITY) continue;
        const float f = exp2f(ms - M);
        L += ls * f;
        acc += *reinterpret_cast<const f32x4*>(part_o + pidx * kDim + d) * f;
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    *reinterpret_cast<uint2*>(out + qh * kDim + d) =
        make_uint2(pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv));
    if (lse && threadIdx.x == 0) lse[qh] = L > 0.0f ? (M + log2f(L)) * 0.69314718055994531f : -INFINITY;
}

}  // namespace

size_t attn_workspace_bytes(int32_t nq, int32_t k) {
    const int ns = attn_splits(nq, k);
    if (ns <= 1) return 0;
    return (size_t)nq * ns * kHeads * (kDim + 2) * sizeof(float);
}

int launch_sparse_attn(const uint16_t* q, const uint8_t* kv, int64_t N, int32_t nq, int32_t q_per_seq,
                       const int32_t* idx, int32_t k, const uint16_t* swa, int64_t T, const int32_t* swa_start,
                       const int32_t* swa_len, float softmax_scale, uint16_t* out, float* lse, void* ws,
                       hipStream_t s) {
    if (nq == 0) return 0;
    const int ns = attn_splits(nq, k);
    const int tiles = attn_total_tiles(k);
    const int per = (tiles + ns - 1) / ns;
    float* part_o = nullptr;
    float* part_ml = nullptr;
    if (ns > 1) {
        part_o = reinterpret_cast<float*>(ws);
        part_ml = part_o + (size_t)nq * ns * kHeads * kDim;
    }
    const float scale_log2 = softmax_scale * 1.4426950408889634f;
    hipLaunchKernelGGL(sparse_attn_kernel, dim3((unsigned)((int64_t)nq * ns)), dim3(kAttThreads), 0, s, q, kv, N,
                       q_per_seq, idx, k, swa, T, swa_start, swa_len, scale_log2, out, lse, part_o, part_ml, ns, per);
    if (ns > 1)
        hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)((int64_t)nq * kHeads)), dim3(128), 0, s, part_o,
                           part_ml, ns, out, lse);
    return 0;
}

}  // namespace csa2
