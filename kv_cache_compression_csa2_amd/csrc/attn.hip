// Sparse MQA attention over the selected FP4 main-KV entries plus the layer's
// sliding-window KV (eogee.com report on DeepSeek-V4.1-Flash, 3.2: a query
// attends only to its Top-K entries and its layer's SWA KV, 64 query heads of
// dim 512 share one KV head; 3.4: the FP4 cache is dequantized before the
// attention math, so no FP4 matrix instruction is needed).
//
// Workgroup = one query (all 64 heads) x a run of 32-key tiles; 4 waves, wave w
// owns heads 16w..16w+15. Per tile:
//   1. the workgroup gathers 32 keys (288-byte records, or bf16 window rows),
//      decodes E2M1 x E4M3 to fp16 (exact: a product of a 2-bit and a 4-bit
//      significand, between 2^-10 and 2688 in magnitude) and stores the tile
//      once in LDS, key-major. The decode is the gfx950 scaled FP4->fp16
//      conversion with the scale's power of two, then one packed fp16 multiply
//      by the scale's significand; window rows are converted bf16 -> fp16;
//   2. each wave computes S^T = K . Q^T (16x16x32 fp16 MFMA, its Q slice held
//      in registers, converted from bf16) and runs the online softmax in the
//      exp2 domain;
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
// fp16 holds every bf16 value of magnitude 2^-14 .. 65504 exactly (smaller
// ones to within 2^-25). Each head's Q is scaled by a power of two that puts
// its largest magnitude in [2^14, 2^15) before the conversion, and the head's
// logit scale carries the inverse, so any finite bf16 Q converts exactly
// (elements below 2^-28 of the head's largest lose bits). Window rows must
// stay below 65504 in magnitude (a status bit reports rows that do not). P is
// rounded to fp16 (its values are <= 2^8) and the softmax denominator sums
// the rounded values.
//
// The running max is refreshed only when it grows by more than 2^8, so the
// 128-register O^T rescale is rare; exp2 arguments stay <= 8. It starts at a
// finite floor (-2^126), so masked keys (logit -inf) need no special case.
// Few queries cannot fill the GPU, so a query's tiles may be split across
// workgroups that write partial results (O / sum in fp16, max, sum) to the
// workspace; a second kernel merges them. O / sum is a convex combination of
// value rows, all below 65504 in magnitude, so fp16 holds it with 8 times the
// resolution of bf16 in the same bytes.
#include <math.h>

#include "device_common.h"
#include "launch.h"

namespace csa2 {

namespace {

constexpr int kTile = 32;                 // keys per tile
constexpr int kRowB = kDim * 2 + 16;      // bytes per LDS key row (16-byte pad)
constexpr int kTileB = kTile * kRowB;     // 33,280 bytes
constexpr int kStgRow = kDim * 2 + 16;    // output staging row: 512 bf16 + pad
static_assert(4 * 16 * kStgRow <= 2 * kTileB, "output staging must fit the tile buffers");
constexpr int kAttThreads = 256;
constexpr float kRescaleSlack = 8.0f;     // log2 units

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kMaxFloor = -8.507059e37f;  // -2^126: running-max floor

CSA2_DEVINL int unit_logical(int u) { return 4 * (u & 15) + (u >> 4); }
CSA2_DEVINL int perm16(int i) { return ((2 * i) & 15) + (i >> 3); }
// i with perm16(i) == r
CSA2_DEVINL int perm16_inv(int r) { return (r >> 1) + 8 * (r & 1); }

// 16x16x32 fp16 MFMA, same operand layout as the bf16 one.
CSA2_DEVINL f32x4 mfma16x16x32h(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Two FP4 channels (byte SEL of w) times the scale -> packed fp16 pair. The
// conversion applies only the scale's exponent (a power of two); `mant` holds
// the scale divided by that power of two twice. Both products are exact.
template <int SEL>
CSA2_DEVINL uint32_t deq_pair(uint32_t w, float pow2, f16x2 mant) {
    const f16x2 v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, pow2, SEL);
    return __builtin_bit_cast(uint32_t, v * mant);
}

CSA2_DEVINL uint4 deq_unit(uint32_t w, float pow2, f16x2 mant) {
    return make_uint4(deq_pair<0>(w, pow2, mant), deq_pair<1>(w, pow2, mant), deq_pair<2>(w, pow2, mant),
                      deq_pair<3>(w, pow2, mant));
}

template <int SEL>
CSA2_DEVINL void split_scale(uint32_t sbytes, float& pow2, f16x2& mant) {
    const float S = __builtin_amdgcn_cvt_f32_fp8((int)sbytes, SEL);  // OCP E4M3 -> f32, exact
    const uint32_t b = __float_as_uint(S);
    pow2 = __uint_as_float(b & 0x7F800000u);
    const _Float16 m = (_Float16)((S == 0.0f) ? S : __uint_as_float((b & 0x807FFFFFu) | 0x3F800000u));
    mant = f16x2{m, m};
}

// Two bf16 (one dword) -> two fp16 (one dword), round to nearest even.
CSA2_DEVINL uint32_t bf16x2_to_f16x2(uint32_t v) {
    const f32x2 f = {__uint_as_float(v << 16), __uint_as_float(v & 0xFFFF0000u)};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
}
CSA2_DEVINL uint4 bf16x8_to_f16x8(uint4 v) {
    return make_uint4(bf16x2_to_f16x2(v.x), bf16x2_to_f16x2(v.y), bf16x2_to_f16x2(v.z), bf16x2_to_f16x2(v.w));
}
CSA2_DEVINL f16x8 as_f16x8(uint4 v) { return __builtin_bit_cast(f16x8, v); }

// Eight bf16 times the power of two `up` -> fp16 (round to nearest even).
CSA2_DEVINL uint32_t bf16x2_to_f16x2_scaled(uint32_t v, float up) {
    const f32x2 f = {__uint_as_float(v << 16) * up, __uint_as_float(v & 0xFFFF0000u) * up};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
}
CSA2_DEVINL uint4 bf16x8_to_f16x8_scaled(uint4 v, float up) {
    return make_uint4(bf16x2_to_f16x2_scaled(v.x, up), bf16x2_to_f16x2_scaled(v.y, up),
                      bf16x2_to_f16x2_scaled(v.z, up), bf16x2_to_f16x2_scaled(v.w, up));
}
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
// Running maximum of bf16 magnitude bits (|x| orders like them), two lanes of
// 16 bits at a time (packed u16 max).
CSA2_DEVINL u16x2 bf16x8_max_mag2(uint4 v, u16x2 m) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; i++) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[i] & 0x7FFF7FFFu));
    return m;
}
// Largest magnitude of eight bf16 as magnitude bits.
CSA2_DEVINL uint32_t bf16x8_max_mag(uint4 v) {
    const u16x2 m = bf16x8_max_mag2(v, u16x2{0, 0});
    return max((uint32_t)m[0], (uint32_t)m[1]);
}

// Two floats -> packed fp16 pair (lo in bits 0..15), round to nearest even.
CSA2_DEVINL uint32_t pack_f16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, f16x2));
}
CSA2_DEVINL float f16_bits_to_float(uint32_t b) { return (float)__builtin_bit_cast(_Float16, (uint16_t)b); }

CSA2_DEVINL f16x8 as_f16x8_2(i16x4 lo, i16x4 hi) {
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(f16x8, v);
}

// Max / sum over the four lanes l, l^16, l^32, l^48 (one head's four key
// groups) with the gfx950 row and half-wave swaps, no LDS round trip.
CSA2_DEVINL float max_over_groups(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
CSA2_DEVINL uint32_t max_over_groups_u(uint32_t v) {
    const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = max(a[0], a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return max(b[0], b[1]);
}
CSA2_DEVINL float sum_over_groups(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

}  // namespace

// Tiles per query: the index slots plus the largest window; the number of
// workgroups sharing a query depends only on (nq, k) so the workspace size can
// be computed before launch.
static inline int attn_total_tiles(int32_t k) { return (k + kTile - 1) / kTile + kMaxWindow / kTile; }

constexpr int kMaxSplits = 16;  // partials per query the merge kernel holds

static inline int attn_splits(int32_t nq, int32_t k) {
    const int tiles = attn_total_tiles(k);
    // Workgroups per query: more splits fill the GPU at small batch but add
    // partial (O, max, sum) traffic and merge work. Measured on MI355X for
    // Top-512 + 128 window (20 tiles): best at 10 / 7 / 4 / 2 / 2 / 1 splits
    // for 8 / 16-32 / 64 / 128 / 256 / 512 queries.
    int want = nq >= 512 ? 1 : nq >= 128 ? 2 : nq >= 64 ? 4 : nq >= 16 ? 7 : 10;
    if (want > tiles) want = tiles;
    if (want > kMaxSplits) want = kMaxSplits;
    const int per = (tiles + want - 1) / want;
    return (tiles + per - 1) / per;
}

namespace {

struct RawRec {
    uint4 codes[2];   // 16 code bytes of each of the thread's two rows
    uint32_t sc[2];   // 2 scale bytes of each row
    int32_t id[2];    // the rows' entry ids (-1: empty slot)
};

// Tiles of split `s` of `nsplit`: main tiles [M*s/nsplit, M*(s+1)/nsplit) and
// window tiles [W*s/nsplit, W*(s+1)/nsplit), so window tiles (whose rows are
// loaded without prefetch) spread over the splits.
CSA2_DEVINL int part_lo(int n, int s, int nsplit) { return (int)(((int64_t)n * s) / nsplit); }

constexpr int kSwaRec = kDim + kDim / 32;  // FP8 window row: 512 E4M3 codes + 16 E8M0 scales

// Window rows are bf16 [T][512] or, with kFp8Win, FP8 rows [T][528] (E4M3
// elements, one E8M0 scale per 32 channels; each gather thread's 32 channels
// are exactly one scale block). E4M3 times a power of two is exact in fp16
// while the block maximum lies in [2^-7, 2^16).
template <bool kFp8Win>
__global__ __launch_bounds__(kAttThreads, 2) void sparse_attn_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ kv, int64_t N, int32_t q_per_seq,
    const int32_t* __restrict__ idx, int32_t k, const void* __restrict__ swa, int64_t T,
    const int32_t* __restrict__ swa_start, const int32_t* __restrict__ swa_len, float scale_log2,
    uint16_t* __restrict__ out, float* __restrict__ lse, uint16_t* __restrict__ part_o, float* __restrict__ part_ml,
    int32_t nsplit, uint32_t* __restrict__ status) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kTileB];
    // 0 or -inf per key, stored at perm16_inv(row) (+16 for the second half)
    // so that a lane's four keys of a half-tile are one 16-byte read
    __shared__ __attribute__((aligned(16))) float key_bias[2][kTile];
    // status bits seen by the workgroup (written only when an input is out of domain)
    __shared__ uint32_t bad_sh;
    // entry ids of this workgroup's main tiles, range-checked (-1: empty)
    extern __shared__ int32_t sid[];

    const int64_t qi = blockIdx.x / nsplit;
    const int split = blockIdx.x % nsplit;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int j = lane & 15, G = lane >> 4;
    const int head = wave * 16 + j;
    const int64_t seq = qi / q_per_seq;
    const int M = N > 0 ? (k + kTile - 1) / kTile : 0;
    constexpr int W = kMaxWindow / kTile;
    const int slen = (swa && swa_len) ? swa_len[qi] : 0;
    const int sst = (swa && swa_start) ? swa_start[qi] : 0;
    const int m0 = part_lo(M, split, nsplit), nmain = part_lo(M, split + 1, nsplit) - m0;
    const int w0 = part_lo(W, split, nsplit), w1 = part_lo(W, split + 1, nsplit);
    // window tiles past the query's window length hold no keys
    const int wlive = (slen + kTile - 1) / kTile;
    const int nwin = (w1 < wlive ? w1 : wlive) > w0 ? (w1 < wlive ? w1 : wlive) - w0 : 0;
    const int ntiles = nmain + nwin;

    f32x4 o[32];
#pragma unroll
    for (int m = 0; m < 32; m++) o[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = kMaxFloor, l_run = 0.0f;

    const uint8_t* kv_seq = kv + seq * N * kRecord;
    const uint16_t* swa_seq = (swa && !kFp8Win) ? static_cast<const uint16_t*>(swa) + seq * T * kDim : nullptr;
    const uint8_t* swa8_seq = (swa && kFp8Win) ? static_cast<const uint8_t*>(swa) + seq * T * kSwaRec : nullptr;
    const int32_t* idx_q = idx + qi * (int64_t)k + (int64_t)m0 * kTile;

    // the workgroup's entry ids, checked once (ids outside [-1, N) are
    // skipped and reported); the status bits gather in bad_sh, cleared here
    // with no dependence on any load and set only after the barrier below
    if (tid == 0) bad_sh = 0u;
    uint32_t bad = 0;
    for (int i = tid; i < nmain * kTile; i += kAttThreads) {
        const int32_t v = (m0 * kTile + i < k) ? idx_q[i] : -1;
        sid[i] = (v >= 0 && v < N) ? v : -1;
        bad |= (v < -1 || v >= N) ? kStatusIdx : 0u;
    }
    if (split == 0 && tid == 0 && swa) {
        bad |= (slen < 0 || slen > kMaxWindow) ? kStatusWinLen : 0u;
        bad |= (slen > 0 && (sst < 0 || (int64_t)sst + slen > T)) ? kStatusWinRange : 0u;
    }
    lds_barrier();
    if (bad) atomicOr(&bad_sh, bad);

    // gather role: rows r0 and r0 + 16 of a tile, 32-dim chunk c
    const int r0 = tid >> 4, c = tid & 15;

    // Branch-free loads (an empty slot reads entry 0 and is zeroed at decode),
    // so nothing between the loads and their use makes the wave wait for them.
    auto load_raw = [&](int lt, RawRec& rw) {
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const int32_t id = sid[lt * kTile + r0 + 16 * h];
            const uint8_t* rec = kv_seq + (int64_t)(id > 0 ? id : 0) * kRecord;
            rw.codes[h] = *reinterpret_cast<const uint4*>(rec + 16 * c);
            rw.sc[h] = *reinterpret_cast<const uint16_t*>(rec + kCodeBytes + 2 * c);
            rw.id[h] = id;
        }
    };
    auto write_main = [&](int buf, const RawRec& rw) {
        uint8_t* base = lds + buf * kTileB;
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const bool ok = rw.id[h] >= 0;
            const uint4 cd = ok ? rw.codes[h] : make_uint4(0u, 0u, 0u, 0u);
            uint8_t* row = base + (r0 + 16 * h) * kRowB + 16 * c;
            float p0, p1;
            f16x2 m0h, m1h;
            split_scale<0>(rw.sc[h], p0, m0h);
            split_scale<1>(rw.sc[h], p1, m1h);
            *reinterpret_cast<uint4*>(row + 0 * 256) = deq_unit(cd.x, p0, m0h);
            *reinterpret_cast<uint4*>(row + 1 * 256) = deq_unit(cd.y, p0, m0h);
            *reinterpret_cast<uint4*>(row + 2 * 256) = deq_unit(cd.z, p1, m1h);
            *reinterpret_cast<uint4*>(row + 3 * 256) = deq_unit(cd.w, p1, m1h);
            if (c == 0) key_bias[buf][perm16_inv(r0) + 16 * h] = ok ? 0.0f : -INFINITY;
        }
    };
    auto write_window = [&](int buf, int wbase) {
        uint8_t* base = lds + buf * kTileB;
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const int r = wbase + r0 + 16 * h;
            const bool ok = r < slen && sst + r >= 0 && sst + r < T;
            uint4 u[4];
            if (ok && kFp8Win) {
                const uint8_t* rec = swa8_seq + (int64_t)(sst + r) * kSwaRec;
                const uint4 c0 = reinterpret_cast<const uint4*>(rec + 32 * c)[0];
                const uint4 c1 = reinterpret_cast<const uint4*>(rec + 32 * c)[1];
                // 448 * 2^(b-127) < 65504 only for scale bytes up to 134; past
                // that the conversion's result is out of fp16's range (a plain
                // store: every writer stores the same bit)
                if (rec[kDim + c] > 134) bad_sh = kStatusNonFinite;
                // the E8M0 byte as the exponent field of a binary32: the
                // conversion applies that power of two
                const float X = __uint_as_float((uint32_t)rec[kDim + c] << 23);
                const uint32_t cw[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
                uint32_t h[16];
#pragma unroll
                for (int i = 0; i < 8; i++) {
                    h[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(cw[i], X, false));
                    h[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(cw[i], X, true));
                }
#pragma unroll
                for (int jj = 0; jj < 4; jj++) u[jj] = make_uint4(h[4 * jj], h[4 * jj + 1], h[4 * jj + 2], h[4 * jj + 3]);
            } else if (ok) {
                const uint4* src = reinterpret_cast<const uint4*>(swa_seq + (int64_t)(sst + r) * kDim) + 4 * c;
#pragma unroll
                for (int jj = 0; jj < 4; jj++) u[jj] = bf16x8_to_f16x8(src[jj]);
            } else {
#pragma unroll
                for (int jj = 0; jj < 4; jj++) u[jj] = make_uint4(0u, 0u, 0u, 0u);
            }
            uint8_t* row = base + (r0 + 16 * h) * kRowB + 16 * c;
#pragma unroll
            for (int jj = 0; jj < 4; jj++) *reinterpret_cast<uint4*>(row + jj * 256) = u[jj];
            if (c == 0) key_bias[buf][perm16_inv(r0) + 16 * h] = ok ? 0.0f : -INFINITY;
        }
    };

    // Records are loaded one tile ahead of their decode: they arrive while the
    // current tile is computed.
    RawRec raw;
    if (nmain > 0) load_raw(0, raw);
    // Q after the record loads: memory counters retire in order, so loads
    // issued first are the ones the first decode can wait for alone.
    // Q^T operand of k-step s: head `head`, the logical dims of physical unit 4s + G.
    f16x8 qf[16];
    float sl2;  // this head's logit scale (log2 units), times 2^-sh
    {
        const uint16_t* qh = q + (qi * kHeads + head) * kDim;
        uint4 qr[16];
        uint32_t amax = 0;  // largest |q| of the head as bf16 magnitude bits
#pragma unroll
        for (int s = 0; s < 16; s++) {
            qr[s] = *reinterpret_cast<const uint4*>(qh + 8 * unit_logical(4 * s + G));
            amax = max(amax, bf16x8_max_mag(qr[s]));
        }
        amax = (uint32_t)max_over_groups_u(amax);
        // 2^sh puts the head's largest magnitude in [2^14, 2^15): exponent
        // field e -> floor(log2 amax) = e - 127 (bf16 subnormals and zero heads
        // take the clamp)
        const int sh = min(max(14 - ((int)(amax >> 7) - 127), -126), 126);
        const float up = __uint_as_float((uint32_t)(127 + sh) << 23);
#pragma unroll
        for (int s = 0; s < 16; s++) qf[s] = as_f16x8(bf16x8_to_f16x8_scaled(qr[s], up));
        sl2 = scale_log2 * __uint_as_float((uint32_t)(127 - sh) << 23);
    }

    const int pr_a = perm16(j), pr_t = perm16(4 * G + (j >> 2));
    for (int lt = 0; lt < ntiles; lt++) {
        const int buf = lt & 1;
        // ---- 1. decode this tile into LDS; load the next main tile's records ----
        if (lt < nmain) {
            write_main(buf, raw);
            if (lt + 1 < nmain) load_raw(lt + 1, raw);
        } else {
            write_window(buf, (w0 + lt - nmain) * kTile);
        }
        lds_barrier();

        const uint8_t* base = lds + buf * kTileB;
        // ---- 2. logits S^T[key][head] for this wave's 16 heads ----
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
        const f32x4 bias0 = *reinterpret_cast<const f32x4*>(&key_bias[buf][4 * G]);
        const f32x4 bias1 = *reinterpret_cast<const f32x4*>(&key_bias[buf][16 + 4 * G]);
        {
            const uint8_t* ra = base + pr_a * kRowB + 16 * G;
            const uint8_t* rb = ra + 16 * kRowB;
#pragma unroll
            for (int s = 0; s < 16; s++) {
                const f16x8 a0 = as_f16x8(*reinterpret_cast<const uint4*>(ra + 64 * s));
                const f16x8 a1 = as_f16x8(*reinterpret_cast<const uint4*>(rb + 64 * s));
                s0 = mfma16x16x32h(a0, qf[s], s0);
                s1 = mfma16x16x32h(a1, qf[s], s1);
            }
        }
        // lane holds logical keys 4G + r of each half-tile, i.e. LDS rows perm16(4G + r)
        float x[8];
#pragma unroll
        for (int r = 0; r < 4; r++) {
            x[r] = fmaf(s0[r], sl2, bias0[r]);
            x[4 + r] = fmaf(s1[r], sl2, bias1[r]);
        }
        float tmax = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
        tmax = max_over_groups(tmax);
        const float m_new = fmaxf(m_run, tmax);
        if (__any(m_new > m_run + kRescaleSlack)) {
            const float corr = __builtin_amdgcn_exp2f(m_run - m_new);
            l_run *= corr;
#pragma unroll
            for (int m = 0; m < 32; m++) o[m] *= corr;
            m_run = m_new;
        }
        uint32_t pk[4];
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
            const f32x2 p = {__builtin_amdgcn_exp2f(x[i] - m_run), __builtin_amdgcn_exp2f(x[i + 1] - m_run)};
            // round to fp16 (nearest even); the denominator sums the rounded values
            const f16x2 h = __builtin_convertvector(p, f16x2);
            l_run += (float)h[0] + (float)h[1];
            pk[i >> 1] = __builtin_bit_cast(uint32_t, h);
        }
        const f16x8 pf = as_f16x8(make_uint4(pk[0], pk[1], pk[2], pk[3]));

        // ---- 3. O^T[dim][head] += V^T[dim][keys] . P^T[keys][head] ----
        {
            const uint8_t* v0 = base + pr_t * kRowB + 8 * (j & 3);
            const uint8_t* v1 = v0 + 16 * kRowB;
#pragma unroll
            for (int mt = 0; mt < 32; mt++) {
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(v0 + 32 * mt));
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(v1 + 32 * mt));
                o[mt] = mfma16x16x32h(as_f16x8_2(lo, hi), pf, o[mt]);
            }
        }
    }

    // ---- finish: lanes with the same head (G = 0..3) hold different keys' sums ----
    const float l_tot = sum_over_groups(l_run);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    // O / l is the output in bf16 (one split) or the split's partial in fp16,
    // which the merge weights by l * 2^(m - max m). The wave's 16 heads x 512 dims
    // go through LDS as rows (1040-byte stride: conflict-free writes) and are
    // stored with 16-byte lanes along each 1 KiB row; straight from the
    // accumulators every store would scatter 16-byte pieces over 16 rows.
    // Lane (head j, group G) holds O^T[physical dim 16mt + 4G + r][head j],
    // logical dims 8*L(2mt + G/2) + 4*(G%2) + r: four consecutive ones per mt.
    lds_barrier();  // every wave is done with the tile buffers
    uint8_t* stg = lds + wave * (16 * kStgRow);
    // Out-of-domain inputs (a window value fp16 cannot hold, a NaN scale,
    // another non-finite input) always leave non-finite values in the output:
    // the packed words' exponent fields are checked once here instead of
    // every input value in the tile loop.
    uint32_t emax = 0;
    {
        uint8_t* row = stg + j * kStgRow + 8 * (G & 1);
        if (nsplit > 1) {
            u16x2 mm = {0, 0};
#pragma unroll
            for (int mt = 0; mt < 32; mt++) {
                const uint2 w2 =
                    make_uint2(pack_f16x2(o[mt][0] * inv, o[mt][1] * inv), pack_f16x2(o[mt][2] * inv, o[mt][3] * inv));
                *reinterpret_cast<uint2*>(row + 16 * unit_logical(2 * mt + (G >> 1))) = w2;
                mm = __builtin_elementwise_max(mm, __builtin_bit_cast(u16x2, w2.x & 0x7C007C00u));
                mm = __builtin_elementwise_max(mm, __builtin_bit_cast(u16x2, w2.y & 0x7C007C00u));
            }
            emax = max(mm[0], mm[1]) == 0x7C00 ? 1u : 0u;
        } else {
            u16x2 mm = {0, 0};
#pragma unroll
            for (int mt = 0; mt < 32; mt++) {
                const uint2 w2 = make_uint2(pack_bf16x2(o[mt][0] * inv, o[mt][1] * inv),
                                            pack_bf16x2(o[mt][2] * inv, o[mt][3] * inv));
                *reinterpret_cast<uint2*>(row + 16 * unit_logical(2 * mt + (G >> 1))) = w2;
                mm = __builtin_elementwise_max(mm, __builtin_bit_cast(u16x2, w2.x & 0x7F807F80u));
                mm = __builtin_elementwise_max(mm, __builtin_bit_cast(u16x2, w2.y & 0x7F807F80u));
            }
            emax = max(mm[0], mm[1]) == 0x7F80 ? 1u : 0u;
        }
        emax |= (l_tot == l_tot && l_tot != INFINITY) ? 0u : 1u;
    }
    if (__any(emax) && lane == 0) atomicOr(&bad_sh, kStatusNonFinite);
    lds_barrier();
    if (tid == 0 && status && bad_sh) atomicOr(status, bad_sh);
    const int64_t prow = nsplit == 1 ? qi * kHeads : (qi * nsplit + split) * kHeads;  // row of head 0
    uint16_t* dst = (nsplit == 1 ? out : part_o) + (prow + wave * 16) * kDim + 8 * lane;
    // Split partials go out with non-temporal stores: written once and read by
    // the merge, they would otherwise sit in L2 as dirty lines, whose later
    // write-back measurably slowed the kernel after the step's attention. The
    // unsplit (large-batch) output keeps ordinary stores, which measured faster.
    if (nsplit > 1) {
#pragma unroll
        for (int i = 0; i < 16; i++)
            __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(stg + i * kStgRow + 16 * lane),
                                        reinterpret_cast<u32x4*>(dst + (int64_t)i * kDim));
    } else {
#pragma unroll
        for (int i = 0; i < 16; i++)
            *reinterpret_cast<uint4*>(dst + (int64_t)i * kDim) = *reinterpret_cast<const uint4*>(stg + i * kStgRow + 16 * lane);
    }
    if (G == 0) {
        // the head index from the hardware lane id: recomputed here rather
        // than kept live (in a register or a spill slot) through the tile loop
        const int head_e = wave * 16 + (int)(__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) & 15);
        if (nsplit == 1) {
            if (lse) lse[qi * kHeads + head_e] = l_tot > 0.0f ? (m_run + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
        } else {
            part_ml[(prow + head_e) * 2 + 0] = l_tot > 0.0f ? m_run : -INFINITY;
            part_ml[(prow + head_e) * 2 + 1] = l_tot;
        }
    }
}

// Merge of split partials: one workgroup per (query, head), 128 threads x 4
// dims. Every split's (max, sum) pair and O slice are loaded up front, so the
// merge waits for memory once.

__global__ __launch_bounds__(128) void attn_merge_kernel(const uint16_t* __restrict__ part_o,
                                                         const float* __restrict__ part_ml, int32_t nsplit,
                                                         uint16_t* __restrict__ out, float* __restrict__ lse) {
    const int64_t qh = blockIdx.x;  // qi * 64 + head
    const int64_t qi = qh / kHeads, head = qh % kHeads;
    const int d = threadIdx.x * 4;
    f32x2 ml[kMaxSplits];
    uint2 po[kMaxSplits];
#pragma unroll
    for (int s = 0; s < kMaxSplits; s++) {
        if (s < nsplit) {
            const int64_t pidx = (qi * nsplit + s) * kHeads + head;
            ml[s] = *reinterpret_cast<const f32x2*>(part_ml + pidx * 2);
            po[s] = *reinterpret_cast<const uint2*>(part_o + pidx * kDim + d);
        }
    }
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < kMaxSplits; s++)
        if (s < nsplit) M = fmaxf(M, ml[s][0]);
    float L = 0.0f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kMaxSplits; s++) {
        if (s < nsplit && ml[s][0] != -INFINITY) {
            const float f = ml[s][1] * exp2f(ml[s][0] - M);  // the partial is O / l
            L += f;
            acc += f32x4{f16_bits_to_float(po[s].x & 0xFFFFu), f16_bits_to_float(po[s].x >> 16),
                         f16_bits_to_float(po[s].y & 0xFFFFu), f16_bits_to_float(po[s].y >> 16)} * f;
        }
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    uint32_t* o32 = reinterpret_cast<uint32_t*>(out + qh * kDim + d);  // non-temporal, as the split partials
    __builtin_nontemporal_store(pack_bf16x2(acc[0] * inv, acc[1] * inv), o32);
    __builtin_nontemporal_store(pack_bf16x2(acc[2] * inv, acc[3] * inv), o32 + 1);
    if (lse && threadIdx.x == 0) lse[qh] = L > 0.0f ? (M + log2f(L)) * 0.69314718055994531f : -INFINITY;
}

}  // namespace

// Workspace: the status word (kStatusBytes, so the partials stay aligned),
// then the split partials when a query's tiles are split.
size_t attn_workspace_bytes(int32_t nq, int32_t k) {
    const int ns = attn_splits(nq, k);
    if (ns <= 1) return kStatusBytes;
    return kStatusBytes + (size_t)nq * ns * kHeads * (kDim * sizeof(uint16_t) + 2 * sizeof(float));
}

int launch_sparse_attn(const uint16_t* q, const uint8_t* kv, int64_t N, int32_t nq, int32_t q_per_seq,
                       const int32_t* idx, int32_t k, const void* swa, bool swa_fp8, int64_t T, const int32_t* swa_start,
                       const int32_t* swa_len, float softmax_scale, uint16_t* out, float* lse, void* ws,
                       hipStream_t s) {
    if (nq == 0) return 0;
    const int ns = attn_splits(nq, k);
    // dynamic LDS: the largest share of main-tile entry ids a split holds
    const int mt = N > 0 ? (k + kTile - 1) / kTile : 0;
    const size_t sid_bytes = (size_t)((mt + ns - 1) / ns) * kTile * sizeof(int32_t);
    uint16_t* part_o = nullptr;
    float* part_ml = nullptr;
    uint32_t* status = reinterpret_cast<uint32_t*>(ws);
    if (ns > 1) {
        part_o = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(ws) + kStatusBytes);
        part_ml = reinterpret_cast<float*>(part_o + (size_t)nq * ns * kHeads * kDim);
    }
    const float scale_log2 = softmax_scale * 1.4426950408889634f;
    const dim3 grid((unsigned)((int64_t)nq * ns));
    if (swa_fp8)
        hipLaunchKernelGGL(sparse_attn_kernel<true>, grid, dim3(kAttThreads), sid_bytes, s, q, kv, N, q_per_seq, idx,
                           k, swa, T, swa_start, swa_len, scale_log2, out, lse, part_o, part_ml, ns, status);
    else
        hipLaunchKernelGGL(sparse_attn_kernel<false>, grid, dim3(kAttThreads), sid_bytes, s, q, kv, N, q_per_seq, idx,
                           k, swa, T, swa_start, swa_len, scale_log2, out, lse, part_o, part_ml, ns, status);
    if (ns > 1)
        hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)((int64_t)nq * kHeads)), dim3(128), 0, s, part_o,
                           part_ml, ns, out, lse);
    return 0;
}

}  // namespace csa2
