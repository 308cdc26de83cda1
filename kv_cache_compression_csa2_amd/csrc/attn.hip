// Sparse MQA attention over the selected FP4 main-KV entries plus the layer's
// sliding-window KV (eogee.com report on DeepSeek-V4.1-Flash, 3.2: a query
// attends only to its Top-K entries and its layer's SWA KV, 64 query heads of
// dim 512 share one KV head; 3.4: the FP4 cache is dequantized before the
// attention math, so no FP4 matrix instruction is needed).
//
// Workgroup = one query (all 64 heads) x a run of 32-key tiles; 4 waves, wave w
// owns heads 16w..16w+15. Per tile:
//   1. the workgroup gathers 32 keys (288-byte records, or bf16 window rows),
//      decodes E2M1 x E4M3 -> bf16 (exact) and stores the tile in LDS twice:
//      K-major [key][dim] for the logits and dim-major [dim][key] for P.V;
//   2. each wave computes S^T = K . Q^T (16x16x32 bf16 MFMA, its Q slice held
//      in registers), applies the online softmax in the exp2 domain, and
//   3. accumulates O^T += V^T . P^T, with P^T taken straight from the S^T
//      accumulator registers (the keys of the contraction are visited in the
//      order those registers hold them).
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

constexpr int kTile = 32;            // keys per tile
constexpr int kKRow = kDim + 8;      // bf16 per K-major LDS row (16-byte pad)
constexpr int kVRow = kTile + 4;     // bf16 per dim-major LDS row (8-byte pad)
constexpr int kAttThreads = 256;
constexpr float kRescaleSlack = 8.0f;  // log2 units

}  // namespace

// Tiles per query: the index slots plus the largest window; the number of
// workgroups sharing a query depends only on (nq, k) so the workspace size can
// be computed before launch.
static inline int attn_total_tiles(int32_t k) { return (k + kTile - 1) / kTile + kMaxWindow / kTile; }

static inline int attn_splits(int32_t nq, int32_t k) {
    const int tiles = attn_total_tiles(k);
    int want = (512 + nq - 1) / (nq > 0 ? nq : 1);
    if (want < 1) want = 1;
    if (want > tiles) want = tiles;
    const int per = (tiles + want - 1) / want;
    return (tiles + per - 1) / per;
}

namespace {

__global__ __launch_bounds__(kAttThreads, 2) void sparse_attn_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ kv, int64_t N, int32_t q_per_seq,
    const int32_t* __restrict__ idx, int32_t k, const uint16_t* __restrict__ swa, int64_t T,
    const int32_t* __restrict__ swa_start, const int32_t* __restrict__ swa_len, float scale_log2,
    uint16_t* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_o, float* __restrict__ part_ml,
    int32_t nsplit, int32_t tiles_per_split) {
    __shared__ __attribute__((aligned(16))) uint16_t Ks[kTile * kKRow];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[kDim * kVRow];
    __shared__ uint32_t key_ok[kTile];

    const int64_t qi = blockIdx.x / nsplit;
    const int split = blockIdx.x % nsplit;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hl = lane & 15, g = lane >> 4;
    const int head = wave * 16 + hl;
    const int64_t seq = qi / q_per_seq;
    const int main_tiles = (k + kTile - 1) / kTile;
    const int slen = (swa && swa_len) ? swa_len[qi] : 0;
    const int sst = (swa && swa_start) ? swa_start[qi] : 0;
    const int total_tiles = main_tiles + kMaxWindow / kTile;
    const int t_begin = split * tiles_per_split;
    int t_end = t_begin + tiles_per_split;
    t_end = t_end < total_tiles ? t_end : total_tiles;

    // Q^T operand (B of the logits MFMA): head `head`, dims 32s + 8g .. +8.
    bf16x8 qf[16];
    {
        const uint4* src = reinterpret_cast<const uint4*>(q + (qi * kHeads + head) * kDim) + g;
#pragma unroll
        for (int s = 0; s < 16; s++) qf[s] = as_bf16x8(src[4 * s]);
    }

    f32x4 o[32];
#pragma unroll
    for (int m = 0; m < 32; m++) o[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.0f;

    const uint8_t* kv_seq = kv + seq * N * kRecord;
    const uint16_t* swa_seq = swa ? swa + seq * T * kDim : nullptr;
    const int32_t* idx_q = idx + qi * (int64_t)k;

    for (int t = t_begin; t < t_end; t++) {
        const bool is_main = t < main_tiles;
        const int wbase = (t - main_tiles) * kTile;  // first window row of a window tile
        if (!is_main && wbase >= slen) break;        // no window keys left (uniform)

        // ---- 1. gather + decode the tile into LDS ----
#pragma unroll
        for (int it = 0; it < 2; it++) {
            const int item = tid + it * kAttThreads;  // 0..511
            const int kq4 = item >> 6;                // key quad 0..7
            const int oct = item & 63;                // dims 8*oct .. +8
            uint32_t vals[4][4];                      // [key in quad][bf16 pair]
#pragma unroll
            for (int kk = 0; kk < 4; kk++) {
                const int key = kq4 * 4 + kk;
                bool ok;
                if (is_main) {
                    const int slot = t * kTile + key;
                    const int32_t id = slot < k ? idx_q[slot] : -1;
                    ok = id >= 0 && id < N;
                    if (ok) {
                        const uint8_t* rec = kv_seq + (int64_t)id * kRecord;
                        const uint32_t codes = *reinterpret_cast<const uint32_t*>(rec + oct * 4);
                        const float hs = 0.5f * e4m3_to_float(rec[kCodeBytes + (oct >> 1)]);
                        dequant8(codes, hs, vals[kk]);
                    }
                } else {
                    const int r = wbase + key;
                    ok = r < slen && sst + r >= 0 && sst + r < T;
                    if (ok) {
                        const uint4 v = *reinterpret_cast<const uint4*>(swa_seq + (int64_t)(sst + r) * kDim + oct * 8);
                        vals[kk][0] = v.x;
                        vals[kk][1] = v.y;
                        vals[kk][2] = v.z;
                        vals[kk][3] = v.w;
                    }
                }
                if (!ok) vals[kk][0] = vals[kk][1] = vals[kk][2] = vals[kk][3] = 0u;
                if (oct == 0) key_ok[key] = ok ? 1u : 0u;
                *reinterpret_cast<uint4*>(&Ks[key * kKRow + oct * 8]) =
                    make_uint4(vals[kk][0], vals[kk][1], vals[kk][2], vals[kk][3]);
            }
            // dim-major: dim 8*oct + d, keys 4*kq4 .. +4
#pragma unroll
            for (int d = 0; d < 8; d++) {
                const int pr = d >> 1, hi = d & 1;
                uint32_t e[4];
#pragma unroll
                for (int kk = 0; kk < 4; kk++) e[kk] = hi ? (vals[kk][pr] >> 16) : (vals[kk][pr] & 0xFFFFu);
                *reinterpret_cast<uint2*>(&Vt[(oct * 8 + d) * kVRow + kq4 * 4]) =
                    make_uint2(e[0] | (e[1] << 16), e[2] | (e[3] << 16));
            }
        }
        __syncthreads();

        // ---- 2. logits S^T[key][head] for this wave's 16 heads ----
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
        {
            const uint16_t* r0 = &Ks[hl * kKRow + g * 8];
            const uint16_t* r1 = &Ks[(16 + hl) * kKRow + g * 8];
#pragma unroll
            for (int s = 0; s < 16; s++) {
                const bf16x8 a0 = as_bf16x8(*reinterpret_cast<const uint4*>(r0 + 32 * s));
                const bf16x8 a1 = as_bf16x8(*reinterpret_cast<const uint4*>(r1 + 32 * s));
                s0 = mfma16x16x32(a0, qf[s], s0);
                s1 = mfma16x16x32(a1, qf[s], s1);
            }
        }
        // lane holds keys 4g+r (s0) and 16+4g+r (s1), r = 0..3, of head `head`
        float x[8];
#pragma unroll
        for (int r = 0; r < 4; r++) {
            x[r] = key_ok[4 * g + r] ? s0[r] * scale_log2 : -INFINITY;
            x[4 + r] = key_ok[16 + 4 * g + r] ? s1[r] * scale_log2 : -INFINITY;
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
            const uint32_t u0 = __float_as_uint(p0), u1 = __float_as_uint(p1);
            const uint32_t b0 = (u0 + 0x7FFFu + ((u0 >> 16) & 1u)) >> 16;
            const uint32_t b1 = (u1 + 0x7FFFu + ((u1 >> 16) & 1u)) >> 16;
            l_run += bf16_bits_to_float(b0) + bf16_bits_to_float(b1);
            pk[i >> 1] = b0 | (b1 << 16);
        }
        const bf16x8 pf = as_bf16x8(make_uint4(pk[0], pk[1], pk[2], pk[3]));

        // ---- 3. O^T[dim][head] += V^T[dim][keys] . P^T[keys][head] ----
        {
            const uint16_t* vrow = &Vt[hl * kVRow + 4 * g];
#pragma unroll
            for (int m = 0; m < 32; m++) {
                const uint2 lo = *reinterpret_cast<const uint2*>(vrow + (16 * m) * kVRow);
                const uint2 hi = *reinterpret_cast<const uint2*>(vrow + (16 * m) * kVRow + 16);
                const bf16x8 av = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
                o[m] = mfma16x16x32(av, pf, o[m]);
            }
        }
        __syncthreads();
    }

    // ---- finish: lanes with the same head (g = 0..3) hold different keys' sums ----
    float l_tot = l_run;
    l_tot += __shfl_xor(l_tot, 16);
    l_tot += __shfl_xor(l_tot, 32);
    // lane holds O^T[dim 16m + 4g + r][head]
    if (nsplit == 1) {
        const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        uint16_t* orow = out + (qi * kHeads + head) * kDim + 4 * g;
#pragma unroll
        for (int m = 0; m < 32; m++) {
            uint32_t b[4];
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const uint32_t u = __float_as_uint(o[m][r] * inv);
                b[r] = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
            }
            *reinterpret_cast<uint2*>(orow + 16 * m) = make_uint2(b[0] | (b[1] << 16), b[2] | (b[3] << 16));
        }
        if (lse && g == 0)
            lse[qi * kHeads + head] = l_tot > 0.0f ? (m_run + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
    } else {
        const int64_t pidx = qi * nsplit + split;
        float* po = part_o + (pidx * kHeads + head) * kDim + 4 * g;
#pragma unroll
        for (int m = 0; m < 32; m++) *reinterpret_cast<f32x4*>(po + 16 * m) = o[m];
        if (g == 0) {
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
    uint32_t b[4];
#pragma unroll
    for (int r = 0; r < 4; r++) {
        const uint32_t u = __float_as_uint(acc[r] * inv);
        b[r] = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    }
    *reinterpret_cast<uint2*>(out + qh * kDim + d) = make_uint2(b[0] | (b[1] << 16), b[2] | (b[3] << 16));
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
