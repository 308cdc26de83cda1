// Exact per-segment Top-K selection over keys held in registers, shared by
// the Top-K kernels and the fused indexer + Top-K kernel. Order of merit:
// larger key first, equal keys by lower position (the callers hand keys over
// in position order).
#pragma once

#include "device_common.h"

namespace csa2 {
namespace tk {

// Order-preserving key of a score: larger key = larger score, -0 folded onto
// +0, -inf and NaN to key 0 (never chosen).
CSA2_DEVINL uint32_t score_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (f != f || u == 0xFF800000u) return 0u;
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kRegMaxKpt = 32;        // keys per thread
constexpr int kRegMaxKeys = 1024 * kRegMaxKpt;  // 32768 per chunk
constexpr int kRegMaxCand = 16384;    // merge capacity per row

// Histograms of the three radix digits (key bits 31..20, 19..10, 9..0), all
// cleared once at the start.
template <int NT>
struct RegTk {
    uint32_t h1[4096];
    uint32_t h2[1024];
    uint32_t h3[1024];
    uint32_t wsum[NT / 64];
    uint32_t sel_bin, sel_above, total;
};

// Inclusive prefix sum over the 64 lanes with DPP: row_shr 1, 2, 4, 8 within
// each 16-lane row, then row_bcast15 / row_bcast31 carry row totals forward.
CSA2_DEVINL uint32_t wave_incl_scan(uint32_t x) {
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);
    return x;
}

// Exclusive scan over the block in thread order (one barrier); *total = sum.
// wsum must not be rewritten until every thread has returned (the callers
// place a barrier in between).
template <int NT>
CSA2_DEVINL uint32_t reg_block_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t x = wave_incl_scan(v);
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; i++) {
        const uint32_t sw = wsum[i];
        before += (i < wave) ? sw : 0u;
        tot += sw;
    }
    *total = tot;
    return before + x - v;
}

// From histogram h of nbins bins, finds the bin holding the rem-th largest
// counted key, counting from the top bin: sets sh.sel_bin and sh.sel_above
// (keys in higher bins). rem == 0 means rem = min(k, all counted keys), which
// is also stored in sh.total. Two barriers; the results are readable after.
template <int NT>
CSA2_DEVINL void reg_pick_bin(const uint32_t* h, RegTk<NT>& sh, int nbins, uint32_t rem, uint32_t k) {
    constexpr int kMaxPer = 4096 / NT;
    const int tid = threadIdx.x;
    const int per = nbins / NT;
    uint32_t c[kMaxPer], loc = 0;
#pragma unroll
    for (int j = 0; j < kMaxPer; j++) {
        c[j] = (j < per) ? h[nbins - 1 - (tid * per + j)] : 0u;
        loc += c[j];
    }
    uint32_t tot;
    uint32_t above = reg_block_scan<NT>(loc, sh.wsum, &tot);
    if (rem == 0) {
        rem = tot < k ? tot : k;
        if (tid == 0) sh.total = rem;
    }
    if (above < rem && rem <= above + loc) {
        for (int j = 0; j < per; j++) {
            if (above + c[j] >= rem) {
                sh.sel_bin = nbins - 1 - (tid * per + j);
                sh.sel_above = above;
                break;
            }
            above += c[j];
        }
    }
    __syncthreads();
}

// Exact selection over the keys held in registers (thread t holds positions
// t*KPT .. t*KPT+KPT-1 of the segment; key 0 = never selected): a 3-pass MSB
// radix select (12, 10, 10 bits) over LDS histograms finds the k-th largest
// key T, then emit(slot, u) is called for every key > T and for the first
// `need` keys == T, slots ascending with position (one packed block scan of
// the per-thread counts). Returns the number selected, min(k, #nonzero keys).
//
// kNarrow (used for merged candidates, whose values sit in a narrow band at
// the top of the row): the first digit ends at the highest bit where the
// largest and smallest key differ -- every key shares the bits above it -- so
// the first histogram spreads instead of piling into a few bins. The three
// digits then cover bits [0, s1 + 12); s1 <= 20 always.
template <int NT, int KPT, bool kNarrow, class Emit>
CSA2_DEVINL uint32_t reg_select_emit(const uint32_t (&key)[KPT], uint32_t k, RegTk<NT>& sh, Emit emit) {
    const int tid = threadIdx.x;
    for (int i = tid; i < 4096; i += NT) sh.h1[i] = 0;
    for (int i = tid; i < 1024; i += NT) sh.h2[i] = 0;
    int s1 = 20;        // digit 1 = key bits [s1, s1 + 12)
    uint32_t high = 0;  // bits >= s1 + 12, shared by every nonzero key
    if (kNarrow) {
        uint32_t mx = 0u, mn = 0xFFFFFFFFu;
#pragma unroll
        for (int u = 0; u < KPT; u++) {
            mx = max(mx, key[u]);
            if (key[u]) mn = min(mn, key[u]);
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
            mn = min(mn, (uint32_t)__shfl_xor((int)mn, o));
        }
        if ((tid & 63) == 0) {
            sh.h3[tid >> 6] = mx;
            sh.h3[512 + (tid >> 6)] = mn;
        }
        __syncthreads();
        uint32_t bmax = 0u, bmin = 0xFFFFFFFFu;
#pragma unroll
        for (int i = 0; i < NT / 64; i++) {
            bmax = max(bmax, sh.h3[i]);
            bmin = min(bmin, sh.h3[512 + i]);
        }
        if (bmax != 0u) {
            const int h = bmax > bmin ? 31 - __builtin_clz(bmax ^ bmin) : 0;  // highest differing bit
            s1 = h >= 31 ? 20 : (h >= 11 ? h - 11 : 0);
            high = (s1 + 12 < 32) ? (bmax & ~((1u << (s1 + 12)) - 1u)) : 0u;
        }
        __syncthreads();  // every thread has read h3 before it is cleared
    }
    for (int i = tid; i < 1024; i += NT) sh.h3[i] = 0;
    const int s2 = s1 >= 10 ? s1 - 10 : 0;  // digit 2 = bits [s2, s1)
    const int s3 = s2 >= 10 ? s2 - 10 : 0;  // digit 3 = bits [s3, s2); s3 == 0
    const uint32_t m2 = (1u << (s1 - s2)) - 1u, m3 = (1u << (s2 - s3)) - 1u;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < KPT; u++)
        if (key[u]) atomicAdd(&sh.h1[(key[u] >> s1) & 4095u], 1u);
    __syncthreads();
    reg_pick_bin<NT>(sh.h1, sh, 4096, 0u, k);
    const uint32_t kk = sh.total;
    if (kk == 0) return 0;
    uint32_t prefix = sh.sel_bin, rem = kk - sh.sel_above;  // T's bits [s1, s1 + 12)
#pragma unroll
    for (int u = 0; u < KPT; u++)
        if (key[u] && ((key[u] >> s1) & 4095u) == prefix) atomicAdd(&sh.h2[(key[u] >> s2) & m2], 1u);
    __syncthreads();
    reg_pick_bin<NT>(sh.h2, sh, 1024, rem, k);
    prefix = (prefix << (s1 - s2)) | sh.sel_bin;  // bits [s2, s1 + 12)
    rem -= sh.sel_above;
    const uint32_t m12 = (1u << (12 + s1 - s2)) - 1u;
#pragma unroll
    for (int u = 0; u < KPT; u++)
        if (key[u] && ((key[u] >> s2) & m12) == prefix) atomicAdd(&sh.h3[(key[u] >> s3) & m3], 1u);
    __syncthreads();
    reg_pick_bin<NT>(sh.h3, sh, 1024, rem, k);
    const uint32_t T = high | (((prefix << (s2 - s3)) | sh.sel_bin) << s3);
    const uint32_t need = rem - sh.sel_above;

    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int u = 0; u < KPT; u++) {
        gt += key[u] > T;
        eq += key[u] == T;
    }
    uint32_t tot;
    const uint32_t before = reg_block_scan<NT>((gt << 16) | eq, sh.wsum, &tot);
    const uint32_t gt_before = before >> 16, eq_before = before & 0xFFFFu;
    uint32_t slot = gt_before + (eq_before < need ? eq_before : need);
    uint32_t eq_run = eq_before;
#pragma unroll
    for (int u = 0; u < KPT; u++) {
        const bool is_eq = key[u] == T;
        const bool sel = key[u] > T || (is_eq && eq_run < need);
        eq_run += is_eq;
        if (sel && slot < kk) emit(slot, u);  // slot < kk always holds; the check keeps stores in bounds regardless
        slot += sel;
    }
    return kk;
}

}  // namespace tk
}  // namespace csa2
