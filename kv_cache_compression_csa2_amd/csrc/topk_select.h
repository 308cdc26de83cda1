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

// The score whose key is k (the inverse of score_key on keys >= 1); key 0
// (no score) maps to -inf, which no score exceeds.
CSA2_DEVINL float key_score(uint32_t k) {
    if (k == 0u) return -__builtin_inff();
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

constexpr int kRegMaxKpt = 32;        // keys per thread
constexpr int kRegMaxKeys = 1024 * kRegMaxKpt;  // 32768 per chunk
constexpr int kRegMaxCand = 16384;    // merge capacity per row
constexpr int kLst = 512;             // keys of the first digit's chosen bin finished by one wave
constexpr int kStage = 2048;          // largest selection staged in LDS for coalesced output

constexpr int kBins1 = 4096;          // first-digit bins (one more holds key 0)

// Histograms of the three radix digits (key bits 31..20, 19..10, 9..0 when
// the keys span the whole range; h2 and h3 only when the first digit leaves
// more than kLst keys in the k-th key's bin), the gathered keys of that bin,
// and per-wave scan / min / max words. h1 doubles as the output staging area
// once the threshold is known.
template <int NT>
struct alignas(16) RegTk {
    uint32_t h1[kBins1 + 4];
    uint32_t h2[1024];
    uint32_t h3[1024];
    uint32_t lst[kLst];
    uint32_t wsum[NT / 64];
    uint32_t wmax[NT / 64], wmin[NT / 64];
    uint32_t lst_n;
    uint32_t bc[4];  // results of one wave's pick, read by the others
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

// Max / min over the 64 lanes, in every lane: the same DPP row shifts and row
// broadcasts as the scan, then lane 63's value. A lane whose source is out of
// range keeps its own value.
CSA2_DEVINL uint32_t wave_max_u32(uint32_t x) {
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x111, 0xF, 0xF, false));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x112, 0xF, 0xF, false));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x114, 0xF, 0xF, false));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x118, 0xF, 0xF, false));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x142, 0xA, 0xF, false));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x143, 0xC, 0xF, false));
    return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}
CSA2_DEVINL uint32_t wave_min_u32(uint32_t x) {
    x = min(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x111, 0xF, 0xF, false));
    x = min(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x112, 0xF, 0xF, false));
    x = min(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x114, 0xF, 0xF, false));
    x = min(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x118, 0xF, 0xF, false));
    x = min(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x142, 0xA, 0xF, false));
    x = min(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x143, 0xC, 0xF, false));
    return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// Exclusive scan over the block in thread order (one barrier); *total = sum.
// wsum must not be rewritten until every thread has returned (the callers
// place a barrier in between).
template <int NT>
CSA2_DEVINL uint32_t reg_block_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t x = wave_incl_scan(v);
    if (lane == 63) wsum[wave] = x;
    lds_barrier();
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

// Bin of histogram h (NBINS bins, counted from the top bin down) holding the
// rem-th counted key and the count of keys in the bins above it; rem == 0
// stands for min(cap, all counted keys). Returns that rank (0: no keys, bin
// and above unset); 1 <= rem <= all counted keys otherwise. Every wave
// computes it on its own, so no barrier is needed: lane l sums the P =
// NBINS/64 bins of ranks [P*l, P*l + P) (reads rotated across lanes to spread
// LDS banks), a wave scan finds the lane whose range holds the rank, and a
// second scan over that lane's P bins the bin.
template <int NBINS>
CSA2_DEVINL uint32_t wave_pick(const uint32_t* h, uint32_t rem, uint32_t cap, uint32_t& bin, uint32_t& above) {
    constexpr int P = NBINS / 64;
    const int lane = threadIdx.x & 63;
    const uint32_t* blk = h + NBINS - P * (lane + 1);
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < P / 4; j++) {
        const int jj = (j + lane) & (P / 4 - 1);
        const uint4 v = *reinterpret_cast<const uint4*>(blk + 4 * jj);
        c += v.x + v.y + v.z + v.w;
    }
    const uint32_t incl = wave_incl_scan(c);
    if (rem == 0) {
        const uint32_t all = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
        rem = all < cap ? all : cap;
        if (rem == 0) return 0;
    }
    const uint64_t hit = __ballot(incl - c < rem && rem <= incl);
    const int L = (int)__builtin_ctzll(hit);
    const uint32_t base = (uint32_t)__builtin_amdgcn_readlane((int)(incl - c), L);
    const uint32_t ci = lane < P ? h[NBINS - 1 - (P * L + lane)] : 0u;
    const uint32_t incl2 = wave_incl_scan(ci) + base;
    const uint64_t hit2 = __ballot(lane < P && incl2 - ci < rem && rem <= incl2);
    const int I = (int)__builtin_ctzll(hit2);
    bin = (uint32_t)(NBINS - 1 - (P * L + I));
    above = (uint32_t)__builtin_amdgcn_readlane((int)(incl2 - ci), I);
    return rem;
}

// Bits [0, s1) of the rem-th largest of the n keys in lst (n <= kLst, all
// nonzero, all equal in the bits above s1). On return rem is that key's rank
// among the keys equal to it and n_eq their number. Up to 64 keys: one key
// per lane, each lane counts the keys above and at its own (a broadcast loop,
// no serial dependence between steps). More: MSB first with wave ballots.
CSA2_DEVINL uint32_t wave_bit_select(const uint32_t* lst, int n, int s1, uint32_t& rem, uint32_t& n_eq) {
    const int lane = threadIdx.x & 63;
    if (n <= 64) {
        const uint32_t mine = lane < n ? lst[lane] : 0u;
        uint32_t gt = 0, ge = 0;
        for (int j = 0; j < n; j++) {
            const uint32_t kj = (uint32_t)__builtin_amdgcn_readlane((int)mine, j);
            gt += kj > mine;
            ge += kj >= mine;
        }
        // lanes holding the rem-th largest key (all equal; take the first)
        const uint64_t hit = __ballot(lane < n && gt < rem && rem <= ge);
        const int L = (int)__builtin_ctzll(hit);
        const uint32_t T = (uint32_t)__builtin_amdgcn_readlane((int)mine, L);
        rem -= (uint32_t)__builtin_amdgcn_readlane((int)gt, L);
        n_eq = (uint32_t)__builtin_amdgcn_readlane((int)(ge - gt), L);
        return T & ((1u << s1) - 1u);
    }
    const int nv = (n + 63) >> 6;  // occupied lane rows (uniform)
    uint32_t v[kLst / 64];
#pragma unroll
    for (int i = 0; i < kLst / 64; i++) v[i] = (i < nv && lane + 64 * i < n) ? lst[lane + 64 * i] : 0u;
    const uint32_t low = (1u << s1) - 1u;  // s1 <= 20
    uint32_t prefix = 0;
    for (int b = s1 - 1; b >= 0; b--) {
        const uint32_t mask = low & ~((1u << b) - 1u);  // bits [b, s1)
        const uint32_t want = prefix | (1u << b);
        uint32_t cnt = 0;
#pragma unroll
        for (int i = 0; i < kLst / 64; i++)
            if (i < nv) cnt += (uint32_t)__popcll(__ballot(v[i] != 0u && (v[i] & mask) == want));
        if (cnt >= rem)
            prefix = want;
        else
            rem -= cnt;
    }
    uint32_t e = 0;
#pragma unroll
    for (int i = 0; i < kLst / 64; i++)
        if (i < nv) e += (uint32_t)__popcll(__ballot(v[i] != 0u && (v[i] & low) == prefix));
    n_eq = e;
    return prefix;
}

// Exact selection over the keys held in registers (thread t holds positions
// t*KPT .. t*KPT+KPT-1 of the segment; key 0 = never selected). An MSB radix
// select finds the k-th largest key T: a 12-bit first digit over an LDS
// histogram, then -- when T's bin holds at most kLst keys, the usual case --
// those keys are gathered and one wave resolves T among them (every wave, in
// workgroups of at most four waves, so no barrier is needed): a rank count
// with one key per lane up to 64 keys, else the remaining bits MSB-first with
// ballots; a crowded bin takes two more 10-bit histogram digits. The bin and
// the threshold are found the same way. Every key > T and the
// first `need` keys == T are selected, slots ascending with position (one
// packed block scan of the per-thread counts; when every key equal to T is
// taken, a key is selected iff it is >= T). out(slot, key, val(u)) is called
// for every slot < the returned count, min(k, #nonzero keys): by consecutive
// threads from an LDS copy when the selection has at most kStage keys, else
// by the key's owner thread.
// The per-key passes are branch-free except where a wave holds a selected or
// gathered key.
//
// kNarrow (for keys in a narrow band, e.g. one row's scores or merged
// candidates): the first digit ends at the highest bit where the largest and
// smallest key differ -- every key shares the bits above it -- so the first
// histogram spreads instead of piling into a few bins. Digits then cover bits
// [0, s1 + 12); s1 <= 20 always.
template <int NT, int KPT, bool kNarrow, class Val, class Out>
CSA2_DEVINL uint32_t reg_select_emit(const uint32_t (&key)[KPT], uint32_t k, RegTk<NT>& sh, Val val, Out out) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    constexpr bool kRedundant = NT <= 256;
    for (int i = tid; i < (kBins1 + 4) / 4; i += NT) reinterpret_cast<uint4*>(sh.h1)[i] = make_uint4(0u, 0u, 0u, 0u);
    if (tid == 0) sh.lst_n = 0;
    if (kNarrow) {
        uint32_t mx = 0u, mn = 0xFFFFFFFFu;
#pragma unroll
        for (int u = 0; u < KPT; u++) {
            mx = max(mx, key[u]);
            mn = min(mn, key[u] ? key[u] : 0xFFFFFFFFu);
        }
        mx = wave_max_u32(mx);
        mn = wave_min_u32(mn);
        if (lane == 0) {
            sh.wmax[wave] = mx;
            sh.wmin[wave] = mn;
        }
    }
    lds_barrier();
    int s1 = 20;        // digit 1 = key bits [s1, s1 + 12)
    uint32_t high = 0;  // bits >= s1 + 12, shared by every nonzero key
    if (kNarrow) {
        uint32_t bmax = 0u, bmin = 0xFFFFFFFFu;
#pragma unroll
        for (int i = 0; i < NT / 64; i++) {
            bmax = max(bmax, sh.wmax[i]);
            bmin = min(bmin, sh.wmin[i]);
        }
        if (bmax != 0u) {
            const int h = bmax > bmin ? 31 - __builtin_clz(bmax ^ bmin) : 0;  // highest differing bit
            s1 = h >= 31 ? 20 : (h >= 11 ? h - 11 : 0);
            high = (s1 + 12 < 32) ? (bmax & ~((1u << (s1 + 12)) - 1u)) : 0u;
        }
    }
    // key 0 counts in the spare bin kBins1, outside the histogram proper
#pragma unroll
    for (int u = 0; u < KPT; u++) atomicAdd(&sh.h1[key[u] ? ((key[u] >> s1) & 4095u) : (uint32_t)kBins1], 1u);
    lds_barrier();
    // kk = min(k, nonzero keys) and T's first digit: with at most four waves
    // every wave finds them itself; else wave 0 does and the others wait at
    // one barrier
    uint32_t kk, b1, above;
    if (kRedundant) {
        b1 = above = 0;
        kk = wave_pick<kBins1>(sh.h1, 0u, k, b1, above);
    } else {
        if (wave == 0) {
            uint32_t bb = 0, ab = 0;
            const uint32_t kk0 = wave_pick<kBins1>(sh.h1, 0u, k, bb, ab);
            if (lane == 0) {
                sh.bc[0] = kk0;
                sh.bc[1] = bb;
                sh.bc[2] = ab;
            }
        }
        lds_barrier();
        kk = sh.bc[0];
        b1 = sh.bc[1];
        above = sh.bc[2];
    }
    if (kk == 0) return 0;
    uint32_t rem = kk - above;  // rank of T within bin b1
    const uint32_t nb1 = sh.h1[b1];
    uint32_t T;
    bool all_eq = false;  // every key equal to T is selected
    if (nb1 <= (uint32_t)kLst) {
        // keys of bin b1: every nonzero key shares the bits above the digit
        const uint32_t lo = high | (b1 << s1), width = 1u << s1;
#pragma unroll
        for (int u = 0; u < KPT; u++) {
            const bool m = key[u] != 0u && key[u] - lo < width;
            const uint64_t bal = __ballot(m);
            if (bal) {
                uint32_t base = 0;
                if (lane == 0) base = __hip_atomic_fetch_add(&sh.lst_n, (uint32_t)__popcll(bal), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                base = (uint32_t)__builtin_amdgcn_readfirstlane((int)base);
                const uint32_t r = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
                if (m) sh.lst[base + r] = key[u];
            }
        }
        lds_barrier();
        if (kRedundant) {
            uint32_t n_eq = 0;
            const uint32_t low = wave_bit_select(sh.lst, (int)nb1, s1, rem, n_eq);
            T = high | (b1 << s1) | low;
            all_eq = rem == n_eq;
        } else {
            if (wave == 0) {
                uint32_t r = rem, n_eq = 0;
                const uint32_t low = wave_bit_select(sh.lst, (int)nb1, s1, r, n_eq);
                if (lane == 0) {
                    sh.bc[0] = low;
                    sh.bc[1] = r;
                    sh.bc[3] = n_eq;
                }
            }
            lds_barrier();
            T = high | (b1 << s1) | sh.bc[0];
            rem = sh.bc[1];
            all_eq = rem == sh.bc[3];
        }
    } else {
        for (int i = tid; i < 1024; i += NT) {
            sh.h2[i] = 0;
            sh.h3[i] = 0;
        }
        lds_barrier();
        const int s2 = s1 >= 10 ? s1 - 10 : 0;  // digit 2 = bits [s2, s1)
        const int s3 = s2 >= 10 ? s2 - 10 : 0;  // digit 3 = bits [s3, s2); s3 == 0
        const uint32_t m2 = (1u << (s1 - s2)) - 1u, m3 = (1u << (s2 - s3)) - 1u;
        uint32_t prefix = b1;  // T's bits [s1, s1 + 12)
#pragma unroll
        for (int u = 0; u < KPT; u++)
            if (key[u] && key[u] - (high | (prefix << s1)) < (1u << s1)) atomicAdd(&sh.h2[(key[u] >> s2) & m2], 1u);
        lds_barrier();
        uint32_t b2 = 0;
        wave_pick<1024>(sh.h2, rem, 0u, b2, above);
        rem -= above;
        prefix = (prefix << (s1 - s2)) | b2;  // bits [s2, s1 + 12)
#pragma unroll
        for (int u = 0; u < KPT; u++)
            if (key[u] && key[u] - (high | (prefix << s2)) < (1u << s2)) atomicAdd(&sh.h3[(key[u] >> s3) & m3], 1u);
        lds_barrier();
        uint32_t b3 = 0;
        wave_pick<1024>(sh.h3, rem, 0u, b3, above);
        rem -= above;
        T = high | (((prefix << (s2 - s3)) | b3) << s3);
    }
    const uint32_t need = rem;
    // per-thread start slot (and, when some keys equal to T are left out, the
    // count of keys == T before this thread)
    uint32_t slot0, eq0 = 0;
    uint32_t tot;
    if (all_eq) {
        uint32_t ge = 0;
#pragma unroll
        for (int u = 0; u < KPT; u++) ge += key[u] >= T;
        // its barrier also ends every read of h1 above, which the staging overwrites
        slot0 = reg_block_scan<NT>(ge, sh.wsum, &tot);
    } else {
        uint32_t gt = 0, eq = 0;
#pragma unroll
        for (int u = 0; u < KPT; u++) {
            gt += key[u] > T;
            eq += key[u] == T;
        }
        const uint32_t before = reg_block_scan<NT>((gt << 16) | eq, sh.wsum, &tot);
        eq0 = before & 0xFFFFu;
        slot0 = (before >> 16) + (eq0 < need ? eq0 : need);
    }
    // Up to kStage selected keys go through LDS (keys in h1[0, kStage),
    // payloads in h1[kStage, 2 kStage)) and are written out by consecutive
    // threads; larger selections are written by their owner threads.
    auto pass = [&](auto&& take) {
        uint32_t slot = slot0;
        if (all_eq) {
#pragma unroll
            for (int u = 0; u < KPT; u++) {
                const bool sel = key[u] >= T;
                if (sel) take(slot, u);
                slot += sel;
            }
        } else {
            uint32_t eq_run = eq0;
#pragma unroll
            for (int u = 0; u < KPT; u++) {
                const bool is_eq = key[u] == T;
                const bool sel = key[u] > T || (is_eq && eq_run < need);
                eq_run += is_eq;
                if (sel) take(slot, u);
                slot += sel;
            }
        }
    };
    if (kk <= (uint32_t)kStage) {
        pass([&](uint32_t slot, int u) {
            if (slot < (uint32_t)kStage) {  // always; keeps the stores in bounds regardless
                sh.h1[slot] = key[u];
                sh.h1[kStage + slot] = (uint32_t)val(u);
            }
        });
        lds_barrier();
        for (uint32_t s2 = tid; s2 < kk; s2 += NT) out(s2, sh.h1[s2], (int32_t)sh.h1[kStage + s2]);
    } else {
        pass([&](uint32_t slot, int u) {
            if (slot < kk) out(slot, key[u], (int32_t)val(u));
        });
    }
    return kk;
}

// One wave keeps the k best of n > k keys held in LDS at key[0, n) (payloads
// id[0, n)), positions in arrival order: larger key first, equal keys by lower
// position. The kept ones move to the front, key[0, kept) / id[0, kept), in
// position order. Lane l holds positions [P*l, P*l + P) (contiguous runs, so
// lane order is position order); every load is done before the first store,
// so the compaction can run in place. The threshold t is built bit by bit from
// the top (the largest t with at least k keys >= t, counted with one ballot per
// key slot), starting below the highest bit where the largest and smallest
// keys differ. Exact (slack 0, or when the search runs to the last bit): keys
// above the k-th largest are kept, then equal ones in position order until k
// are; that key is returned. With slack > 0 the search stops as soon as at
// most k + slack keys are >= t: all of them are kept (k <= kept <= k + slack)
// and t is returned -- a lower bound of the k-th largest key that need not be
// a key itself (0 when it would map to no finite score). Every dropped key
// then has at least k larger ones, so no key of the top k is lost. Must be
// called by all 64 lanes of the wave (wave-uniform n, k and slack); key 0
// marks no key and never appears among valid positions.
template <int C, typename Id>
CSA2_DEVINL uint32_t wave_keep_topk(uint32_t* key, Id* id, uint32_t n, uint32_t k, uint32_t slack, uint32_t& kept) {
    constexpr int P = C / 64;
    static_assert(P * 64 == C, "buffer size must be a multiple of 64");
    const uint32_t lane = threadIdx.x & 63;
    uint32_t kv[P];
    Id iv[P];
    uint32_t lmax = 0u, lmin = 0xFFFFFFFFu;
#pragma unroll
    for (int j = 0; j < P; j++) {
        const uint32_t p = lane * P + j;
        kv[j] = p < n ? key[p] : 0u;
        iv[j] = id[p];
        lmax = max(lmax, kv[j]);
        lmin = p < n ? min(lmin, kv[j]) : lmin;
    }
    const uint32_t hi = wave_max_u32(lmax), lo = wave_min_u32(lmin);
    uint32_t t = hi;
    uint32_t cnt_t = n;  // keys >= t (every valid key shares t's bits so far)
    if (hi != lo) {
        const int top = 31 - __builtin_clz(hi ^ lo);
        t = top == 31 ? 0u : hi & ~((2u << top) - 1u);  // the bits every key shares
        for (int b = top; b >= 0 && cnt_t > k + slack; b--) {
            const uint32_t c = t | (1u << b);
            uint32_t cnt = 0;
#pragma unroll
            for (int j = 0; j < P; j++) cnt += (uint32_t)__builtin_popcountll(__ballot(kv[j] >= c));
            if (cnt >= k) {
                t = c;
                cnt_t = cnt;
            }
        }
    }
    // keep every key >= t when they are few enough, else the exact k
    const bool all_ge = cnt_t <= k + slack;
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int j = 0; j < P; j++) {
        const bool v = lane * P + j < n;
        gt += (uint32_t)(v && kv[j] > t);
        eq += (uint32_t)(v && kv[j] == t);
    }
    const uint32_t igt = wave_incl_scan(gt), ieq = wave_incl_scan(eq);
    const uint32_t ngt = (uint32_t)__builtin_amdgcn_readlane((int)igt, 63);
    const uint32_t need = all_ge ? (uint32_t)__builtin_amdgcn_readlane((int)ieq, 63) : k - ngt;  // equal keys to keep
    const uint32_t nkeep = ngt + need;
    uint32_t e = ieq - eq;  // equal keys at lower positions
    // A stable partition of [0, n): kept keys to [0, nkeep) and the others to
    // [nkeep, n), both in position order, so every store is unconditional (no
    // divergent branch per key); positions past n are rewritten in place.
    uint32_t o = (igt - gt) + min(e, need);                 // kept keys at lower positions
    uint32_t d = nkeep + min(lane * P, n) - o;              // discarded keys at lower positions, offset by nkeep
#pragma unroll
    for (int j = 0; j < P; j++) {
        const uint32_t p = lane * P + j;
        const bool iseq = p < n && kv[j] == t;
        const bool keep = p < n && (kv[j] > t || (iseq && e < need));
        e += (uint32_t)iseq;
        const uint32_t dst = p >= n ? p : (keep ? o : d);
        o += (uint32_t)keep;
        d += (uint32_t)(!keep && p < n);
        key[dst] = kv[j];
        id[dst] = iv[j];
    }
    kept = nkeep;
    // valid keys are at least key(-FLT_MAX) = 2^23: a smaller t admits every score
    return t < 0x00800000u ? 0u : t;
}

}  // namespace tk
}  // namespace csa2
