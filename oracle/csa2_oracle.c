/*
 * CSA2 hot-path oracle: a plain, slow CPU statement of what the path computes.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library calls, links or
 * includes this file; only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark load it. It shares no code, header or table with the HIP
 * kernels: every value below is derived again here from the format and method
 * definitions.
 *
 * Sources (web pages on DeepSeek-V4.1-Flash):
 *   [EOG]  eogee.com, "DeepSeek V4.1-Flash 技术报告深度解析：CED 架构与 KV Cache
 *          极限压缩" -- 3.2 (CSA2 modes, indexer, Top-K + SWA attention, head
 *          geometry), 3.3 (hierarchical sparse indexer, block max, 2048 x 8
 *          pool), 3.4 (FP4 main KV: E2M1 values, one E4M3 scale per 16
 *          channels, dequantize before attention).
 *   [TIT]  titansim.online blog on DeepSeek-V4.1-Flash, "核心机制与研究方法",
 *          CSA2 paragraph (Full / Reindex / Reuse; Top-512).
 *   [NXB]  m.nxbn.cn repository walkthrough, 2.3 (E2M1 + E4M3 per 16 channels)
 *          and 3.3 (index_n_heads 32, index_head_dim 128, index_topk 512,
 *          candidate_topk_blocks 2048, candidate_block_size 8).
 *   [OCP]  OCP Microscaling Formats (MX) v1.0, the "OCP standard" [EOG] 3.4
 *          names: E2M1 and E4M3 element encodings, E8M0 shared scales and
 *          the rule that picks a block's shared scale.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   indexer score = sum_h w_h * max(q_h . k, 0); block score = max of its 8
 *   positions; key == value; softmax scale 1/sqrt(512); ties -> lower index;
 *   scale = E4M3(amax / 6) rounded to nearest even, saturating at 448;
 *   elements rounded to the nearest E2M1 grid value, ties to the even code.
 *   FP4 indexer K (the pages' storage precision, implied by the 890 B/token
 *   accounting of [TIT] and [EOG] 5.3: 2.5 entries/token x (288 B main KV +
 *   68 B indexer K); [EOG] 3.4 says the predecessor already ran FP4 on the
 *   indexer Q/K and names the OCP MXFP4 standard for the cache): read as OCP
 *   MXFP4 proper, 128 E2M1 codes (64 B) + one E8M0 scale per 32 channels
 *   (4 B), X = 2^(floor(log2 amax) - 2), elements = nearest E2M1 value of
 *   x / X, ties to even, saturating at 6.
 *   FP8 window KV ([EOG] 3.4 keeps the SWA KV in FP8; the element type and
 *   scaling follow the OCP MX standard the same passage names, i.e. MXFP8):
 *   E4M3 elements, one E8M0 scale per 32 channels, X = 2^(floor(log2 amax) -
 *   8), elements = nearest E4M3 value of x / X, ties to even, saturating.
 *
 * Precision: bf16 / E4M3 / E2M1 inputs are decoded exactly into double; dot
 * products, weighted sums and the softmax accumulate in double. The scale
 * choice (amax / 6) is made in float, as the path defines it, and scores are
 * stored as float because the score array handed to Top-K is float.
 *
 * Parallelism: OpenMP over independent queries / rows only.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_IDX_HEADS 32
#define ORC_IDX_DIM 128
#define ORC_HEADS 64
#define ORC_DIM 512
#define ORC_GROUP 16
#define ORC_RECORD (ORC_DIM / 2 + ORC_DIM / ORC_GROUP) /* 256 code bytes + 32 scale bytes */
#define ORC_KBLOCK 32                                   /* channels per indexer-K E8M0 scale */
#define ORC_KREC (ORC_IDX_DIM / 2 + ORC_IDX_DIM / ORC_KBLOCK) /* 64 code bytes + 4 E8M0 scales */
#define ORC_WBLOCK 32                                   /* channels per FP8 window scale */
#define ORC_WREC (ORC_DIM + ORC_DIM / ORC_WBLOCK)       /* 512 E4M3 codes + 16 E8M0 scales */

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

int orc_record_bytes(void) { return ORC_RECORD; }
int orc_kidx_record_bytes(void) { return ORC_KREC; }
int orc_swa_record_bytes(void) { return ORC_WREC; }

/* bf16 -> double: the bf16 bits are the high half of an IEEE binary32. */
static double bf16_value(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* [OCP] E4M3: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent 15
 * with mantissa 7 is NaN, there is no infinity; exponent 0 is subnormal. */
double orc_e4m3_value(uint8_t b) {
    int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        mag = ldexp((double)m / 8.0, -6);
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* [OCP] E2M1: sign, 2 exponent bits (bias 1), 1 mantissa bit; exponent 0 is
 * subnormal (0 or 0.5). [EOG] 3.4 names E2M1 as the main-KV element type. */
double orc_e2m1_value(uint8_t nib) {
    int s = (nib >> 3) & 1, e = (nib >> 1) & 3, m = nib & 1;
    double mag;
    if (e == 0)
        mag = 0.5 * (double)m;
    else
        mag = ldexp(1.0 + (double)m / 2.0, e - 1);
    return s ? -mag : mag;
}

/* Nearest non-negative finite E4M3 value to v >= 0 (codes 0x00..0x7E are
 * increasing in value); an exact tie goes to the even code (mantissa LSB 0);
 * anything above the largest finite value (448) takes 448. */
uint8_t orc_e4m3_encode_nonneg(float v) {
    double x = (double)v;
    int best = 0;
    double bestd = INFINITY;
    if (!(x < 448.0)) return 0x7E; /* saturate, +inf and NaN included */
    for (int c = 0; c <= 0x7E; c++) {
        double d = fabs(x - orc_e4m3_value((uint8_t)c));
        if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) {
            bestd = d;
            best = c;
        }
    }
    return (uint8_t)best;
}

/* Nearest E2M1 grid value v*S to x (S > 0), ties to the even code; values
 * beyond 6S take 6S; magnitude code 0 is always +0. Returns the 4-bit code. */
uint8_t orc_e2m1_encode(double x, double S) {
    double a = fabs(x);
    int best = 0;
    double bestd = INFINITY;
    if (a >= 6.0 * S) {
        best = 7;
    } else {
        for (int c = 0; c < 8; c++) {
            double d = fabs(a - orc_e2m1_value((uint8_t)c) * S);
            if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) {
                bestd = d;
                best = c;
            }
        }
    }
    if (best != 0 && x < 0) best |= 8;
    return (uint8_t)best;
}

/* [EOG] 3.4, [NXB] 2.3: one main-KV entry = 512 channels of E2M1 plus one
 * E4M3 scale per 16 channels, no second-level scale. Record layout (this
 * build's choice): bytes [0,256) hold channel 2j in the low nibble and 2j+1
 * in the high nibble of byte j; bytes [256,288) hold the scale of channels
 * 16g..16g+15 in byte 256+g. Quantization happens after RoPE, so x already
 * carries it. Scale = E4M3(amax/6), amax/6 computed in float. */
void orc_fp4_pack(const uint16_t* x, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; r++) {
        const uint16_t* xr = x + r * ORC_DIM;
        uint8_t* o = out + r * ORC_RECORD;
        memset(o, 0, ORC_RECORD);
        for (int g = 0; g < ORC_DIM / ORC_GROUP; g++) {
            float amax = 0.0f;
            for (int c = 0; c < ORC_GROUP; c++) {
                float v = (float)bf16_value(xr[g * ORC_GROUP + c]);
                float a = fabsf(v);
                if (a > amax) amax = a;
            }
            float a6 = amax / 6.0f;
            uint8_t sb = orc_e4m3_encode_nonneg(a6);
            double S = orc_e4m3_value(sb);
            o[ORC_DIM / 2 + g] = sb;
            for (int c = 0; c < ORC_GROUP; c++) {
                int ch = g * ORC_GROUP + c;
                uint8_t code = (S == 0.0) ? 0 : orc_e2m1_encode(bf16_value(xr[ch]), S);
                o[ch / 2] |= (uint8_t)(code << (4 * (ch & 1)));
            }
        }
    }
}

/* Value of channel c of one record: E2M1(code) * E4M3(scale). Exact in double. */
static double record_value(const uint8_t* rec, int c) {
    uint8_t code = (rec[c / 2] >> (4 * (c & 1))) & 15;
    return orc_e2m1_value(code) * orc_e4m3_value(rec[ORC_DIM / 2 + c / ORC_GROUP]);
}

void orc_fp4_unpack(const uint8_t* in, int64_t n, double* out) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; r++)
        for (int c = 0; c < ORC_DIM; c++) out[r * ORC_DIM + c] = record_value(in + r * ORC_RECORD, c);
}

/* [OCP] E8M0 scale: the value 2^(b - 127); b = 255 is NaN. */
double orc_e8m0_value(uint8_t b) { return b == 255 ? NAN : ldexp(1.0, (int)b - 127); }

/* OCP MX shared-scale exponent of a block whose largest magnitude is amax, for
 * elements whose largest power of two is 2^emax: floor(log2 amax) - emax,
 * clamped to the E8M0 range [-127, 127]; an all-zero block takes -127. */
static int mx_scale_exp(double amax, int emax) {
    int e, xe = -127;
    if (amax > 0.0) {
        frexp(amax, &e); /* amax = f * 2^e, 0.5 <= f < 1: floor(log2 amax) = e - 1 */
        xe = e - 1 - emax;
        if (xe < -127) xe = -127;
        if (xe > 127) xe = 127;
    }
    return xe;
}

/* FP4 indexer-K entry, read as OCP MXFP4 ([EOG] 3.4 names the OCP MXFP4
 * standard and says the indexer Q/K already ran in FP4; the 68 B size comes
 * from the 890 B/token accounting). Per block of 32 channels: X =
 * 2^(floor(log2 amax) - 2), 2 being the exponent of E2M1's largest power of
 * two (4); each element is the E2M1 value nearest to x / X (exact: X is a
 * power of two), ties to the even code, magnitudes past 6 taking 6, zero
 * magnitude +0. Layout: bytes [0,64) hold channel 2j in the low nibble and
 * 2j+1 in the high nibble of byte j; byte 64+g holds the E8M0 scale of
 * channels 32g..32g+31. */
void orc_kidx_fp4_pack(const uint16_t* x, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; r++) {
        const uint16_t* xr = x + r * ORC_IDX_DIM;
        uint8_t* o = out + r * ORC_KREC;
        memset(o, 0, ORC_KREC);
        for (int g = 0; g < ORC_IDX_DIM / ORC_KBLOCK; g++) {
            double amax = 0.0;
            for (int c = 0; c < ORC_KBLOCK; c++) {
                double a = fabs(bf16_value(xr[g * ORC_KBLOCK + c]));
                if (a > amax) amax = a;
            }
            int xe = mx_scale_exp(amax, 2);
            o[ORC_IDX_DIM / 2 + g] = (uint8_t)(xe + 127);
            for (int c = 0; c < ORC_KBLOCK; c++) {
                int ch = g * ORC_KBLOCK + c;
                /* nearest grid value v * X of x: the same rule as the main KV
                 * with the power-of-two scale X */
                uint8_t code = orc_e2m1_encode(bf16_value(xr[ch]), ldexp(1.0, xe));
                o[ch / 2] |= (uint8_t)(code << (4 * (ch & 1)));
            }
        }
    }
}

/* Channel c of an FP4 indexer-K entry: E2M1(code) * E8M0(scale of its block),
 * exact in double. */
static double kidx_fp4_value(const uint8_t* rec, int c) {
    return orc_e2m1_value((rec[c / 2] >> (4 * (c & 1))) & 15) * orc_e8m0_value(rec[ORC_IDX_DIM / 2 + c / ORC_KBLOCK]);
}

void orc_kidx_fp4_unpack(const uint8_t* in, int64_t n, double* out) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; r++)
        for (int c = 0; c < ORC_IDX_DIM; c++) out[r * ORC_IDX_DIM + c] = kidx_fp4_value(in + r * ORC_KREC, c);
}


/* FP8 window-KV row ([EOG] 3.4: the quantization-sensitive SWA KV stays in
 * FP8; read here as the OCP MX block format that passage names, with E4M3
 * elements). Per block of 32 channels: X = 2^(floor(log2 amax) - 8), 8 being
 * the exponent of the largest power of two E4M3 holds, clamped to the E8M0
 * range [-127, 127] (amax = 0 gives 2^-127); each element is the nearest E4M3
 * value of x / X (exact: X is a power of two), ties to the even code, values
 * past 448 taking 448; a zero magnitude is +0. Layout: bytes 0..511 the codes
 * in channel order, byte 512 + g the scale of channels 32g .. 32g+31.
 * Inputs are finite. */
void orc_swa_fp8_pack(const uint16_t* x, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; r++) {
        const uint16_t* row = x + r * ORC_DIM;
        uint8_t* rec = out + r * ORC_WREC;
        for (int g = 0; g < ORC_DIM / ORC_WBLOCK; g++) {
            double amax = 0.0;
            for (int i = 0; i < ORC_WBLOCK; i++) {
                double a = fabs(bf16_value(row[g * ORC_WBLOCK + i]));
                if (a > amax) amax = a;
            }
            int xe = mx_scale_exp(amax, 8);
            rec[ORC_DIM + g] = (uint8_t)(xe + 127);
            for (int i = 0; i < ORC_WBLOCK; i++) {
                double v = bf16_value(row[g * ORC_WBLOCK + i]);
                uint8_t mag = orc_e4m3_encode_nonneg((float)ldexp(fabs(v), -xe));
                rec[g * ORC_WBLOCK + i] = (uint8_t)(mag | ((v < 0.0 && mag != 0) ? 0x80 : 0x00));
            }
        }
    }
}

/* Value of channel c of one FP8 window row: E4M3(code) * E8M0(scale). Exact in double. */
static double swa_fp8_value(const uint8_t* rec, int c) {
    return orc_e4m3_value(rec[c]) * orc_e8m0_value(rec[ORC_DIM + c / ORC_WBLOCK]);
}

void orc_swa_fp8_unpack(const uint8_t* in, int64_t n, double* out) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; r++)
        for (int c = 0; c < ORC_DIM; c++) out[r * ORC_DIM + c] = swa_fp8_value(in + r * ORC_WREC, c);
}

/* Indexer K of entry `row` decoded to double: bf16 (kfmt 0, [.][128] uint16)
 * or the FP4 entry above (kfmt 1, [.][68] bytes). */
static void load_key(const void* k, int kfmt, int64_t row, double* kd) {
    if (kfmt == 0) {
        const uint16_t* kr = (const uint16_t*)k + row * ORC_IDX_DIM;
        for (int c = 0; c < ORC_IDX_DIM; c++) kd[c] = bf16_value(kr[c]);
    } else {
        const uint8_t* kr = (const uint8_t*)k + row * ORC_KREC;
        for (int c = 0; c < ORC_IDX_DIM; c++) kd[c] = kidx_fp4_value(kr, c);
    }
}

/* Indexer score of one entry ([EOG] 3.2: the indexer Q and indexer K score a
 * main-KV entry; 32 heads x 128 dims per [NXB] 3.3):
 *   score = sum_h w_h * max(q_h . k, 0).
 * qd holds the query's 32 x 128 values already decoded to double, kd the key. */
static double index_score(const double* qd /*[32][128]*/, const float* w /*[32]*/, const double* kd /*[128]*/) {
    double s = 0.0;
    for (int h = 0; h < ORC_IDX_HEADS; h++) {
        double d = 0.0;
        for (int c = 0; c < ORC_IDX_DIM; c++) d += qd[h * ORC_IDX_DIM + c] * kd[c];
        s += (double)w[h] * (d > 0.0 ? d : 0.0);
    }
    return s;
}

/* The 32 x 128 indexer query of query q decoded to double: bf16 (qfmt 0,
 * [.][32][128] uint16) or, for the indexer Q in FP4 ([EOG] 3.4: the
 * predecessor already trained the indexer Q and K in FP4), one MXFP4 entry per
 * head in the indexer-K entry format above (qfmt 1, [.][32][68] bytes). */
static void decode_query(const void* q_all, int qfmt, int64_t q, double* qd) {
    if (qfmt == 0) {
        const uint16_t* qq = (const uint16_t*)q_all + q * ORC_IDX_HEADS * ORC_IDX_DIM;
        for (int t = 0; t < ORC_IDX_HEADS * ORC_IDX_DIM; t++) qd[t] = bf16_value(qq[t]);
    } else {
        const uint8_t* qq = (const uint8_t*)q_all + q * ORC_IDX_HEADS * ORC_KREC;
        for (int h = 0; h < ORC_IDX_HEADS; h++)
            for (int c = 0; c < ORC_IDX_DIM; c++) qd[h * ORC_IDX_DIM + c] = kidx_fp4_value(qq + h * ORC_KREC, c);
    }
}

/* Full-mode scoring ([TIT] CSA2 Full mode; [EOG] 3.3 first indexer scans every
 * visible position). Query q reads sequence q / q_per_seq; entries at or past
 * n_visible[q] (or N when n_visible is NULL) score -inf. Scores are stored as
 * float. When block_size > 0, block j's score is the max over its positions
 * [j*bs, j*bs+bs) ([EOG] 3.3: each block takes its highest index score). */
static void index_full_any(const void* q_idx, int qfmt, const float* w, const void* k_idx, int kfmt, int64_t N,
                           int32_t nq, int32_t q_per_seq, const int32_t* n_visible, float* scores,
                           int32_t block_size, float* block_scores) {
    const int64_t CH = 4096; /* entries per parallel work item */
    int64_t nch = (N + CH - 1) / CH;
    double* qd = (double*)malloc(sizeof(double) * (size_t)(nq > 0 ? nq : 1) * ORC_IDX_HEADS * ORC_IDX_DIM);
    for (int32_t q = 0; q < nq; q++) decode_query(q_idx, qfmt, q, qd + (int64_t)q * ORC_IDX_HEADS * ORC_IDX_DIM);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t item = 0; item < (int64_t)nq * nch; item++) {
        int32_t q = (int32_t)(item / nch);
        int64_t i0 = (item % nch) * CH;
        int64_t seq = q / q_per_seq;
        int64_t nv = n_visible ? n_visible[q] : N;
        const double* qq = qd + (int64_t)q * ORC_IDX_HEADS * ORC_IDX_DIM;
        const float* ww = w + (int64_t)q * ORC_IDX_HEADS;
        float* srow = scores + (int64_t)q * N;
        double kd[ORC_IDX_DIM];
        for (int64_t i = i0; i < i0 + CH && i < N; i++) {
            if (i < nv) {
                load_key(k_idx, kfmt, seq * N + i, kd);
                srow[i] = (float)index_score(qq, ww, kd);
            } else {
                srow[i] = -INFINITY;
            }
        }
    }
    free(qd);
    if (block_size > 0) {
        int64_t nb = (N + block_size - 1) / block_size;
        for (int32_t q = 0; q < nq; q++) {
            const float* srow = scores + (int64_t)q * N;
            for (int64_t j = 0; j < nb; j++) {
                float m = -INFINITY;
                for (int64_t i = j * block_size; i < (j + 1) * block_size && i < N; i++)
                    if (srow[i] > m) m = srow[i];
                block_scores[(int64_t)q * nb + j] = m;
            }
        }
    }
}

void orc_index_full(const uint16_t* q_idx, const float* w, const uint16_t* k_idx, int64_t N, int32_t nq,
                    int32_t q_per_seq, const int32_t* n_visible, float* scores, int32_t block_size,
                    float* block_scores) {
    index_full_any(q_idx, 0, w, k_idx, 0, N, nq, q_per_seq, n_visible, scores, block_size, block_scores);
}

/* Full-mode scoring over the FP4 indexer-K cache ([N][68] entries). */
void orc_index_full_fp4k(const uint16_t* q_idx, const float* w, const uint8_t* k_fp4, int64_t N, int32_t nq,
                         int32_t q_per_seq, const int32_t* n_visible, float* scores, int32_t block_size,
                         float* block_scores) {
    index_full_any(q_idx, 0, w, k_fp4, 1, N, nq, q_per_seq, n_visible, scores, block_size, block_scores);
}

/* Full-mode scoring with both the indexer Q and the indexer K as MXFP4 entries
 * ([EOG] 3.4: the indexer Q/K already ran in FP4 in the predecessor; entry
 * format of orc_kidx_fp4_pack, one entry per query head): q_fp4 [nq][32][68],
 * k_fp4 [nseq][N][68]. The score is the same formula over the decoded values,
 * accumulated in double and stored as float. */
void orc_index_full_fp4qk(const uint8_t* q_fp4, const float* w, const uint8_t* k_fp4, int64_t N, int32_t nq,
                          int32_t q_per_seq, const int32_t* n_visible, float* scores, int32_t block_size,
                          float* block_scores) {
    index_full_any(q_fp4, 1, w, k_fp4, 1, N, nq, q_per_seq, n_visible, scores, block_size, block_scores);
}

/* Candidate pool ([EOG] 3.3): the chosen blocks' positions, in block order.
 * A block id < 0 (padding) gives id -1 for its positions. */
void orc_pool_ids(const int32_t* blocks, int32_t nq, int32_t nb, int32_t block_size, int32_t* pool) {
    for (int64_t q = 0; q < nq; q++)
        for (int64_t j = 0; j < nb; j++) {
            int32_t b = blocks[q * nb + j];
            for (int t = 0; t < block_size; t++)
                pool[(q * nb + j) * block_size + t] = (b < 0) ? -1 : b * block_size + t;
        }
}

/* Reindex-mode scoring ([TIT] Reindex mode; [EOG] 3.3 later indexers score only
 * inside the pool): the layer's own (Q_idx, w) over the shared indexer K, for
 * the pool positions only. Positions whose id is -1 or not visible score -inf. */
static void index_reindex_any(const void* q_idx, int qfmt, const float* w, const void* k_idx, int kfmt, int64_t N,
                              int32_t nq, int32_t q_per_seq, const int32_t* n_visible, const int32_t* pool,
                              int64_t pool_len, float* pool_scores) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t q = 0; q < nq; q++) {
        double qd[ORC_IDX_HEADS * ORC_IDX_DIM];
        int64_t seq = q / q_per_seq;
        int64_t nv = n_visible ? n_visible[q] : N;
        if (nv > N) nv = N;
        decode_query(q_idx, qfmt, q, qd);
        const float* ww = w + (int64_t)q * ORC_IDX_HEADS;
        double kd[ORC_IDX_DIM];
        for (int64_t p = 0; p < pool_len; p++) {
            int64_t id = pool[(int64_t)q * pool_len + p];
            if (id >= 0 && id < nv) {
                load_key(k_idx, kfmt, seq * N + id, kd);
                pool_scores[(int64_t)q * pool_len + p] = (float)index_score(qd, ww, kd);
            } else {
                pool_scores[(int64_t)q * pool_len + p] = -INFINITY;
            }
        }
    }
}

void orc_index_reindex(const uint16_t* q_idx, const float* w, const uint16_t* k_idx, int64_t N, int32_t nq,
                       int32_t q_per_seq, const int32_t* n_visible, const int32_t* pool, int64_t pool_len,
                       float* pool_scores) {
    index_reindex_any(q_idx, 0, w, k_idx, 0, N, nq, q_per_seq, n_visible, pool, pool_len, pool_scores);
}

/* Reindex-mode scoring over the FP4 indexer-K cache. */
void orc_index_reindex_fp4k(const uint16_t* q_idx, const float* w, const uint8_t* k_fp4, int64_t N, int32_t nq,
                            int32_t q_per_seq, const int32_t* n_visible, const int32_t* pool, int64_t pool_len,
                            float* pool_scores) {
    index_reindex_any(q_idx, 0, w, k_fp4, 1, N, nq, q_per_seq, n_visible, pool, pool_len, pool_scores);
}

/* Reindex-mode scoring with the indexer Q and K both as MXFP4 entries
 * (q_fp4 [nq][32][68], as orc_index_full_fp4qk). */
void orc_index_reindex_fp4qk(const uint8_t* q_fp4, const float* w, const uint8_t* k_fp4, int64_t N, int32_t nq,
                             int32_t q_per_seq, const int32_t* n_visible, const int32_t* pool, int64_t pool_len,
                             float* pool_scores) {
    index_reindex_any(q_fp4, 1, w, k_fp4, 1, N, nq, q_per_seq, n_visible, pool, pool_len, pool_scores);
}

typedef struct {
    float s;
    int64_t i;
} orc_pair;

/* Rank order: higher score first; equal scores (-0 == +0) by lower position. */
static int pair_rank_cmp(const void* a, const void* b) {
    const orc_pair* x = (const orc_pair*)a;
    const orc_pair* y = (const orc_pair*)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->i < y->i) ? -1 : (x->i > y->i);
}

static int i64_cmp(const void* a, const void* b) {
    int64_t x = *(const int64_t*)a, y = *(const int64_t*)b;
    return (x > y) - (x < y);
}

/* Per-row Top-K ([TIT] Full / Reindex select Top-512; [EOG] 3.3 picks the
 * best blocks): sort the row's finite-or-+inf scores by (score desc, position
 * asc), keep the first min(K, count); -inf and NaN are never chosen. Output:
 * the chosen positions ascending (mapped through id_map when given), padded
 * with -1 to K. Positions at or past row_len[r] are not candidates. */
void orc_topk(const float* scores, int32_t rows, int64_t ncols, int64_t ld, const int32_t* row_len, int32_t k,
              const int32_t* id_map, int32_t* out_idx) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t r = 0; r < rows; r++) {
        int64_t len = row_len ? row_len[r] : ncols;
        if (len > ncols) len = ncols;
        orc_pair* v = (orc_pair*)malloc(sizeof(orc_pair) * (size_t)(len > 0 ? len : 1));
        int64_t cnt = 0;
        for (int64_t i = 0; i < len; i++) {
            float s = scores[(int64_t)r * ld + i];
            if (isnan(s) || s == -INFINITY) continue;
            v[cnt].s = s;
            v[cnt].i = i;
            cnt++;
        }
        qsort(v, (size_t)cnt, sizeof(orc_pair), pair_rank_cmp);
        int64_t take = cnt < k ? cnt : k;
        int64_t* ids = (int64_t*)malloc(sizeof(int64_t) * (size_t)(take > 0 ? take : 1));
        for (int64_t t = 0; t < take; t++) ids[t] = v[t].i;
        qsort(ids, (size_t)take, sizeof(int64_t), i64_cmp);
        for (int64_t t = 0; t < k; t++) {
            int32_t o = -1;
            if (t < take) o = id_map ? id_map[(int64_t)r * ld + ids[t]] : (int32_t)ids[t];
            out_idx[(int64_t)r * k + t] = o;
        }
        free(ids);
        free(v);
    }
}

/* Sparse MQA attention ([EOG] 3.2: a query attends only to its selected entries
 * plus its layer's SWA KV; 64 query heads of dim 512 share one KV head; [EOG]
 * 3.4: the FP4 cache is dequantized before the attention math). Keys = values
 * = [deq(main[i]) for i in idx, skipping -1] followed by swa rows
 * [start, start+len). One softmax per head over all of them:
 *   l_j = scale * (q_h . k_j); out_h = sum_j softmax(l)_j v_j;
 *   lse_h = log sum_j exp(l_j). No key at all: out = 0, lse = -inf. */
static void sparse_attn_any(const uint16_t* q, const uint8_t* kv, int64_t N, int32_t nq, int32_t q_per_seq,
                            const int32_t* idx, int32_t k, const void* swa, int swa_fmt, int64_t T,
                            const int32_t* swa_start, const int32_t* swa_len, double softmax_scale, double* out,
                            double* lse) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t qi = 0; qi < nq; qi++) {
        int64_t seq = qi / q_per_seq;
        int64_t slen = swa_len ? swa_len[qi] : 0;
        int64_t sst = swa_start ? swa_start[qi] : 0;
        int64_t nkeys_max = (int64_t)k + slen;
        double* keys = (double*)malloc(sizeof(double) * (size_t)(nkeys_max > 0 ? nkeys_max : 1) * ORC_DIM);
        double* logit = (double*)malloc(sizeof(double) * (size_t)(nkeys_max > 0 ? nkeys_max : 1));
        int64_t nk = 0;
        for (int32_t t = 0; t < k; t++) {
            int32_t id = idx[(int64_t)qi * k + t];
            if (id < 0) continue;
            const uint8_t* rec = kv + (seq * N + id) * ORC_RECORD;
            for (int c = 0; c < ORC_DIM; c++) keys[nk * ORC_DIM + c] = record_value(rec, c);
            nk++;
        }
        for (int64_t t = 0; t < slen; t++) {
            const int64_t r = seq * T + sst + t;
            if (swa_fmt == 1) {
                const uint8_t* rec = (const uint8_t*)swa + r * ORC_WREC;
                for (int c = 0; c < ORC_DIM; c++) keys[nk * ORC_DIM + c] = swa_fp8_value(rec, c);
            } else {
                const uint16_t* row = (const uint16_t*)swa + r * ORC_DIM;
                for (int c = 0; c < ORC_DIM; c++) keys[nk * ORC_DIM + c] = bf16_value(row[c]);
            }
            nk++;
        }
        for (int h = 0; h < ORC_HEADS; h++) {
            const uint16_t* qh = q + ((int64_t)qi * ORC_HEADS + h) * ORC_DIM;
            double* oh = out + ((int64_t)qi * ORC_HEADS + h) * ORC_DIM;
            if (nk == 0) {
                for (int c = 0; c < ORC_DIM; c++) oh[c] = 0.0;
                if (lse) lse[(int64_t)qi * ORC_HEADS + h] = -INFINITY;
                continue;
            }
            double m = -INFINITY;
            for (int64_t j = 0; j < nk; j++) {
                double d = 0.0;
                for (int c = 0; c < ORC_DIM; c++) d += bf16_value(qh[c]) * keys[j * ORC_DIM + c];
                logit[j] = softmax_scale * d;
                if (logit[j] > m) m = logit[j];
            }
            double den = 0.0;
            for (int c = 0; c < ORC_DIM; c++) oh[c] = 0.0;
            for (int64_t j = 0; j < nk; j++) {
                double p = exp(logit[j] - m);
                den += p;
                for (int c = 0; c < ORC_DIM; c++) oh[c] += p * keys[j * ORC_DIM + c];
            }
            for (int c = 0; c < ORC_DIM; c++) oh[c] /= den;
            if (lse) lse[(int64_t)qi * ORC_HEADS + h] = m + log(den);
        }
        free(logit);
        free(keys);
    }
}

void orc_sparse_attn(const uint16_t* q, const uint8_t* kv, int64_t N, int32_t nq, int32_t q_per_seq,
                     const int32_t* idx, int32_t k, const uint16_t* swa, int64_t T, const int32_t* swa_start,
                     const int32_t* swa_len, double softmax_scale, double* out, double* lse) {
    sparse_attn_any(q, kv, N, nq, q_per_seq, idx, k, swa, 0, T, swa_start, swa_len, softmax_scale, out, lse);
}

/* The same attention with the window rows as FP8 records (orc_swa_fp8_pack). */
void orc_sparse_attn_fp8w(const uint16_t* q, const uint8_t* kv, int64_t N, int32_t nq, int32_t q_per_seq,
                          const int32_t* idx, int32_t k, const uint8_t* swa_fp8, int64_t T,
                          const int32_t* swa_start, const int32_t* swa_len, double softmax_scale, double* out,
                          double* lse) {
    sparse_attn_any(q, kv, N, nq, q_per_seq, idx, k, swa_fp8, 1, T, swa_start, swa_len, softmax_scale, out, lse);
}
