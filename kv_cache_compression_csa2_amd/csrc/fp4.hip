// FP4 main-KV records: pack (bf16 -> E2M1 codes + E4M3 scales) and unpack.
// Format: eogee.com report on DeepSeek-V4.1-Flash, 3.4 (E2M1 elements, one
// E4M3 scale per 16 channels, no second-level scale); nxbn.cn walkthrough 2.3.
#include "device_common.h"
#include "launch.h"

namespace csa2 {

// One thread per 16-channel group: 32 threads per 512-channel row, so a wave
// covers two rows; loads are 32 contiguous bytes per thread.
__global__ __launch_bounds__(256) void fp4_pack_kernel(const uint16_t* __restrict__ x, int64_t n,
                                                       uint8_t* __restrict__ out) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t row = t >> 5;
    const int g = (int)(t & 31);
    if (row >= n) return;
    const uint4* src = reinterpret_cast<const uint4*>(x + row * kDim + g * kGroup);
    const uint4 v0 = src[0], v1 = src[1];
    const uint32_t wv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    float xs[16];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        xs[2 * i] = bf16_bits_to_float(wv[i] & 0xFFFFu);
        xs[2 * i + 1] = bf16_bits_to_float(wv[i] >> 16);
    }
#pragma unroll
    for (int i = 0; i < 16; i++) amax = fmaxf(amax, fabsf(xs[i]));
    const uint32_t sb = e4m3_encode_rne_sat(amax / 6.0f);
    const float S = e4m3_to_float(sb);
    // Midpoints of the E2M1 grid times S (exact in fp32): an exact tie goes to
    // the neighbour with the even code, so the comparison is >= where the upper
    // neighbour is even (0.75, 1.75, 3.5) and > otherwise.
    const float t025 = 0.25f * S, t075 = 0.75f * S, t125 = 1.25f * S, t175 = 1.75f * S;
    const float t250 = 2.5f * S, t350 = 3.5f * S, t500 = 5.0f * S;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const float a = fabsf(xs[i]);
        uint32_t c = (uint32_t)(a > t025) + (uint32_t)(a >= t075) + (uint32_t)(a > t125) + (uint32_t)(a >= t175) +
                     (uint32_t)(a > t250) + (uint32_t)(a >= t350) + (uint32_t)(a > t500);
        if (S == 0.0f) c = 0;
        if (c != 0 && xs[i] < 0.0f) c |= 8u;
        if (i < 8)
            lo |= c << (4 * i);
        else
            hi |= c << (4 * (i - 8));
    }
    uint8_t* rec = out + row * kRecord;
    *reinterpret_cast<uint2*>(rec + g * 8) = make_uint2(lo, hi);
    rec[kCodeBytes + g] = (uint8_t)sb;
}

// One thread per 16-channel group: 8 code bytes + 1 scale byte -> 32 bytes.
__global__ __launch_bounds__(256) void fp4_unpack_kernel(const uint8_t* __restrict__ in, int64_t n,
                                                         uint16_t* __restrict__ y) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t row = t >> 5;
    const int g = (int)(t & 31);
    if (row >= n) return;
    const uint8_t* rec = in + row * kRecord;
    const uint2 c = *reinterpret_cast<const uint2*>(rec + g * 8);
    const float hs = 0.5f * e4m3_to_float(rec[kCodeBytes + g]);
    uint32_t o[8];
    dequant8(c.x, hs, o);
    dequant8(c.y, hs, o + 4);
    uint4* dst = reinterpret_cast<uint4*>(y + row * kDim + g * kGroup);
    dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
    dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
}

// FP4 indexer-K entries in the OCP MXFP4 format (68 bytes: 64 code bytes, then
// one E8M0 scale per 32 channels), the storage precision implied by the pages'
// 890 B/token accounting (titansim blog; eogee.com report 5.3) in the standard
// eogee.com report 3.4 names. Per block: X = 2^(floor(log2 amax) - 2), 2 being
// the exponent of E2M1's largest power of two, clamped to E8M0's [-127, 127];
// element = nearest E2M1 value of x/X (exact: X is a power of two), ties to the
// even code, past 6 saturating to 6; zero magnitude is +0.
// 16 threads per 128-channel row, 8 channels each: threads 4g..4g+3 of a row
// (aligned lanes of one wave) hold block g. The block maximum is taken on the
// bf16 bit patterns (|x| orders like its 15 low bits), and floor(log2 amax)
// is the exponent field minus 127 for normal values; bf16 subnormals and
// zero blocks fall below the clamp, so the rule needs no float log.
__global__ __launch_bounds__(256) void kidx_fp4_pack_kernel(const uint16_t* __restrict__ x, int64_t n,
                                                            uint8_t* __restrict__ out) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t row = t >> 4;
    const int sl = (int)(t & 15);
    const bool ok = row < n;
    const uint4 v = ok ? reinterpret_cast<const uint4*>(x + row * kIdxDim)[sl] : make_uint4(0u, 0u, 0u, 0u);
    const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
    uint32_t amax_bits = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) amax_bits = max(amax_bits, max(wv[i] & 0x7FFFu, (wv[i] >> 16) & 0x7FFFu));
    amax_bits = max(amax_bits, (uint32_t)__shfl_xor((int)amax_bits, 1));
    amax_bits = max(amax_bits, (uint32_t)__shfl_xor((int)amax_bits, 2));
    if (!ok) return;
    int xe = (int)(amax_bits >> 7) - 127 - 2;
    xe = xe < -127 ? -127 : xe;  // the largest bf16 exponent keeps xe <= 125
    const float inv_x = __uint_as_float((uint32_t)(127 - xe) << 23);  // 2^-xe, a normal float
    uint32_t codes = 0;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const float xv = bf16_bits_to_float((wv[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
        const float a = fabsf(xv) * inv_x;  // exact, or below 2^-126 where the code is 0 anyway
        // nearest grid value; ties go to the even code (>= where the upper
        // neighbour is even: 0.75, 1.75, 3.5)
        uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                     (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
        if (c != 0 && xv < 0.0f) c |= 8u;
        codes |= c << (4 * i);
    }
    uint8_t* dst = out + row * kKidxRecord;
    reinterpret_cast<uint32_t*>(dst)[sl] = codes;
    if ((sl & 3) == 0) dst[kIdxDim / 2 + (sl >> 2)] = (uint8_t)(xe + 127);
}

// FP8 window-KV rows: E4M3 elements with one E8M0 scale per 32 channels, the
// OCP MX block format (eogee.com report 3.4 keeps the window KV in FP8 and
// names the OCP MX standard for the cache formats). Per block:
// X = 2^(floor(log2 amax) - 8), 8 being the exponent of E4M3's largest power
// of two, clamped to E8M0's [-127, 127]; element = nearest E4M3 value of x/X
// (exact: X is a power of two), ties to even, saturating at 448; a zero
// magnitude is +0. Row: 512 code bytes in channel order, then 16 scale bytes.
// Thread = one 32-channel block; 16 threads per row.
constexpr int kSwaRec = kDim + kDim / 32;  // 528

__global__ __launch_bounds__(256) void swa_fp8_pack_kernel(const uint16_t* __restrict__ x, int64_t n,
                                                           uint8_t* __restrict__ out) {
    const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    const int64_t row = t >> 4;
    const int g = (int)(t & 15);
    if (row >= n) return;
    const uint4* src = reinterpret_cast<const uint4*>(x + row * kDim + 32 * g);
    float xs[32];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const uint4 v = src[i];
        const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int k = 0; k < 4; k++) {
            xs[8 * i + 2 * k] = bf16_bits_to_float(wv[k] & 0xFFFFu);
            xs[8 * i + 2 * k + 1] = bf16_bits_to_float(wv[k] >> 16);
        }
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; i++) amax = fmaxf(amax, fabsf(xs[i]));
    int xe = -127;
    if (amax > 0.0f) {
        // amax = m * 2^e with 0.5 <= m < 1, so floor(log2 amax) = e - 1
        xe = __builtin_amdgcn_frexp_expf(amax) - 1 - 8;
        xe = xe < -127 ? -127 : (xe > 127 ? 127 : xe);
    }
    uint32_t codes[8];
#pragma unroll
    for (int w = 0; w < 8; w++) {
        uint32_t word = 0;
#pragma unroll
        for (int b = 0; b < 4; b++) {
            const float v = xs[4 * w + b];
            uint32_t c = e4m3_encode_rne_sat(ldexpf(fabsf(v), -xe));
            if (c != 0 && v < 0.0f) c |= 0x80u;
            word |= c << (8 * b);
        }
        codes[w] = word;
    }
    uint8_t* dst = out + row * kSwaRec;
    reinterpret_cast<uint4*>(dst + 32 * g)[0] = make_uint4(codes[0], codes[1], codes[2], codes[3]);
    reinterpret_cast<uint4*>(dst + 32 * g)[1] = make_uint4(codes[4], codes[5], codes[6], codes[7]);
    dst[kDim + g] = (uint8_t)(xe + 127);
}

int launch_swa_fp8_pack(const uint16_t* x, int64_t n, uint8_t* out, hipStream_t s) {
    if (n == 0) return 0;
    const int64_t blocks = (n * 16 + 255) / 256;
    hipLaunchKernelGGL(swa_fp8_pack_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, n, out);
    return 0;
}

int launch_kidx_fp4_pack(const uint16_t* x, int64_t n, uint8_t* out, hipStream_t s) {
    if (n == 0) return 0;
    const int64_t blocks = (n * 16 + 255) / 256;
    hipLaunchKernelGGL(kidx_fp4_pack_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, n, out);
    return 0;
}

int launch_fp4_pack(const uint16_t* x, int64_t n, uint8_t* out, hipStream_t s) {
    if (n == 0) return 0;
    const int64_t threads = n * 32;
    const int64_t blocks = (threads + 255) / 256;
    hipLaunchKernelGGL(fp4_pack_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, n, out);
    return 0;
}

int launch_fp4_unpack(const uint8_t* in, int64_t n, uint16_t* y, hipStream_t s) {
    if (n == 0) return 0;
    const int64_t threads = n * 32;
    const int64_t blocks = (threads + 255) / 256;
    hipLaunchKernelGGL(fp4_unpack_kernel, dim3((unsigned)blocks), dim3(256), 0, s, in, n, y);
    return 0;
}

}  // namespace csa2
