// Device helpers shared by the CSA2 HIP kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define CSA2_DEVINL __device__ __forceinline__

namespace csa2 {

constexpr int kDim = 512;      // main-KV channels = attention head dim
constexpr int kHeads = 64;     // attention query heads (one shared KV head)
constexpr int kIdxHeads = 32;  // indexer heads
constexpr int kIdxDim = 128;   // indexer head dim
constexpr int kGroup = 16;     // channels per E4M3 scale
constexpr int kCodeBytes = kDim / 2;
constexpr int kRecord = kCodeBytes + kDim / kGroup;  // 288
constexpr int kMaxWindow = 128;
constexpr int kKidxBlock = 32;                            // channels per E8M0 scale of an FP4 indexer-K entry
constexpr int kKidxRecord = kIdxDim / 2 + kIdxDim / kKidxBlock;  // 68

// Attention status bits (the first word of its workspace; ORed, never cleared).
constexpr uint32_t kStatusIdx = 1u;       // a selected id outside [-1, N)
constexpr uint32_t kStatusWinLen = 2u;    // swa_len outside [0, 128]
constexpr uint32_t kStatusWinRange = 4u;  // window rows outside [0, T)
constexpr uint32_t kStatusNonFinite = 8u; // a non-finite output (a window value fp16 cannot hold, a NaN scale, ...)
constexpr size_t kStatusBytes = 256;      // the status word's share of the workspace

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

CSA2_DEVINL bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }
CSA2_DEVINL bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

CSA2_DEVINL float bf16_bits_to_float(uint32_t b) { return __uint_as_float(b << 16); }

// Two floats -> packed bf16 pair (lo in bits 0..15), round to nearest even:
// one v_cvt_pk_bf16_f32 on gfx950.
CSA2_DEVINL uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// 32x32x16 bf16 MFMA: A 32x16 (lane l: row l%32, k (l/32)*8..+8), B 16x32
// (lane l: col l%32, same k), C/D 32x32 (lane l, reg r: col l%32,
// row (r/4)*8 + (l/32)*4 + r%4).
CSA2_DEVINL f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16x16x32 bf16 MFMA: A 16x32 (lane l: row l%16, k (l/16)*8..+8), B 32x16
// (lane l: col l%16, same k), C/D 16x16 (lane l, reg r: col l%16, row (l/16)*4 + r).
CSA2_DEVINL f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// OCP E4M3 byte -> float (exact): exponent bias 7, exponent 0 subnormal
// (m * 2^-9), 0x7F / 0xFF NaN.
CSA2_DEVINL float e4m3_to_float(uint32_t b) {
    const uint32_t e = (b >> 3) & 15u, m = b & 7u;
    float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
    if (e == 15u && m == 7u) mag = __builtin_nanf("");
    return (b & 0x80u) ? -mag : mag;
}

// Nearest E4M3 code of v >= 0 (v finite or +inf), ties to even, saturating at
// 448 (0x7E). Rounds the binary32 significand to 3 bits directly; values under
// 2^-6 are counted in units of the subnormal step 2^-9.
CSA2_DEVINL uint32_t e4m3_encode_rne_sat(float v) {
    if (v < 0.015625f) return (uint32_t)__builtin_rintf(v * 512.0f);  // 0..8, 8 == 2^-6 == code 0x08
    uint32_t u = __float_as_uint(v);
    u += 0x7FFFFu + ((u >> 20) & 1u);
    const uint32_t code = (u >> 20) - (120u << 3);
    return code > 0x7Eu ? 0x7Eu : code;
}

// Eight FP4 channels -> four packed bf16 pairs. `w` holds channels 2b (bits
// 8b..8b+3) and 2b+1 (bits 8b+4..8b+7) for b = 0..3; `half_scale` = S/2.
// |E2M1| * 2 is an integer in {0,1,2,3,4,6,8,12}; the product with S/2 is exact
// in fp32 and in bf16, so the bf16 is the high half of the fp32 result.
CSA2_DEVINL void dequant8(uint32_t w, float half_scale, uint32_t out[4]) {
    const uint32_t ilo = __builtin_amdgcn_perm(0x0C080604u, 0x03020100u, w & 0x07070707u);
    const uint32_t ihi = __builtin_amdgcn_perm(0x0C080604u, 0x03020100u, (w >> 4) & 0x07070707u);
#pragma unroll
    for (int b = 0; b < 4; b++) {
        const float fe = (float)((ilo >> (8 * b)) & 0xFFu) * half_scale;
        const float fo = (float)((ihi >> (8 * b)) & 0xFFu) * half_scale;
        // sign of the product = sign of the scale XOR the code's sign bit
        const uint32_t ue = __float_as_uint(fe) ^ ((w << (28 - 8 * b)) & 0x80000000u);
        const uint32_t uo = __float_as_uint(fo) ^ ((w << (24 - 8 * b)) & 0x80000000u);
        out[b] = __builtin_amdgcn_perm(uo, ue, 0x07060302u);
    }
}

// Workgroup barrier that orders LDS only. __syncthreads() also drains every
// outstanding global load (s_waitcnt vmcnt(0)), which would stall prefetches
// that are meant to stay in flight across the barrier.
CSA2_DEVINL void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// max(x, 0) for a float that is not NaN, taken on its bit pattern: a float
// with the sign bit clear compares like its int32 bits, one with the sign bit
// set is a negative int32. One v_max_i32, where fmaxf(x, 0) on a value the
// compiler cannot prove canonical costs a canonicalising max as well.
CSA2_DEVINL float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Lanes 0..31 receive x from lane l + 32 (v_permlane32_swap exchanges lanes
// 32..63 of its first operand with lanes 0..31 of its second; element 1 of the
// result is the second operand after the swap). Lanes 32..63 get their own x.
CSA2_DEVINL float from_upper_half(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[1]);
}

// Maximum over the aligned group of 8 lanes, in every lane of the group, with
// DPP moves (quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror)
// instead of LDS-routed shuffles.
CSA2_DEVINL float max8_lanes(float v) {
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, true)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, true)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, true)));
    return v;
}

CSA2_DEVINL float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

}  // namespace csa2
