// Query quantization shared by the standalone preparation kernels and the
// kernels that quantize their own queries (the indexer, the sparse MLA), so
// both produce the same codes bit for bit.
#pragma once

#include "device_common.h"

namespace dsa {

// Indexer query head: fp8 E4M3FN codes with one power-of-two scale 2^e, e the
// smallest exponent with amax <= 448 * 2^e (0 for an all-zero head).  With
// amax = m * 2^E, m in [0.5, 1), and 448 = 0.875 * 2^9: e = E - 9 if
// m <= 0.875, else E - 8.
__device__ __forceinline__ int idx_q_exponent(float amax) {
    int e = 0;
    if (amax > 0.0f) {
        int ex;
        const float m = frexpf(amax, &ex);
        e = (m <= 0.875f) ? ex - 9 : ex - 8;
    }
    return e;
}

// q * 2^-e is taken in two exact power-of-two steps, (q * f1) * f2, so that
// no factor leaves the fp32 range.
struct IdxQFactors {
    float f1, f2;
};
__device__ __forceinline__ IdxQFactors idx_q_factors(int e) {
    const int h1 = (-e) / 2, h2 = -e - h1;
    return IdxQFactors{ldexpf(1.0f, h1), ldexpf(1.0f, h2)};
}

// Two codes (round to nearest even into E4M3FN; |q * 2^-e| <= 448 by
// construction) in the low 16 bits.
__device__ __forceinline__ uint32_t idx_q_code2(float x0, float x1, IdxQFactors f) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32((x0 * f.f1) * f.f2, (x1 * f.f1) * f.f2, 0, false) & 0xFFFFu;
}

// MLA query head: scale s = 2^ceil(log2(amax / 448)) (1 for a zero head).
__device__ __forceinline__ float mla_q_scale(float amax) {
    float s = 1.0f;
    if (amax > 0.0f) {
        int e;
        const float m = frexpf(amax / 448.0f, &e);   // amax / 448 = m 2^e, m in [0.5, 1)
        s = ldexpf(1.0f, m == 0.5f ? e - 1 : e);      // smallest power of two >= amax / 448
    }
    return s;
}

// Two fp8 E4M3FN terms of four scaled values x = q / s: hi = RNE(x),
// lo = RNE(16 (x - hi)), packed four bytes to a word each.  x - hi is exact
// in fp32; a bf16 value has 8 significant bits and hi carries the top 4, so
// lo is exact too wherever 16 (x - hi) is an E4M3 value.
__device__ __forceinline__ void mla_q_split4(float x0, float x1, float x2, float x3, uint32_t& hw, uint32_t& lw) {
    const float x[4] = {x0, x1, x2, x3};
    float l4[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const uint32_t hbyte = __builtin_amdgcn_cvt_pk_fp8_f32(x[u], 0.0f, 0, false) & 0xFFu;
        l4[u] = 16.0f * (x[u] - __builtin_amdgcn_cvt_f32_fp8(hbyte, 0));
    }
    int hp = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
    hp = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, hp, true);
    int lp = __builtin_amdgcn_cvt_pk_fp8_f32(l4[0], l4[1], 0, false);
    lp = __builtin_amdgcn_cvt_pk_fp8_f32(l4[2], l4[3], lp, true);
    hw = (uint32_t)hp;
    lw = (uint32_t)lp;
}

// bf16 bit patterns of a 16-byte chunk -> 8 floats.
__device__ __forceinline__ void bf16x8_to_f32(const uint4& c, float (&v)[8]) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        v[2 * k] = __uint_as_float(w[k] << 16);
        v[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
    }
}

}  // namespace dsa
