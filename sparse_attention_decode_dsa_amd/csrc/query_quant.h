// Indexer query quantization, shared by the standalone kernel
// (dsa_quantize_q) and the indexer, which quantizes its own queries, so both
// produce the same codes bit for bit.
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
