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

// q * 2^-e in one exact step (v_ldexp_f32: a single rounding, and only where
// the result is below the fp32 normal range, far under the smallest fp8
// subnormal, so every such value still codes to a signed zero).
struct IdxQFactors {
    int neg_e;
};
__device__ __forceinline__ IdxQFactors idx_q_factors(int e) {
    return IdxQFactors{-e};
}

// Two codes (round to nearest even into E4M3FN; |q * 2^-e| <= 448 by
// construction) in the low 16 bits.
__device__ __forceinline__ uint32_t idx_q_code2(float x0, float x1, IdxQFactors f) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(x0, f.neg_e),
                                                     __builtin_amdgcn_ldexpf(x1, f.neg_e), 0, false) & 0xFFFFu;
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
