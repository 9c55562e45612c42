// Query preparation, one wavefront per (row, head):
//   - indexer queries (128 bf16) -> fp8 E4M3FN codes, one power-of-two scale;
//   - MLA queries (576 bf16) -> two fp8 E4M3FN terms and one power-of-two
//     scale s, q = s (hi + lo / 16), read by the sparse MLA kernel's fp8
//     QK products.
// Each has a kernel of its own; a third does both in one launch (the
// indexer pairs first, then the MLA pairs), which is what a decode step
// uses.
#include "device_common.h"
#include "launch.h"

namespace dsa {

__device__ __forceinline__ void quantize_idx_pair(const uint16_t* __restrict__ q, int pair, int lane,
                                                  uint8_t* __restrict__ code, float* __restrict__ scale) {
    const uint32_t w = reinterpret_cast<const uint32_t*>(q + (size_t)pair * 128)[lane];
    const float x0 = __uint_as_float(w << 16);
    const float x1 = __uint_as_float(w & 0xFFFF0000u);
    const float amax = wave_max(fmaxf(fabsf(x0), fabsf(x1)));

    // Smallest e with amax <= 448 * 2^e.  With amax = m * 2^E, m in [0.5, 1)
    // and 448 = 0.875 * 2^9: e = E - 9 if m <= 0.875, else E - 8.
    int e = 0;
    if (amax > 0.0f) {
        int ex;
        const float m = frexpf(amax, &ex);
        e = (m <= 0.875f) ? ex - 9 : ex - 8;
    }
    // q * 2^-e in two exact power-of-two steps so no factor leaves fp32 range.
    const int h1 = (-e) / 2, h2 = -e - h1;
    const float f1 = ldexpf(1.0f, h1), f2 = ldexpf(1.0f, h2);
    const float y0 = (x0 * f1) * f2;
    const float y1 = (x1 * f1) * f2;
    // Round to nearest even into E4M3FN; |y| <= 448 by construction.
    const int packed = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
    reinterpret_cast<uint16_t*>(code + (size_t)pair * 128)[lane] = (uint16_t)(packed & 0xFFFF);
    if (lane == 0) scale[pair] = ldexpf(1.0f, e);
}

__global__ __launch_bounds__(256) void quantize_q_kernel(const uint16_t* __restrict__ q, int32_t n_pairs,
                                                         uint8_t* __restrict__ code,
                                                         float* __restrict__ scale) {
    const int pair = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (pair >= n_pairs) return;  // whole wavefront leaves together
    quantize_idx_pair(q, pair, threadIdx.x & 63, code, scale);
}

// MLA query of one (row, head): s = 2^ceil(log2(max|q| / 448)) (1 for a zero
// head), hi = RNE_E4M3(q / s), lo = RNE_E4M3(16 (q / s - hi)).  q / s - hi is
// exact in fp32; a bf16 value has 8 significant bits and hi carries the top
// 4, so lo is exact too wherever 16 (q / s - hi) is an E4M3 value (always,
// unless q / s is below E4M3's normal range).  Lane l converts elements
// [8l, 8l + 8) and, for l < 8, [512 + 8l, 512 + 8l + 8).
__device__ __forceinline__ void quantize_mla_pair(const uint16_t* __restrict__ q, int pair, int lane,
                                                  uint8_t* __restrict__ terms, float* __restrict__ scale) {
    constexpr int kD = 576;
    const uint8_t* src = reinterpret_cast<const uint8_t*>(q + (size_t)pair * kD);
    const uint4 c0 = *reinterpret_cast<const uint4*>(src + 16 * lane);
    uint4 c1 = uint4{0u, 0u, 0u, 0u};
    if (lane < 8) c1 = *reinterpret_cast<const uint4*>(src + 16 * (64 + lane));
    const uint32_t w[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    float v[16];
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        v[2 * k] = __uint_as_float(w[k] << 16);
        v[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
        amax = fmaxf(amax, fmaxf(fabsf(v[2 * k]), fabsf(v[2 * k + 1])));
    }
    amax = wave_max(amax);
    float s = 1.0f;
    if (amax > 0.0f) {
        int e;
        const float m = frexpf(amax / 448.0f, &e);   // amax / 448 = m 2^e, m in [0.5, 1)
        s = ldexpf(1.0f, m == 0.5f ? e - 1 : e);      // smallest power of two >= amax / 448
    }
    const float inv = 1.0f / s;                        // exact: s is a power of two
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        float l4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float x = v[4 * k + u] * inv;
            const uint32_t hbyte = __builtin_amdgcn_cvt_pk_fp8_f32(x, 0.0f, 0, false) & 0xFFu;
            l4[u] = 16.0f * (x - __builtin_amdgcn_cvt_f32_fp8(hbyte, 0));
        }
        int hp = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * k] * inv, v[4 * k + 1] * inv, 0, false);
        hp = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * k + 2] * inv, v[4 * k + 3] * inv, hp, true);
        int lp = __builtin_amdgcn_cvt_pk_fp8_f32(l4[0], l4[1], 0, false);
        lp = __builtin_amdgcn_cvt_pk_fp8_f32(l4[2], l4[3], lp, true);
        hw[k] = (uint32_t)hp;
        lw[k] = (uint32_t)lp;
    }
    uint8_t* hi = terms + (size_t)pair * 2 * kD;
    uint8_t* lo = hi + kD;
    *reinterpret_cast<uint2*>(hi + 8 * lane) = uint2{hw[0], hw[1]};
    *reinterpret_cast<uint2*>(lo + 8 * lane) = uint2{lw[0], lw[1]};
    if (lane < 8) {
        *reinterpret_cast<uint2*>(hi + 8 * (64 + lane)) = uint2{hw[2], hw[3]};
        *reinterpret_cast<uint2*>(lo + 8 * (64 + lane)) = uint2{lw[2], lw[3]};
    }
    if (lane == 0) scale[pair] = s;
}

__global__ __launch_bounds__(256) void quantize_mla_q_kernel(const uint16_t* __restrict__ q, int32_t n_pairs,
                                                             uint8_t* __restrict__ terms,
                                                             float* __restrict__ scale) {
    const int pair = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (pair >= n_pairs) return;  // whole wavefront leaves together
    quantize_mla_pair(q, pair, threadIdx.x & 63, terms, scale);
}

// Wavefront w < n_idx prepares indexer pair w, the next n_mla wavefronts the
// MLA pairs.
__global__ __launch_bounds__(256) void prepare_queries_kernel(const uint16_t* __restrict__ q_idx, int32_t n_idx,
                                                              uint8_t* __restrict__ code, float* __restrict__ scale,
                                                              const uint16_t* __restrict__ q_mla, int32_t n_mla,
                                                              uint8_t* __restrict__ terms,
                                                              float* __restrict__ mla_scale) {
    const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (w < n_idx) quantize_idx_pair(q_idx, w, lane, code, scale);
    else if (w - n_idx < n_mla) quantize_mla_pair(q_mla, w - n_idx, lane, terms, mla_scale);
}

hipError_t launch_prepare_queries(const uint16_t* q_idx, int32_t n_idx, uint8_t* code, float* scale,
                                  const uint16_t* q_mla, int32_t n_mla, uint8_t* terms, float* mla_scale,
                                  hipStream_t stream) {
    const int64_t waves = (int64_t)n_idx + n_mla;
    if (waves == 0) return hipSuccess;
    prepare_queries_kernel<<<(int)((waves + 3) / 4), 256, 0, stream>>>(q_idx, n_idx, code, scale, q_mla, n_mla,
                                                                       terms, mla_scale);
    return hipGetLastError();
}

hipError_t launch_quantize_mla_q(const uint16_t* q, int32_t n_pairs, uint8_t* terms, float* scale,
                                 hipStream_t stream) {
    if (n_pairs == 0) return hipSuccess;
    quantize_mla_q_kernel<<<(n_pairs + 3) / 4, 256, 0, stream>>>(q, n_pairs, terms, scale);
    return hipGetLastError();
}

hipError_t launch_quantize_q(const uint16_t* q, int32_t n_pairs, uint8_t* code, float* scale,
                             hipStream_t stream) {
    if (n_pairs == 0) return hipSuccess;
    const int blocks = (n_pairs + 3) / 4;
    quantize_q_kernel<<<blocks, 256, 0, stream>>>(q, n_pairs, code, scale);
    return hipGetLastError();
}

}  // namespace dsa
