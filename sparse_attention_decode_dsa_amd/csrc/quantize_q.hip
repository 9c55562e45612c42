// Query preparation, one wavefront per (row, head):
//   - indexer queries (128 bf16) -> fp8 E4M3FN codes, one power-of-two scale;
//   - MLA queries (576 bf16) -> two fp8 E4M3FN terms and one power-of-two
//     scale s, q = s (hi + lo / 16), read by the sparse MLA kernel's fp8
//     QK products.
// The indexer and the sparse MLA kernel quantize their own queries with the
// same helpers (query_quant.h); these kernels expose that step on its own.
#include "device_common.h"
#include "launch.h"
#include "query_quant.h"

namespace dsa {

__device__ __forceinline__ void quantize_idx_pair(const uint16_t* __restrict__ q, int pair, int lane,
                                                  uint8_t* __restrict__ code, float* __restrict__ scale) {
    const uint32_t w = reinterpret_cast<const uint32_t*>(q + (size_t)pair * 128)[lane];
    const float x0 = __uint_as_float(w << 16);
    const float x1 = __uint_as_float(w & 0xFFFF0000u);
    const int e = idx_q_exponent(wave_max(fmaxf(fabsf(x0), fabsf(x1))));
    reinterpret_cast<uint16_t*>(code + (size_t)pair * 128)[lane] = (uint16_t)idx_q_code2(x0, x1, idx_q_factors(e));
    if (lane == 0) scale[pair] = ldexpf(1.0f, e);
}

__global__ __launch_bounds__(256) void quantize_q_kernel(const uint16_t* __restrict__ q, int32_t n_pairs,
                                                         uint8_t* __restrict__ code,
                                                         float* __restrict__ scale) {
    const int pair = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (pair >= n_pairs) return;  // whole wavefront leaves together
    quantize_idx_pair(q, pair, threadIdx.x & 63, code, scale);
}

// MLA query of one (row, head) (mla_q_scale, mla_q_split4).  Lane l converts
// elements [8l, 8l + 8) and, for l < 8, [512 + 8l, 512 + 8l + 8).
__device__ __forceinline__ void quantize_mla_pair(const uint16_t* __restrict__ q, int pair, int lane,
                                                  uint8_t* __restrict__ terms, float* __restrict__ scale) {
    constexpr int kD = 576;
    const uint8_t* src = reinterpret_cast<const uint8_t*>(q + (size_t)pair * kD);
    const uint4 c0 = *reinterpret_cast<const uint4*>(src + 16 * lane);
    uint4 c1 = uint4{0u, 0u, 0u, 0u};
    if (lane < 8) c1 = *reinterpret_cast<const uint4*>(src + 16 * (64 + lane));
    float v0[8], v1[8];
    bf16x8_to_f32(c0, v0);
    bf16x8_to_f32(c1, v1);
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fmaxf(fabsf(v0[k]), fabsf(v1[k])));
    const float s = mla_q_scale(wave_max(amax));
    const float inv = 1.0f / s;                        // exact: s is a power of two
    uint32_t hw[4], lw[4];
    mla_q_split4(v0[0] * inv, v0[1] * inv, v0[2] * inv, v0[3] * inv, hw[0], lw[0]);
    mla_q_split4(v0[4] * inv, v0[5] * inv, v0[6] * inv, v0[7] * inv, hw[1], lw[1]);
    mla_q_split4(v1[0] * inv, v1[1] * inv, v1[2] * inv, v1[3] * inv, hw[2], lw[2]);
    mla_q_split4(v1[4] * inv, v1[5] * inv, v1[6] * inv, v1[7] * inv, hw[3], lw[3]);
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
