// Indexer query quantization on its own, one wavefront per (row, head):
// 128 bf16 -> fp8 E4M3FN codes with one power-of-two scale.  The indexer
// quantizes its queries with the same helpers (query_quant.h).
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

hipError_t launch_quantize_q(const uint16_t* q, int32_t n_pairs, uint8_t* code, float* scale,
                             hipStream_t stream) {
    if (n_pairs == 0) return hipSuccess;
    const int blocks = (n_pairs + 3) / 4;
    quantize_q_kernel<<<blocks, 256, 0, stream>>>(q, n_pairs, code, scale);
    return hipGetLastError();
}

}  // namespace dsa
