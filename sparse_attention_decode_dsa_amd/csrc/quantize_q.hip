// bf16 indexer queries -> fp8 E4M3FN codes with one power-of-two scale per
// (row, head).  One wavefront per (row, head): 128 values, two per lane.
#include "device_common.h"
#include "launch.h"

namespace dsa {

__global__ __launch_bounds__(256) void quantize_q_kernel(const uint16_t* __restrict__ q, int32_t n_pairs,
                                                         uint8_t* __restrict__ code,
                                                         float* __restrict__ scale) {
    const int pair = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (pair >= n_pairs) return;  // whole wavefront leaves together
    const int lane = threadIdx.x & 63;
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

hipError_t launch_quantize_q(const uint16_t* q, int32_t n_pairs, uint8_t* code, float* scale,
                             hipStream_t stream) {
    if (n_pairs == 0) return hipSuccess;
    const int blocks = (n_pairs + 3) / 4;
    quantize_q_kernel<<<blocks, 256, 0, stream>>>(q, n_pairs, code, scale);
    return hipGetLastError();
}

}  // namespace dsa
