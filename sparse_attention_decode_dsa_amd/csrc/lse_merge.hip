// Merge of split-K partials by their natural-log LSE.
// One wavefront per (row, head): lane s (< n_splits) reads lse_s, the
// wavefront finds m = max_s lse_s and the weights e^{lse_s - m}; each lane
// then accumulates 8 of the 512 output columns over the splits.
#include "device_common.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kDv = 512;

__global__ __launch_bounds__(256) void lse_merge_kernel(MergeArgs a) {
    const int rh = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (rh >= a.n_rows * a.n_heads) return;  // whole wavefront leaves together
    const int lane = threadIdx.x & 63;
    const int ns = a.n_splits;
    const float* lse_p = a.part_lse + (size_t)rh * ns;
    const float my = lane < ns ? lse_p[lane] : -INFINITY;
    const float m = wave_max(my);
    float* lse_out = a.out_lse;
    uint16_t* dst = a.out + (size_t)rh * kDv + 8 * lane;
    if (m == -INFINITY) {
        // No split saw a token.
        reinterpret_cast<uint4*>(dst)[0] = uint4{0u, 0u, 0u, 0u};
        if (lse_out != nullptr && lane == 0) lse_out[rh] = -INFINITY;
        return;
    }
    const float wmine = lane < ns ? __expf(my - m) : 0.0f;  // e^{-inf} = 0 for empty splits
    const float tot = wave_sum(wmine);
    const float inv = 1.0f / tot;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const float* po = a.part_o + (size_t)rh * ns * kDv + 8 * lane;
    for (int s = 0; s < ns; ++s) {
        const float w = __shfl(wmine, s) * inv;
        if (w == 0.0f) continue;  // uniform across the wavefront
        const float4 x0 = reinterpret_cast<const float4*>(po + (size_t)s * kDv)[0];
        const float4 x1 = reinterpret_cast<const float4*>(po + (size_t)s * kDv)[1];
        acc[0] += w * x0.x; acc[1] += w * x0.y; acc[2] += w * x0.z; acc[3] += w * x0.w;
        acc[4] += w * x1.x; acc[5] += w * x1.y; acc[6] += w * x1.z; acc[7] += w * x1.w;
    }
    uint4 o;
    o.x = (uint32_t)f32_to_bf16_rne(acc[0]) | ((uint32_t)f32_to_bf16_rne(acc[1]) << 16);
    o.y = (uint32_t)f32_to_bf16_rne(acc[2]) | ((uint32_t)f32_to_bf16_rne(acc[3]) << 16);
    o.z = (uint32_t)f32_to_bf16_rne(acc[4]) | ((uint32_t)f32_to_bf16_rne(acc[5]) << 16);
    o.w = (uint32_t)f32_to_bf16_rne(acc[6]) | ((uint32_t)f32_to_bf16_rne(acc[7]) << 16);
    reinterpret_cast<uint4*>(dst)[0] = o;
    if (lse_out != nullptr && lane == 0) lse_out[rh] = m + __logf(tot);
}

}  // namespace

hipError_t launch_lse_merge(const MergeArgs& a, hipStream_t stream) {
    const int pairs = a.n_rows * a.n_heads;
    if (pairs == 0) return hipSuccess;
    lse_merge_kernel<<<(pairs + 3) / 4, 256, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace dsa
