// LSE merge followed by the value projection W_UV (page "[ROCm] Support
// decode context parallel (DCP) for GLM-5 / DeepSeek-V3.2", Future work:
// projecting V before the LSE merge).  The projection is linear and the
// merge is a weighted sum whose weights add to one, so merging first and
// projecting once gives the same result as projecting every split.
//
// A workgroup (4 wavefronts) owns 16 rows of one head.
//   merge:   wavefront w merges rows 4w..4w+3 as the LSE merge does (lane s
//            reads lse_s; wave max and sum give the weights; each lane
//            accumulates 8 latent columns over the splits) and writes the
//            merged latent in bf16 (round to nearest even) to LDS, rows 520
//            entries apart so that the 16 rows of a matrix-core read fall on
//            distinct banks;
//   project: D[16 rows x Dv] = A[16 x 512] x B[512 x Dv] on bf16 matrix cores
//            (v_mfma_f32_16x16x32_bf16), A from LDS, B = head h's weights
//            [Dv, 512] (16 contiguous bytes per lane and K step, shared
//            through L2 by the head's row blocks); wavefront w produces
//            output columns [32w, 32w + 32).
#include "device_common.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kLatent = 512;
constexpr int kDvOut = 128;
constexpr int kRowsPerWg = 16;
constexpr int kAStride = kLatent + 8;   // bf16 entries per LDS row

__global__ __launch_bounds__(256) void merge_project_kernel(MergeProjectArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t s_a[kRowsPerWg * kAStride];
    const int h = blockIdx.y;
    const int r0 = blockIdx.x * kRowsPerWg;
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int ns = a.n_splits;

    // Merge rows r0 + 4 wv + i into LDS (zeros for rows past the batch and
    // rows no split saw).
#pragma unroll 1
    for (int i = 0; i < 4; ++i) {
        const int lr = 4 * wv + i;
        const int row = r0 + lr;
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (row < a.n_rows) {
            const size_t rh = (size_t)row * a.n_heads + h;
            const float my = lane < ns ? a.part_lse[rh * ns + lane] : -INFINITY;
            const float m = wave_max(my);
            if (m == -INFINITY) {
                if (a.out_lse != nullptr && lane == 0) a.out_lse[rh] = -INFINITY;
            } else {
                const float wmine = lane < ns ? __expf(my - m) : 0.0f;
                const float tot = wave_sum(wmine);
                const float inv = 1.0f / tot;
                const float* po = a.part_o + rh * ns * kLatent + 8 * lane;
                for (int s = 0; s < ns; ++s) {
                    const float w = __shfl(wmine, s) * inv;
                    if (w == 0.0f) continue;  // uniform across the wavefront
                    const float4 x0 = reinterpret_cast<const float4*>(po + (size_t)s * kLatent)[0];
                    const float4 x1 = reinterpret_cast<const float4*>(po + (size_t)s * kLatent)[1];
                    acc[0] += w * x0.x; acc[1] += w * x0.y; acc[2] += w * x0.z; acc[3] += w * x0.w;
                    acc[4] += w * x1.x; acc[5] += w * x1.y; acc[6] += w * x1.z; acc[7] += w * x1.w;
                }
                if (a.out_lse != nullptr && lane == 0) a.out_lse[rh] = m + __logf(tot);
            }
        }
        uint4 o;
        o.x = (uint32_t)f32_to_bf16_rne(acc[0]) | ((uint32_t)f32_to_bf16_rne(acc[1]) << 16);
        o.y = (uint32_t)f32_to_bf16_rne(acc[2]) | ((uint32_t)f32_to_bf16_rne(acc[3]) << 16);
        o.z = (uint32_t)f32_to_bf16_rne(acc[4]) | ((uint32_t)f32_to_bf16_rne(acc[5]) << 16);
        o.w = (uint32_t)f32_to_bf16_rne(acc[6]) | ((uint32_t)f32_to_bf16_rne(acc[7]) << 16);
        *reinterpret_cast<uint4*>(s_a + lr * kAStride + 8 * lane) = o;
    }
    __syncthreads();

    // Projection: lane (n, g) reads A row n and B column n, K entries
    // [32 ks + 8 g, 32 ks + 8 g + 8); accumulator entry i is row 4g + i.
    const int n = lane & 15;
    const int g = lane >> 4;
    const uint16_t* arow = s_a + n * kAStride + 8 * g;
    const uint16_t* wcol0 = a.w_uv + ((size_t)h * kDvOut + 32 * wv + n) * kLatent + 8 * g;
    const uint16_t* wcol1 = wcol0 + 16 * kLatent;
    v4f acc0 = v4f{0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
#pragma unroll 4
    for (int ks = 0; ks < kLatent / 32; ++ks) {
        const v8bf av = *reinterpret_cast<const v8bf*>(arow + 32 * ks);
        const v8bf b0 = *reinterpret_cast<const v8bf*>(wcol0 + 32 * ks);
        const v8bf b1 = *reinterpret_cast<const v8bf*>(wcol1 + 32 * ks);
        acc0 = mfma_bf16_16x16x32(av, b0, acc0);
        acc1 = mfma_bf16_16x16x32(av, b1, acc1);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = r0 + 4 * g + i;
        if (row < a.n_rows) {
            uint16_t* dst = a.out + ((size_t)row * a.n_heads + h) * kDvOut + 32 * wv + n;
            dst[0] = f32_to_bf16_rne(acc0[i]);
            dst[16] = f32_to_bf16_rne(acc1[i]);
        }
    }
}

}  // namespace

hipError_t launch_merge_project(const MergeProjectArgs& a, hipStream_t stream) {
    if (a.n_rows == 0) return hipSuccess;
    merge_project_kernel<<<dim3((a.n_rows + kRowsPerWg - 1) / kRowsPerWg, a.n_heads), 256, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace dsa
