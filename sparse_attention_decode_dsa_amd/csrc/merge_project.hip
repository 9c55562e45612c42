// LSE merge followed by the value projection W_UV (page "[ROCm] Support
// decode context parallel (DCP) for GLM-5 / DeepSeek-V3.2", Future work:
// projecting V before the LSE merge).  The projection is linear and the
// merge is a weighted sum whose weights add to one, so merging first and
// projecting once gives the same result as projecting every split.
//
// A workgroup (4 wavefronts) owns 8 rows of one head (one workgroup per
// compute unit at bulk decode; 4 and 16 rows measured slower).
//   merge:   wavefront w merges rows 2w and 2w+1: lane s reads lse_s of both,
//            wave max and sum give the weights, and each lane accumulates 8
//            latent columns over the (row, split) pairs, eight pairs'
//            partials in flight at a time; the first eight go out
//            together with the LSEs and the weights (one memory round trip
//            for up to four splits).  The merged latent goes to LDS in bf16
//            (round to nearest even), rows 520 entries apart so that a
//            matrix-core read of 16 rows falls on distinct banks; the tile's
//            other rows are zero;
//   project: D[16 rows x Dv] = A[16 x 512] x B[512 x Dv] on bf16 matrix cores
//            (v_mfma_f32_16x16x32_bf16), A from LDS, B = head h's weights
//            [Dv, 512] (16 contiguous bytes per lane and K step, shared
//            through L2 by the head's row blocks, all loaded at entry so that
//            they arrive during the merge); wavefront w produces output
//            columns [32w, 32w + 32).
#include "device_common.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kLatent = 512;
constexpr int kDvOut = 128;
constexpr int kRowsPerWg = 8;    // rows merged per workgroup (the tile has 16)
constexpr int kRpw = kRowsPerWg / 4;   // rows merged per wavefront
constexpr int kTileRows = 16;
constexpr int kAStride = kLatent + 8;   // bf16 entries per LDS row
constexpr int kPairs = 8;        // (row, split) partials in flight per wavefront

__global__ __launch_bounds__(256) void merge_project_kernel(MergeProjectArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t s_a[kTileRows * kAStride];
    // Grid x is the head: workgroups are dealt to the XCDs round-robin in
    // dispatch order, so head h always lands on XCD h % 8 and each XCD's L2
    // fetches the weights of its heads once for all their row blocks.
    const int h = blockIdx.x;
    const int r0 = blockIdx.y * kRowsPerWg;
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int ns = a.n_splits;

    // The tile's rows past the merged ones are zero.
    for (int i = threadIdx.x; i < (kTileRows - kRowsPerWg) * kAStride / 8; i += 256)
        reinterpret_cast<uint4*>(s_a + kRowsPerWg * kAStride)[i] = uint4{0u, 0u, 0u, 0u};

    // This wavefront's rows (a row past the batch reads the last row and
    // gets weight 0).
    int rh[kRpw];
    bool live[kRpw];
    float wmine[kRpw], inv[kRpw], m[kRpw], tot[kRpw];
#pragma unroll
    for (int j = 0; j < kRpw; ++j) {
        const int row = r0 + kRpw * wv + j;
        live[j] = row < a.n_rows;
        rh[j] = min(row, a.n_rows - 1) * a.n_heads + h;
    }
    float my[kRpw];
#pragma unroll
    for (int j = 0; j < kRpw; ++j) my[j] = live[j] && lane < ns ? a.part_lse[(size_t)rh[j] * ns + lane] : -INFINITY;
    // The partials of (row, split) pairs [p0, p0 + kPairs) into x.
    const int np = kRpw * ns;
    float4 x[kPairs][2];
    auto load_pairs = [&](int p0) {
#pragma unroll
        for (int b = 0; b < kPairs; ++b) {
            const int p = min(p0 + b, np - 1);
            const int j = p / ns;
            const uint16_t* src = a.part_o + ((size_t)rh[j] * ns + (p - j * ns)) * kLatent + 8 * lane;
            const uint4 u = *reinterpret_cast<const uint4*>(src);   // 8 bf16 partials
            x[b][0] = float4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                             __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u)};
            x[b][1] = float4{__uint_as_float(u.z << 16), __uint_as_float(u.z & 0xFFFF0000u),
                             __uint_as_float(u.w << 16), __uint_as_float(u.w & 0xFFFF0000u)};
        }
    };
    // The first pairs go out with the LSEs, before their weights are known.
    load_pairs(0);
    // Head h's weights for this lane, all loaded now (they depend on
    // nothing).  Loads complete in order, so the LSEs go first, then the
    // partials, then the weights: each wait leaves the later loads in
    // flight.  B column 32 wv + n (and + 16), K entries [32 ks + 8 g, +8)
    // for every K step.
    const int n = lane & 15;
    const int g = lane >> 4;
    constexpr int kSteps = kLatent / 32;
    v8bf bw[2][kSteps];
    {
        const uint16_t* wcol0 = a.w_uv + ((size_t)h * kDvOut + 32 * wv + n) * kLatent + 8 * g;
#pragma unroll
        for (int ks = 0; ks < kSteps; ++ks) {
            bw[0][ks] = *reinterpret_cast<const v8bf*>(wcol0 + 32 * ks);
            bw[1][ks] = *reinterpret_cast<const v8bf*>(wcol0 + 16 * kLatent + 32 * ks);
        }
    }
    // Keep the scheduler from sinking these loads below the reductions:
    // LSEs, first partials and weights are then in flight together.
    __builtin_amdgcn_sched_barrier(0);

#pragma unroll
    for (int j = 0; j < kRpw; ++j) {
        m[j] = wave_max(my[j]);
        wmine[j] = m[j] != -INFINITY && lane < ns ? __expf(my[j] - m[j]) : 0.0f;   // 0 for empty splits
        tot[j] = wave_sum(wmine[j]);
        inv[j] = tot[j] > 0.0f ? 1.0f / tot[j] : 0.0f;
    }
    float acc[kRpw][8];
#pragma unroll
    for (int j = 0; j < kRpw; ++j)
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[j][k] = 0.0f;
    // Pairs p = j * ns + s, kPairs at a time; pairs past the end reload the
    // last one and get weight 0.  A split of weight 0 adds nothing, whatever
    // its partial holds.
    for (int p0 = kPairs; ; p0 += kPairs) {
#pragma unroll
        for (int b = 0; b < kPairs; ++b) {
            const int p = p0 - kPairs + b;
            const int j = min(p / ns, kRpw - 1);
            const int sidx = min(p - j * ns, ns - 1);
            float wsel = wmine[0], isel = inv[0];
#pragma unroll
            for (int jj = 1; jj < kRpw; ++jj)
                if (jj == j) { wsel = wmine[jj]; isel = inv[jj]; }
            const float wj = __shfl(wsel, sidx) * isel;
            const float w = p < np ? wj : 0.0f;
            const bool use = w != 0.0f;
#pragma unroll
            for (int jj = 0; jj < kRpw; ++jj) {
                const bool u = use && jj == j;
                acc[jj][0] += u ? w * x[b][0].x : 0.0f; acc[jj][1] += u ? w * x[b][0].y : 0.0f;
                acc[jj][2] += u ? w * x[b][0].z : 0.0f; acc[jj][3] += u ? w * x[b][0].w : 0.0f;
                acc[jj][4] += u ? w * x[b][1].x : 0.0f; acc[jj][5] += u ? w * x[b][1].y : 0.0f;
                acc[jj][6] += u ? w * x[b][1].z : 0.0f; acc[jj][7] += u ? w * x[b][1].w : 0.0f;
            }
        }
        if (p0 >= np) break;
        load_pairs(p0);
    }
#pragma unroll
    for (int j = 0; j < kRpw; ++j) {
        const int lr = kRpw * wv + j;
        if (live[j] && a.out_lse != nullptr && lane == 0)
            a.out_lse[rh[j]] = m[j] == -INFINITY ? -INFINITY : m[j] + __logf(tot[j]);
        uint4 o;
        o.x = (uint32_t)f32_to_bf16_rne(acc[j][0]) | ((uint32_t)f32_to_bf16_rne(acc[j][1]) << 16);
        o.y = (uint32_t)f32_to_bf16_rne(acc[j][2]) | ((uint32_t)f32_to_bf16_rne(acc[j][3]) << 16);
        o.z = (uint32_t)f32_to_bf16_rne(acc[j][4]) | ((uint32_t)f32_to_bf16_rne(acc[j][5]) << 16);
        o.w = (uint32_t)f32_to_bf16_rne(acc[j][6]) | ((uint32_t)f32_to_bf16_rne(acc[j][7]) << 16);
        *reinterpret_cast<uint4*>(s_a + lr * kAStride + 8 * lane) = o;
    }
    __syncthreads();

    // Projection: lane (n, g) reads A row n and B column n, K entries
    // [32 ks + 8 g, 32 ks + 8 g + 8); accumulator entry i is row 4g + i.
    const uint16_t* arow = s_a + n * kAStride + 8 * g;
    v4f acc0 = v4f{0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
#pragma unroll
    for (int ks = 0; ks < kSteps; ++ks) {
        const v8bf av = *reinterpret_cast<const v8bf*>(arow + 32 * ks);
        acc0 = mfma_bf16_16x16x32(av, bw[0][ks], acc0);
        acc1 = mfma_bf16_16x16x32(av, bw[1][ks], acc1);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int lr = 4 * g + i;
        const int row = r0 + lr;
        if (lr < kRowsPerWg && row < a.n_rows) {
            uint16_t* dst = a.out + ((size_t)row * a.n_heads + h) * kDvOut + 32 * wv + n;
            dst[0] = f32_to_bf16_rne(acc0[i]);
            dst[16] = f32_to_bf16_rne(acc1[i]);
        }
    }
}

}  // namespace

hipError_t launch_merge_project(const MergeProjectArgs& a, hipStream_t stream) {
    if (a.n_rows == 0) return hipSuccess;
    merge_project_kernel<<<dim3(a.n_heads, (a.n_rows + kRowsPerWg - 1) / kRowsPerWg), 256, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace dsa
