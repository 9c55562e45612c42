// Merge of split-K partials by their natural-log LSE.
// One wavefront per (row, head): lane s (< n_splits) reads lse_s, the
// wavefront finds m = max_s lse_s and the weights e^{lse_s - m}; each lane
// then accumulates 8 of the 512 output columns over the splits.  A split of
// weight 0 adds nothing, whatever its partial holds.  Up to four splits the
// partials are read one split at a time; above four, eight splits' loads
// are in flight together (each measured the faster at its split counts).
// The partials are read once, with the non-temporal hint: the merge itself
// runs about 0.3 us slower that way, but replayed bulk-decode steps run about
// 4 us faster, all of it in the next step's indexer (kernel traces of the
// replays: 60.8 -> 56.1 us), which the cached reads of the partials slowed.
#include "device_common.h"
#include "launch.h"

namespace dsa {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// 16 bytes of a partial, loaded with the non-temporal hint.
__device__ __forceinline__ float4 load_partial(const float* p) {
    const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    return float4{v.x, v.y, v.z, v.w};
}

constexpr int kDv = 512;
constexpr int kBatch = 8;   // splits whose partials are in flight together (many-split kernel)

// The (row, head) pair of this wavefront, its split weights and the merged
// LSE; false (after writing the empty result) when no split saw a token.
struct MergeHead {
    int rh, lane, ns;
    float wmine;   // e^{lse_lane - m} on lanes < ns, else 0
    float inv;     // 1 / sum of the weights
    float m, tot;
};

__device__ __forceinline__ bool merge_head(const MergeArgs& a, MergeHead& h) {
    h.rh = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (h.rh >= a.n_rows * a.n_heads) return false;  // whole wavefront leaves together
    h.lane = threadIdx.x & 63;
    h.ns = a.n_splits;
    const float my = h.lane < h.ns ? a.part_lse[(size_t)h.rh * h.ns + h.lane] : -INFINITY;
    h.m = wave_max(my);
    if (h.m == -INFINITY) {
        // No split saw a token.
        reinterpret_cast<uint4*>(a.out + (size_t)h.rh * kDv + 8 * h.lane)[0] = uint4{0u, 0u, 0u, 0u};
        if (a.out_lse != nullptr && h.lane == 0) a.out_lse[h.rh] = -INFINITY;
        return false;
    }
    h.wmine = h.lane < h.ns ? __expf(my - h.m) : 0.0f;  // e^{-inf} = 0 for empty splits
    h.tot = wave_sum(h.wmine);
    h.inv = 1.0f / h.tot;
    return true;
}

__device__ __forceinline__ void merge_store(const MergeArgs& a, const MergeHead& h, const float (&acc)[8]) {
    uint4 o;
    o.x = (uint32_t)f32_to_bf16_rne(acc[0]) | ((uint32_t)f32_to_bf16_rne(acc[1]) << 16);
    o.y = (uint32_t)f32_to_bf16_rne(acc[2]) | ((uint32_t)f32_to_bf16_rne(acc[3]) << 16);
    o.z = (uint32_t)f32_to_bf16_rne(acc[4]) | ((uint32_t)f32_to_bf16_rne(acc[5]) << 16);
    o.w = (uint32_t)f32_to_bf16_rne(acc[6]) | ((uint32_t)f32_to_bf16_rne(acc[7]) << 16);
    reinterpret_cast<uint4*>(a.out + (size_t)h.rh * kDv + 8 * h.lane)[0] = o;
    if (a.out_lse != nullptr && h.lane == 0) a.out_lse[h.rh] = h.m + __logf(h.tot);
}

// Up to four splits: one split's partials at a time, skipped at weight 0.
__global__ __launch_bounds__(256) void lse_merge_few_kernel(MergeArgs a) {
    MergeHead h;
    if (!merge_head(a, h)) return;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const float* po = a.part_o + (size_t)h.rh * h.ns * kDv + 8 * h.lane;
    for (int s = 0; s < h.ns; ++s) {
        const float w = __shfl(h.wmine, s) * h.inv;
        if (w == 0.0f) continue;  // uniform across the wavefront
        const float4 x0 = load_partial(po + (size_t)s * kDv);
        const float4 x1 = load_partial(po + (size_t)s * kDv + 4);
        acc[0] += w * x0.x; acc[1] += w * x0.y; acc[2] += w * x0.z; acc[3] += w * x0.w;
        acc[4] += w * x1.x; acc[5] += w * x1.y; acc[6] += w * x1.z; acc[7] += w * x1.w;
    }
    merge_store(a, h, acc);
}

// More splits: kBatch splits' loads issued before any is used; splits past
// the end reload the last one and get weight 0.
__global__ __launch_bounds__(256) void lse_merge_many_kernel(MergeArgs a) {
    MergeHead h;
    if (!merge_head(a, h)) return;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const float* po = a.part_o + (size_t)h.rh * h.ns * kDv + 8 * h.lane;
    for (int s0 = 0; s0 < h.ns; s0 += kBatch) {
        float4 x[kBatch][2];
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            const float* p = po + (size_t)min(s0 + b, h.ns - 1) * kDv;
            x[b][0] = load_partial(p);
            x[b][1] = load_partial(p + 4);
        }
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            const float w = s0 + b < h.ns ? __shfl(h.wmine, min(s0 + b, h.ns - 1)) * h.inv : 0.0f;
            const bool use = w != 0.0f;
            acc[0] += use ? w * x[b][0].x : 0.0f; acc[1] += use ? w * x[b][0].y : 0.0f;
            acc[2] += use ? w * x[b][0].z : 0.0f; acc[3] += use ? w * x[b][0].w : 0.0f;
            acc[4] += use ? w * x[b][1].x : 0.0f; acc[5] += use ? w * x[b][1].y : 0.0f;
            acc[6] += use ? w * x[b][1].z : 0.0f; acc[7] += use ? w * x[b][1].w : 0.0f;
        }
    }
    merge_store(a, h, acc);
}

}  // namespace

hipError_t launch_lse_merge(const MergeArgs& a, hipStream_t stream) {
    const int pairs = a.n_rows * a.n_heads;
    if (pairs == 0) return hipSuccess;
    if (a.n_splits <= 4) lse_merge_few_kernel<<<(pairs + 3) / 4, 256, 0, stream>>>(a);
    else lse_merge_many_kernel<<<(pairs + 3) / 4, 256, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace dsa
