// Merge of split-K partials by their natural-log LSE.  The partials are bf16
// (the attention rounds each split's normalised output to nearest even);
// the weights and the sum are fp32.
// One wavefront per (row, head): lane s (< n_splits) reads lse_s, the
// wavefront finds m = max_s lse_s and the weights e^{lse_s - m}; each lane
// then accumulates 8 of the 512 output columns over the splits.  A split of
// weight 0 adds nothing, whatever its partial holds.  From two splits on,
// four (up to four splits) or eight splits' loads are in flight together
// (with bf16 partials that is faster at four splits too: bulk decode's merge
// 4.95 -> 3.74 us, paired); a lone split is read directly.
// With fewer than 1024 (row, head) pairs a pair's columns are split over two
// or four wavefronts (each computing the pair's weights itself), so that a
// launch of few rows and many splits still reads the partials on most of the
// chip (long context, 8 rows x 32 heads x 32 splits: see the launch).
// The partials are read once, with the non-temporal hint: the merge itself
// runs about 0.3 us slower that way, but replayed bulk-decode steps run about
// 4 us faster, all of it in the next step's indexer (kernel traces of the
// replays: 60.8 -> 56.1 us), which the cached reads of the partials slowed.
#include "device_common.h"
#include "launch.h"

namespace dsa {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kDv = 512;

// CPL (8, 4 or 2) consecutive output columns per lane: 512 / (64 CPL)
// wavefronts share one (row, head), so a launch with few pairs still spreads
// over the chip.
template <int CPL>
struct Cols {
    static constexpr int kParts = kDv / (kWave * CPL);   // wavefronts per (row, head)
    float v[CPL];
};

// CPL bf16 columns of a partial at p (16-, 8- or 4-byte aligned), loaded
// with the non-temporal hint and widened to fp32.
template <int CPL>
__device__ __forceinline__ void load_cols(const uint16_t* p, float (&x)[CPL]) {
    uint32_t w[CPL / 2];
    if constexpr (CPL == 8) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else if constexpr (CPL == 4) {
        const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
        w[0] = v.x; w[1] = v.y;
    } else {
        w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
    }
#pragma unroll
    for (int i = 0; i < CPL / 2; ++i) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
}

// The wavefront's (row, head) pair and columns, its split weights and the
// merged LSE; false (after writing the empty result) when no split saw a
// token.
struct MergeHead {
    int rh, lane, ns, col;   // col: the lane's first output column
    float wmine;   // e^{lse_lane - m} on lanes < ns, else 0
    float inv;     // 1 / sum of the weights
    float m, tot;
};

template <int CPL>
__device__ __forceinline__ void store_cols(uint16_t* dst, const float (&acc)[CPL]) {
    uint32_t w[CPL / 2];
#pragma unroll
    for (int i = 0; i < CPL / 2; ++i)
        w[i] = (uint32_t)f32_to_bf16_rne(acc[2 * i]) | ((uint32_t)f32_to_bf16_rne(acc[2 * i + 1]) << 16);
    if constexpr (CPL == 8) *reinterpret_cast<uint4*>(dst) = uint4{w[0], w[1], w[2], w[3]};
    else if constexpr (CPL == 4) *reinterpret_cast<uint2*>(dst) = uint2{w[0], w[1]};
    else *reinterpret_cast<uint32_t*>(dst) = w[0];
}

template <int CPL>
__device__ __forceinline__ bool merge_head(const MergeArgs& a, MergeHead& h) {
    constexpr int kParts = Cols<CPL>::kParts;
    const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
    h.rh = w / kParts;
    if (h.rh >= a.n_rows * a.n_heads) return false;  // whole wavefront leaves together
    h.lane = threadIdx.x & 63;
    h.col = (w % kParts) * kWave * CPL + CPL * h.lane;
    h.ns = a.n_splits;
    const float my = h.lane < h.ns ? a.part_lse[(size_t)h.rh * h.ns + h.lane] : -INFINITY;
    h.m = wave_max(my);
    if (h.m == -INFINITY) {
        // No split saw a token.
        const float zero[CPL] = {};
        store_cols<CPL>(a.out + (size_t)h.rh * kDv + h.col, zero);
        if (a.out_lse != nullptr && h.col == 0) a.out_lse[h.rh] = -INFINITY;
        return false;
    }
    h.wmine = h.lane < h.ns ? __expf(my - h.m) : 0.0f;  // e^{-inf} = 0 for empty splits
    h.tot = wave_sum(h.wmine);
    h.inv = 1.0f / h.tot;
    return true;
}

template <int CPL>
__device__ __forceinline__ void merge_store(const MergeArgs& a, const MergeHead& h, const float (&acc)[CPL]) {
    store_cols<CPL>(a.out + (size_t)h.rh * kDv + h.col, acc);
    if (a.out_lse != nullptr && h.col == 0) a.out_lse[h.rh] = h.m + __logf(h.tot);
}

// One split (or a few): one split's partials at a time, skipped at weight 0.
template <int CPL>
__global__ __launch_bounds__(256) void lse_merge_few_kernel(MergeArgs a) {
    MergeHead h;
    if (!merge_head<CPL>(a, h)) return;
    float acc[CPL] = {};
    const uint16_t* po = a.part_o + (size_t)h.rh * h.ns * kDv + h.col;
    for (int s = 0; s < h.ns; ++s) {
        const float w = __shfl(h.wmine, s) * h.inv;
        if (w == 0.0f) continue;  // uniform across the wavefront
        float x[CPL];
        load_cols<CPL>(po + (size_t)s * kDv, x);
#pragma unroll
        for (int i = 0; i < CPL; ++i) acc[i] += w * x[i];
    }
    merge_store<CPL>(a, h, acc);
}

// More splits: kBatch (4 or 8) splits' loads issued before any is used;
// splits past the end reload the last one and get weight 0.
template <int CPL, int kBatch>
__global__ __launch_bounds__(256) void lse_merge_many_kernel(MergeArgs a) {
    MergeHead h;
    if (!merge_head<CPL>(a, h)) return;
    float acc[CPL] = {};
    const uint16_t* po = a.part_o + (size_t)h.rh * h.ns * kDv + h.col;
    for (int s0 = 0; s0 < h.ns; s0 += kBatch) {
        float x[kBatch][CPL];
#pragma unroll
        for (int b = 0; b < kBatch; ++b) load_cols<CPL>(po + (size_t)min(s0 + b, h.ns - 1) * kDv, x[b]);
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            const float w = s0 + b < h.ns ? __shfl(h.wmine, min(s0 + b, h.ns - 1)) * h.inv : 0.0f;
            const bool use = w != 0.0f;
#pragma unroll
            for (int i = 0; i < CPL; ++i) acc[i] += use ? w * x[b][i] : 0.0f;
        }
    }
    merge_store<CPL>(a, h, acc);
}

template <int CPL>
hipError_t launch_cpl(const MergeArgs& a, hipStream_t stream) {
    const int64_t waves = (int64_t)a.n_rows * a.n_heads * Cols<CPL>::kParts;
    const unsigned wgs = (unsigned)((waves + 3) / 4);
    if (a.n_splits == 1) lse_merge_few_kernel<CPL><<<wgs, 256, 0, stream>>>(a);
    else if (a.n_splits <= 4) lse_merge_many_kernel<CPL, 4><<<wgs, 256, 0, stream>>>(a);
    else lse_merge_many_kernel<CPL, 8><<<wgs, 256, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_lse_merge(const MergeArgs& a, hipStream_t stream) {
    const int pairs = a.n_rows * a.n_heads;
    if (pairs == 0) return hipSuccess;
    // Enough wavefronts to cover the chip: whole (row, head) pairs when there
    // are many, else each pair split over two or four wavefronts.
    if (pairs >= 1024) return launch_cpl<8>(a, stream);
    if (pairs >= 512) return launch_cpl<4>(a, stream);
    return launch_cpl<2>(a, stream);
}

}  // namespace dsa
