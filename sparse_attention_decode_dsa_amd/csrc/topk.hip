// Exact top-k under (score descending, slot ascending), per split then merged.
//
// One 1024-thread workgroup selects from one list of at most 32768 fp32
// scores held in LDS as order-preserving uint32 keys:
//   1. radix select: four 8-bit passes from the most significant digit, each
//      a histogram of the keys that still match the chosen prefix (one
//      256-bin histogram per wavefront, then summed), find the k-th largest
//      key `thr` and how many keys equal to it are still needed;
//   2. ordered emission: each wavefront owns a contiguous range of list
//      positions and walks it 64 at a time; ballots give every selected
//      position its rank, so the output comes out in list order.  Keys above
//      `thr` are taken; keys equal to `thr` are taken in list order until
//      the count is reached, which keeps the lowest slots among ties.
// Lists are always in ascending slot order, so list order is slot order:
//   - direct (one split): the row's scores [0, row_vis);
//   - split pass: one contiguous slot range of the row -> candidate keys and
//     slots in a workspace;
//   - merge pass: the concatenated candidates of the row's splits, in split
//     order.
// Local top-k per split followed by an exact merge equals the global top-k
// because every member of the global top-k is in its own split's top-k.
#include "device_common.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;

struct TopkSmem {
    uint32_t keys[kTopkMaxList];
    uint32_t hist[kWaves][256];
    uint32_t scan[kWaves + 1];
    uint32_t wave_cnt[kWaves];
    int32_t offs[kMaxSplits + 1];
    uint32_t sel_digit;
    uint32_t sel_need;
    int32_t n;
};

// k-th largest key of s.keys[0, n) (1 <= k <= n) and the number of keys equal
// to it that belong to the top k.
__device__ void radix_select(TopkSmem& s, int n, int k, uint32_t* thr_out, int* need_out) {
    const int tid = threadIdx.x;
    const int wv = tid >> 6;
    uint32_t prefix = 0, mask = 0;
    uint32_t kk = (uint32_t)k;
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        uint32_t* hflat = &s.hist[0][0];
        for (int i = tid; i < kWaves * 256; i += kThreads) hflat[i] = 0;
        __syncthreads();
        for (int i = tid; i < n; i += kThreads) {
            const uint32_t key = s.keys[i];
            if ((key & mask) == prefix) atomicAdd(&s.hist[wv][(key >> shift) & 255u], 1u);
        }
        __syncthreads();
        // Thread t (< 256) owns digit 255 - t, so an exclusive scan counts
        // the keys with a larger digit.
        uint32_t c = 0;
        if (tid < 256) {
#pragma unroll
            for (int w = 0; w < kWaves; ++w) c += s.hist[w][255 - tid];
        }
        uint32_t total;
        const uint32_t above = block_exclusive_scan<kThreads>(tid < 256 ? c : 0u, s.scan, &total);
        if (tid < 256 && above < kk && above + c >= kk) {
            s.sel_digit = 255u - tid;
            s.sel_need = kk - above;
        }
        __syncthreads();
        prefix |= s.sel_digit << shift;
        mask |= 255u << shift;
        kk = s.sel_need;
        __syncthreads();
    }
    *thr_out = prefix;
    *need_out = (int)kk;
}

// Emit the selected positions of s.keys[0, n) in list order: emit(rank, pos).
template <typename Emit>
__device__ void ordered_emit(TopkSmem& s, int n, uint32_t thr, int need_eq, Emit emit) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int per_wave = ((n + kWaves - 1) / kWaves + 63) & ~63;
    const int beg = min(n, wv * per_wave);
    const int end = min(n, beg + per_wave);
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

    // Pass 1: keys equal to thr in each wavefront's range.
    uint32_t eq = 0;
    for (int base = beg; base < end; base += 64) {
        const int i = base + lane;
        const bool e = i < end && s.keys[i] == thr;
        eq += __popcll(__ballot(e));
    }
    uint32_t tot;
    // Lane 0 of each wavefront contributes its count; others contribute 0.
    const uint32_t eq_before = block_exclusive_scan<kThreads>(lane == 0 ? eq : 0u, s.scan, &tot);
    const uint32_t eq_base0 = __shfl(eq_before, 0);
    // Selected count per wavefront.
    uint32_t sel_cnt = 0;
    {
        uint32_t eq_seen = eq_base0;
        for (int base = beg; base < end; base += 64) {
            const int i = base + lane;
            const uint32_t key = i < end ? s.keys[i] : 0u;
            const bool gt = i < end && key > thr;
            const bool e = i < end && key == thr;
            const uint64_t em = __ballot(e);
            const uint32_t my_eq = eq_seen + __popcll(em & lt);
            const bool take = gt || (e && my_eq < (uint32_t)need_eq);
            sel_cnt += __popcll(__ballot(take));
            eq_seen += __popcll(em);
        }
    }
    const uint32_t sel_before = block_exclusive_scan<kThreads>(lane == 0 ? sel_cnt : 0u, s.scan, &tot);
    uint32_t out_base = __shfl(sel_before, 0);
    uint32_t eq_seen = eq_base0;
    for (int base = beg; base < end; base += 64) {
        const int i = base + lane;
        const uint32_t key = i < end ? s.keys[i] : 0u;
        const bool gt = i < end && key > thr;
        const bool e = i < end && key == thr;
        const uint64_t em = __ballot(e);
        const uint32_t my_eq = eq_seen + __popcll(em & lt);
        const bool take = gt || (e && my_eq < (uint32_t)need_eq);
        const uint64_t tm = __ballot(take);
        if (take) emit((int)(out_base + __popcll(tm & lt)), i);
        out_base += __popcll(tm);
        eq_seen += __popcll(em);
    }
}

// Load scores[lo, hi) of a row as keys, flagging NaNs.
__device__ void load_keys(TopkSmem& s, const float* src, int n, int32_t* status) {
    bool nan = false;
    for (int i = threadIdx.x; i < n; i += kThreads) {
        const float f = src[i];
        nan |= (f != f);
        s.keys[i] = monotone_key(f);
    }
    if (__ballot(nan) != 0ull && (threadIdx.x & 63) == 0) flag(status, DSA_DEV_NAN);
}

__device__ int checked_vis(const TopkArgs& a, int r) {
    const int v = a.row_vis[r];
    if (v < 0 || v > a.score_stride) {
        if (threadIdx.x == 0) flag(a.status, DSA_DEV_ROW_RANGE);
        return 0;
    }
    return v;
}

__device__ void pad_tail(int32_t* out, int from, int k) {
    for (int i = from + threadIdx.x; i < k; i += kThreads) out[i] = -1;
}

// One split, or the whole row: grid (n_splits, n_rows).
__global__ __launch_bounds__(kThreads) void topk_split_kernel(TopkArgs a) {
    __shared__ TopkSmem s;
    const int r = blockIdx.y;
    const int j = blockIdx.x;
    const int v = checked_vis(a, r);
    const int c = (v + a.n_splits - 1) / a.n_splits;
    const int lo = min(v, j * c);
    const int hi = min(v, lo + c);
    const int n = hi - lo;
    const int k = a.top_k;
    const bool direct = a.n_splits == 1;
    int32_t* out_idx = direct ? a.topk_idx + (size_t)r * k
                              : a.cand_slot + ((size_t)r * a.n_splits + j) * k;
    uint32_t* out_key = direct ? nullptr : a.cand_key + ((size_t)r * a.n_splits + j) * k;
    const int cnt = min(n, k);
    if (threadIdx.x == 0) {
        if (direct) a.topk_count[r] = cnt;
        else a.cand_count[(size_t)r * a.n_splits + j] = cnt;
    }
    const float* src = a.scores + (size_t)r * a.score_stride + lo;
    if (n <= k) {
        // Everything in the range is selected.
        if (direct) {
            for (int i = threadIdx.x; i < n; i += kThreads) out_idx[i] = lo + i;
            pad_tail(out_idx, n, k);
        } else {
            bool nan = false;
            for (int i = threadIdx.x; i < n; i += kThreads) {
                const float f = src[i];
                nan |= (f != f);
                out_idx[i] = lo + i;
                out_key[i] = monotone_key(f);
            }
            if (__ballot(nan) != 0ull && (threadIdx.x & 63) == 0) flag(a.status, DSA_DEV_NAN);
        }
        return;
    }
    load_keys(s, src, n, a.status);
    __syncthreads();
    uint32_t thr;
    int need;
    radix_select(s, n, k, &thr, &need);
    // The emitters never see rank >= k when the selection is right; the
    // guard keeps a wrong selection from writing past the row.
    if (direct) {
        ordered_emit(s, n, thr, need, [&](int rank, int pos) {
            if (rank < k) out_idx[rank] = lo + pos;
        });
    } else {
        ordered_emit(s, n, thr, need, [&](int rank, int pos) {
            if (rank < k) {
                out_idx[rank] = lo + pos;
                out_key[rank] = s.keys[pos];
            }
        });
    }
}

// Merge of the split candidates of one row: grid (n_rows).
__global__ __launch_bounds__(kThreads) void topk_merge_kernel(TopkArgs a) {
    __shared__ TopkSmem s;
    const int r = blockIdx.x;
    const int k = a.top_k;
    const int ns = a.n_splits;
    int32_t* out_idx = a.topk_idx + (size_t)r * k;
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        const int c = lane < ns ? min(max(a.cand_count[(size_t)r * ns + lane], 0), k) : 0;
        const uint32_t inc = wave_inclusive_scan((uint32_t)c);
        if (lane < ns) s.offs[lane] = (int)(inc - c);
        if (lane == 63) s.n = (int)inc;
    }
    __syncthreads();
    const int n = s.n;
    if (threadIdx.x == 0) a.topk_count[r] = min(n, k);
    const int32_t* cslot = a.cand_slot + (size_t)r * ns * k;
    const uint32_t* ckey = a.cand_key + (size_t)r * ns * k;
    if (n <= k) {
        for (int j = 0; j < ns; ++j) {
            const int o = s.offs[j];
            const int c = (j + 1 < ns ? s.offs[j + 1] : n) - o;
            for (int i = threadIdx.x; i < c; i += kThreads) out_idx[o + i] = cslot[(size_t)j * k + i];
        }
        pad_tail(out_idx, n, k);
        return;
    }
    for (int j = 0; j < ns; ++j) {
        const int o = s.offs[j];
        const int c = (j + 1 < ns ? s.offs[j + 1] : n) - o;
        for (int i = threadIdx.x; i < c; i += kThreads) s.keys[o + i] = ckey[(size_t)j * k + i];
    }
    __syncthreads();
    uint32_t thr;
    int need;
    radix_select(s, n, k, &thr, &need);
    ordered_emit(s, n, thr, need, [&](int rank, int pos) {
        if (rank >= k) return;
        // Split of list position `pos`: last split whose offset is <= pos.
        int lo = 0, hi = ns - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s.offs[mid] <= pos) lo = mid; else hi = mid - 1;
        }
        out_idx[rank] = cslot[(size_t)lo * k + (pos - s.offs[lo])];
    });
}

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t stream) {
    if (a.n_rows == 0) return hipSuccess;
    topk_split_kernel<<<dim3(a.n_splits, a.n_rows), kThreads, 0, stream>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.n_splits == 1) return e;
    topk_merge_kernel<<<a.n_rows, kThreads, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace dsa
