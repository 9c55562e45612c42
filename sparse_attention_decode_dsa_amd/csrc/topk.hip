// Exact top-k under (score descending, slot ascending), per split then merged.
//
// One 1024-thread workgroup selects from one list of at most 32768 fp32
// scores.  Lists are always in ascending slot order, so list order is slot
// order:
//   - direct (one split): the row's scores [0, row_vis);
//   - split pass: one contiguous slot range of the row -> candidate keys and
//     slots in a workspace;
//   - merge pass: the concatenated candidates of the row's splits, in split
//     order.
// Local top-k per split followed by an exact merge equals the global top-k
// because every member of the global top-k is in its own split's top-k.
//
// Scores become order-preserving uint32 keys.  Thread t holds the keys of
// list positions [t*P, t*P + P) in registers (P = ceil(n / 1024) <= 32).
// Selection finds the k-th largest key `thr` and how many keys equal to it
// belong to the top k, with few per-key LDS atomics (they serialise):
//   1. the first key of every thread is a sample of the list; one atomic per
//      thread builds its histogram over the top 12 key bits, and a scan of
//      it gives the bins holding the sample ranks rho -+ delta (rho = k *
//      samples / n, delta = 4 binomial standard deviations + 4);
//   2. keys in bins above that bracket are counted; keys inside it are
//      compacted, in list order, into LDS;
//   3. an exact radix select (12, 10 and 10 bits) over the compacted keys
//      finds the rank k - (keys above) among them.
// If the bracket misses or holds more keys than LDS has room for (heavy
// ties), the same radix select runs over all keys instead.
// Emission: per-thread counts and two workgroup scans give every selected
// position its output rank, so the output comes out in list order.  Keys
// above `thr` are taken; keys equal to `thr` are taken in list order until
// the count is reached, which keeps the lowest slots among ties.
#include "device_common.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kThreads = 1024;
constexpr int kPer = kTopkMaxList / kThreads;   // keys per thread (32)
constexpr int kBins0 = 4096;                    // key bits [31:20]
constexpr int kBins1 = 1024;                    // then [19:10] and [9:0]
constexpr int kCandCap = 4096;

struct TopkSmem {
    union {
        // Staging of the list's keys for the transpose from coalesced loads
        // to each thread's contiguous positions (16-byte chunks XOR-swizzled).
        uint32_t stage[kTopkMaxList];
        struct {
            uint32_t hist[kBins0];
            uint32_t cand_key[kCandCap];
        } sel;
    } u;
    uint32_t scan[kThreads / kWave + 1];
    int32_t offs[kMaxSplits + 1];
    uint32_t sel_digit;
    uint32_t sel_need;
    int32_t n;
};

__device__ __forceinline__ uint32_t bin0(uint32_t key) { return key >> 20; }

// Digit d (of NB bins, scanned from the largest) whose bin holds the kk-th
// largest counted key: s.sel_digit = d, s.sel_need = kk minus the keys in
// larger bins.  Thread t owns the NB/kThreads bins just below
// NB - t * (NB / kThreads).
template <int NB>
__device__ void find_digit(TopkSmem& s, uint32_t kk) {
    constexpr int PER = NB / kThreads;
    const int tid = threadIdx.x;
    uint32_t c[PER];
    uint32_t sum = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        c[j] = s.u.sel.hist[NB - 1 - (tid * PER + j)];
        sum += c[j];
    }
    uint32_t total;
    uint32_t above = block_exclusive_scan<kThreads>(sum, s.scan, &total);
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        if (above < kk && above + c[j] >= kk) {
            s.sel_digit = (uint32_t)(NB - 1 - (tid * PER + j));
            s.sel_need = kk - above;
        }
        above += c[j];
    }
    __syncthreads();
}

__device__ void clear_hist(TopkSmem& s, int nb) {
    for (int i = threadIdx.x; i < nb; i += kThreads) s.u.sel.hist[i] = 0;
    __syncthreads();
}

// Exact kk-th largest key (and the number of equal keys in the top kk)
// among the keys get(i, &key) yields for i in [0, M) on each thread, by
// three histogram passes of 12, 10 and 10 bits.
template <int M, typename Get>
__device__ void radix_select(TopkSmem& s, uint32_t kk, Get get, uint32_t* thr_out, uint32_t* need_out) {
    clear_hist(s, kBins0);
#pragma unroll
    for (int i = 0; i < M; ++i) {
        uint32_t key;
        if (get(i, &key)) atomicAdd(&s.u.sel.hist[bin0(key)], 1u);
    }
    __syncthreads();
    find_digit<kBins0>(s, kk);
    uint32_t prefix = s.sel_digit << 20;
    uint32_t mask = 0xFFF00000u;
    kk = s.sel_need;
#pragma unroll 1
    for (int pass = 0; pass < 2; ++pass) {
        const int shift = pass == 0 ? 10 : 0;
        __syncthreads();
        clear_hist(s, kBins1);
#pragma unroll
        for (int i = 0; i < M; ++i) {
            uint32_t key;
            if (get(i, &key) && (key & mask) == prefix) atomicAdd(&s.u.sel.hist[(key >> shift) & (kBins1 - 1)], 1u);
        }
        __syncthreads();
        find_digit<kBins1>(s, kk);
        prefix |= s.sel_digit << shift;
        mask |= (uint32_t)(kBins1 - 1) << shift;
        kk = s.sel_need;
    }
    __syncthreads();
    *thr_out = prefix;
    *need_out = kk;
}

// k-th largest (1 <= k < n) of the n keys, thread t holding `mine` of them
// in key[0, mine).
__device__ void select_kth(TopkSmem& s, const uint32_t (&key)[kPer], int mine, int n, int k,
                           uint32_t* thr_out, uint32_t* need_out) {
    const int tid = threadIdx.x;
    const int per = (n + kThreads - 1) / kThreads;
    const int samples = (n + per - 1) / per;        // threads holding a key
    // 1. Sample histogram and the bracket of bins around rank k.
    clear_hist(s, kBins0);
    if (mine > 0) atomicAdd(&s.u.sel.hist[bin0(key[0])], 1u);
    __syncthreads();
    const float rho = (float)k * (float)samples / (float)n;
    const float sigma = sqrtf(fmaxf(rho * (1.0f - rho / (float)samples), 0.0f));
    const int delta = (int)ceilf(4.0f * sigma) + 4;
    const int r_hi = (int)rho - delta;
    const int r_lo = (int)ceilf(rho) + delta;
    uint32_t b_hi = kBins0 - 1, b_lo = 0;   // bracket bins, inclusive
    if (r_hi >= 1) {
        find_digit<kBins0>(s, (uint32_t)r_hi);
        b_hi = s.sel_digit;
    }
    if (r_lo <= samples) {
        find_digit<kBins0>(s, (uint32_t)r_lo);
        b_lo = s.sel_digit;
    }
    // 2. Count keys above the bracket; compact the keys inside it in order.
    uint32_t above = 0, inside = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        if (i < mine) {
            const uint32_t b = bin0(key[i]);
            above += b > b_hi;
            inside += (b >= b_lo && b <= b_hi);
        }
    }
    uint32_t tot_above, tot_inside;
    block_exclusive_scan<kThreads>(above, s.scan, &tot_above);
    uint32_t at = block_exclusive_scan<kThreads>(inside, s.scan, &tot_inside);
    const bool fast = tot_above < (uint32_t)k && tot_above + tot_inside >= (uint32_t)k &&
                      tot_inside <= (uint32_t)kCandCap;
    if (fast) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            if (i < mine) {
                const uint32_t b = bin0(key[i]);
                if (b >= b_lo && b <= b_hi) s.u.sel.cand_key[at++] = key[i];
            }
        }
        __syncthreads();
        // 3. Exact rank among the compacted keys (4 per thread).
        const uint32_t nc = tot_inside;
        radix_select<kCandCap / kThreads>(
            s, (uint32_t)k - tot_above,
            [&](int i, uint32_t* kv) {
                const uint32_t j = (uint32_t)tid + (uint32_t)(kThreads * i);
                if (j >= nc) return false;
                *kv = s.u.sel.cand_key[j];
                return true;
            },
            thr_out, need_out);
        return;
    }
    radix_select<kPer>(
        s, (uint32_t)k,
        [&](int i, uint32_t* kv) {
            if (i >= mine) return false;
            *kv = key[i];
            return true;
        },
        thr_out, need_out);
}

// Emit the selected keys in list order: emit(rank, i) for the thread's key i.
template <typename Emit>
__device__ void ordered_emit(TopkSmem& s, const uint32_t (&key)[kPer], int mine, uint32_t thr,
                             uint32_t need_eq, Emit emit) {
    uint32_t eq = 0, gt = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        if (i < mine) {
            eq += key[i] == thr;
            gt += key[i] > thr;
        }
    }
    uint32_t tot;
    const uint32_t eq_before = block_exclusive_scan<kThreads>(eq, s.scan, &tot);
    const uint32_t take_eq = min(eq, need_eq > eq_before ? need_eq - eq_before : 0u);
    uint32_t rank = block_exclusive_scan<kThreads>(gt + take_eq, s.scan, &tot);
    uint32_t eq_left = take_eq;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        if (i < mine) {
            bool take = key[i] > thr;
            if (key[i] == thr && eq_left > 0) {
                take = true;
                --eq_left;
            }
            if (take) emit((int)rank++, i);
        }
    }
}

// Word index in the staging buffer of list element i: 16-byte chunk c =
// i / 4 is stored at chunk c ^ ((c / 8) % 8), so that both the coalesced
// writes (consecutive chunks) and each thread's reads of its own 8
// consecutive chunks spread over distinct bank groups.
__device__ __forceinline__ int stage_index(int i) {
    const int c = i >> 2;
    return ((c ^ ((c >> 3) & 7)) << 2) | (i & 3);
}

// Keys of list positions [base, base + mine) into registers.  `get(i)`
// gives the key of list position i; it is called with consecutive i across
// lanes (coalesced) and every load of a thread is issued before any use.
template <typename Get>
__device__ void load_list(TopkSmem& s, int n, int base, int mine, uint32_t (&key)[kPer], Get get) {
    uint32_t v[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const int i = u * kThreads + (int)threadIdx.x;
        v[u] = i < n ? get(i) : 0u;
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const int i = u * kThreads + (int)threadIdx.x;
        if (i < n) s.u.stage[stage_index(i)] = v[u];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kPer; ++i) key[i] = i < mine ? s.u.stage[stage_index(base + i)] : 0u;
    __syncthreads();
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
    const int per = (n + kThreads - 1) / kThreads;
    const int base = threadIdx.x * per;
    const int mine = max(0, min(per, n - base));
    uint32_t key[kPer];
    bool nan = false;
    load_list(s, n, base, mine, key, [&](int i) {
        const float f = src[i];
        nan |= (f != f);
        return monotone_key(f);
    });
    if (__ballot(nan) != 0ull && (threadIdx.x & 63) == 0) flag(a.status, DSA_DEV_NAN);
    uint32_t thr, need;
    select_kth(s, key, mine, n, k, &thr, &need);
    // A right selection never produces rank >= k; the guard keeps a wrong
    // one from writing past the row.
    if (direct) {
        ordered_emit(s, key, mine, thr, need, [&](int rank, int i) {
            if (rank < k) out_idx[rank] = lo + base + i;
        });
    } else {
        ordered_emit(s, key, mine, thr, need, [&](int rank, int i) {
            if (rank < k) {
                out_idx[rank] = lo + base + i;
                out_key[rank] = key[i];
            }
        });
    }
}

// Split owning position `pos` of the concatenated candidate list: the last
// split whose offset is <= pos (empty splits share the next one's offset).
__device__ __forceinline__ int split_of(const TopkSmem& s, int ns, int pos) {
    int lo = 0, hi = ns - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s.offs[mid] <= pos) lo = mid; else hi = mid - 1;
    }
    return lo;
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
    // Candidate list position -> its entry in the workspace.
    auto entry = [&](int pos) -> size_t {
        const int j = split_of(s, ns, pos);
        return (size_t)j * k + (pos - s.offs[j]);
    };
    const int per = (n + kThreads - 1) / kThreads;
    const int base = threadIdx.x * per;
    const int mine = max(0, min(per, n - base));
    if (n <= k) {
        // Every candidate is selected, in list order.
        int32_t sl[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i) sl[i] = i < mine ? cslot[entry(base + i)] : -1;
#pragma unroll
        for (int i = 0; i < kPer; ++i)
            if (i < mine) out_idx[base + i] = sl[i];
        pad_tail(out_idx, n, k);
        return;
    }
    uint32_t key[kPer];
    load_list(s, n, base, mine, key, [&](int i) { return ckey[entry(i)]; });
    uint32_t thr, need;
    select_kth(s, key, mine, n, k, &thr, &need);
    ordered_emit(s, key, mine, thr, need, [&](int rank, int i) {
        if (rank < k) out_idx[rank] = cslot[entry(base + i)];
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
