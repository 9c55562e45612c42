// Exact top-k under (score descending, slot ascending), per split then merged.
//
// One 1024-thread workgroup selects from one list of at most 32768 fp32
// scores.  Lists are always in ascending slot order, so list order is slot
// order:
//   - direct (one split): the row's scores [0, row_vis);
//   - split pass: one contiguous slot range of the row -> candidate keys and
//     slots in a workspace, at an offset that the row's visible count alone
//     fixes (the candidates of the splits before it), so the row's
//     candidates form one list in split order;
//   - merge pass: that list.
// Local top-k per split followed by an exact merge equals the global top-k
// because every member of the global top-k is in its own split's top-k.
//
// Scores become order-preserving uint32 keys.  Thread t holds the keys of
// list positions [t*p, t*p + p) in registers (p = ceil(n / 1024) rounded up
// to a multiple of 4, at most 32).  Every pass over them is compiled for
// P = 4, 8, 16 or 32 keys; a launch uses the smallest P >= p of its longest
// possible list, so short lists cost proportionally less work per thread.
// Selection finds the k-th largest key `thr` and how many keys equal to it
// belong to the top k, with few per-key LDS atomics (they serialise):
//   1. the first key of every thread is a sample of the list; one atomic per
//      thread builds its histogram over the top 12 key bits, and one scan of
//      it gives the bins holding the sample ranks rho -+ delta (rho = k *
//      samples / n, delta = 4 binomial standard deviations + 4);
//   2. keys in bins above that bracket are counted; keys inside it are
//      compacted, in list order, into LDS;
//   3. an exact radix select over the compacted keys finds the rank
//      k - (keys above) among them: two 12-bit passes when the bracket spans
//      fewer than 16 bins (the first digit is the bin's offset in the bracket
//      and key bits [19:12], the second bits [11:0]), else 12, 10 and 10 bits.
// Barriers are the cost of a workgroup this size, so histograms are cleared
// ahead under barriers that are needed anyway, and the scans alternate two
// scratch arrays, which saves the barrier that would protect one array from
// the next scan.
// If the bracket misses or holds more keys than LDS has room for (heavy
// ties), the same radix select runs over all keys instead.
// Emission: per-thread counts and one workgroup scan give every selected
// position its output rank; positions go to LDS at their ranks and out to
// global memory in one coalesced pass, in list order.  Keys
// above `thr` are taken; keys equal to `thr` are taken in list order until
// the count is reached, which keeps the lowest slots among ties.
#include "device_common.h"
#include "launch.h"

#include <type_traits>

namespace dsa {

namespace {

constexpr int kThreads = 1024;
constexpr int kPer = kTopkMaxList / kThreads;   // most keys per thread (32)
static_assert(kPer == 32, "the largest key count with_keys_per_thread compiles for");
constexpr int kBins0 = 4096;                    // key bits [31:20]
constexpr int kBins1 = 1024;                    // then [19:10] and [9:0]
constexpr int kCandCap = 4096;
constexpr int kComputeUnits = 256;   // MI355X

constexpr int kPtLds = 1024;

// LDS of one selection workgroup.  The staging buffer (the list's keys on
// their way from coalesced loads to each thread's contiguous positions, in
// XOR-swizzled 16-byte chunks: kStage words, the longest list a launch
// allows, or half of it for lists staged in two rounds) shares its space
// with the selection's candidate histograms and with the emitted positions
// (at word 0) and keys (at word kEmitKey), at most kMaxK each plus one dummy
// word per lane.  kPt: room for the page ids of the physical-rows variants.
template <int kStage, bool kPt>
struct TopkSmemT {
    static constexpr int kStageWords = kStage;
    static constexpr int kSelWords = 2 * kBins0 + kCandCap + kWave;
    static constexpr int kUnionWords = kStage > kSelWords ? kStage : kSelWords;
    static constexpr int kEmitKey =
        2 * (kTopkMaxK + kWave) <= kUnionWords ? kTopkMaxK + kWave : kUnionWords / 2;
    static constexpr int kMaxK = kEmitKey - kWave;
    union {
        uint32_t stage[kUnionWords];
        struct {
            uint32_t hist[kBins0];
            uint32_t cand_key[kCandCap + kWave];   // + one dummy word per lane
            uint32_t hist2[kBins0];
        } sel;
    } u;
    uint32_t h0[kBins0];   // sample histogram, cleared before the list is staged
    uint32_t khist[512];   // filter pass: histogram of the kept keys above the cut
    uint32_t bkey[kWave];  // merge: the keys of the threshold bin, and the threshold found among them
    uint32_t bcount;
    uint32_t kept_top;     // filter pass: the key from which the kept-key histogram's last bin starts
    uint32_t sel_thr;
    uint32_t sel_need_eq;
    uint32_t scan[2][kThreads / kWave + 1];
    uint32_t sel_digit;
    uint32_t sel_digit2;
    uint32_t sel_need;
    int32_t pt[kPt ? kPtLds : 1];   // physical rows asked for: the row's request's page ids, when they fit
};
// Every launch's layout but the compact filter's.
using TopkSmem = TopkSmemT<kTopkMaxList, true>;
static_assert(TopkSmem::kEmitKey == kTopkMaxK + kWave && TopkSmem::kMaxK == kTopkMaxK, "full emission space");
// The filter pass for lists of at most 16 keys a thread (16384 keys, staged
// in two rounds) and top_k <= kMaxK (6112): about 67 KB, so two 1024-thread
// workgroups share a CU and overlap their barrier chains.
using TopkSmemCompact = TopkSmemT<kTopkMaxList / 4, false>;
static_assert(sizeof(TopkSmemCompact) <= 80 * 1024, "two compact workgroups per CU");

__device__ __forceinline__ uint32_t bin0(uint32_t key) { return key >> 20; }

// Where a row's selection goes: its slots, and when asked (rows != nullptr)
// the physical row of each slot through the row's request's block table
// (pt: page ids, staged in LDS when they fit; nullptr when the request is
// invalid, which gives -1).  A slot whose page id is outside the pool gives
// -1 and DSA_DEV_PAGE_OOB.
template <bool kRows>
struct OutRow {
    static constexpr bool kHasRows = kRows;   // the launch asked for physical rows
    int32_t* idx;
    int32_t* rows;
    const int32_t* pt;
    int32_t* status;
    int num_pages, page_size, log2_page, max_pages;
    __device__ __forceinline__ int row_of(int slot) const {
        if (pt == nullptr) return -1;
        const int p = slot >> log2_page;
        const int page = p < max_pages ? pt[p] : -1;
        if (page < 0 || page >= num_pages) {
            flag(status, DSA_DEV_PAGE_OOB);
            return -1;
        }
        return page * page_size + (slot & (page_size - 1));
    }
    __device__ __forceinline__ void put(int rank, int slot) const {
        idx[rank] = slot;
        if constexpr (kRows) rows[rank] = row_of(slot);
    }
};

// Row r's output; with physical rows asked for, the page ids of its request
// start loading into LDS (every user of them comes after a barrier).  v: the
// row's checked span.
template <bool kRows>
__device__ __forceinline__ OutRow<kRows> make_out(const TopkArgs& a, TopkSmem& s, int r, int v) {
    OutRow<kRows> o;
    o.idx = a.topk_idx + (size_t)r * a.top_k;
    if constexpr (kRows) {
        o.rows = a.topk_rows + (size_t)r * a.top_k;
        o.pt = nullptr;
        o.status = a.status;
        o.num_pages = a.num_pages;
        o.page_size = a.page_size;
        o.log2_page = a.log2_page;
        o.max_pages = a.max_pages;
        const int b = a.row_req[r];
        if (b < 0 || b >= a.batch || (int64_t)v > (int64_t)a.max_pages * a.page_size) {
            if (threadIdx.x == 0) flag(a.status, DSA_DEV_ROW_RANGE);
        } else {
            const int32_t* g = a.page_table + (size_t)b * a.max_pages;
            if (a.max_pages <= kPtLds) {
                for (int i = threadIdx.x; i < a.max_pages; i += kThreads) s.pt[i] = g[i];
                o.pt = s.pt;
            } else {
                o.pt = g;
            }
        }
    }
    return o;
}


// Keys per thread for a list of n: a multiple of 4 (whole 16-byte chunks),
// at most kPer.
__device__ __forceinline__ int keys_per_thread(int n) {
    return ((n + 4 * kThreads - 1) / (4 * kThreads)) * 4;
}

// Workgroup exclusive scan in two barriers.  Successive scans alternate the
// two scratch arrays (`tog` flips on every call and is the same in every
// thread), so a scan never writes the array the previous one is still
// being read from.
template <class S>
__device__ __forceinline__ uint32_t scan2(S& s, uint32_t v, uint32_t* total, int& tog) {
    constexpr int NW = kThreads / kWave;
    uint32_t* scratch = s.scan[tog];
    tog ^= 1;
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
    const uint32_t inc = wave_inclusive_scan(v);
    if (lane == kWave - 1) scratch[w] = inc;
    __syncthreads();
    if (w == 0) {
        const uint32_t x = lane < NW ? scratch[lane] : 0u;
        const uint32_t xi = wave_inclusive_scan(x);
        if (lane < NW) scratch[lane] = xi - x;
        if (lane == NW - 1) scratch[NW] = xi;
    }
    __syncthreads();
    *total = scratch[NW];
    return inc - v + scratch[w];
}

// Digit d (of NB bins of `hist`, scanned from the largest) whose bin holds
// the kk-th largest counted key: s.sel_digit = d, s.sel_need = kk minus the
// keys in larger bins.  Thread t owns the NB/kThreads bins just below
// NB - t * (NB / kThreads).
template <int NB, class S>
__device__ __forceinline__ void find_digit(S& s, const uint32_t* hist, uint32_t kk, int& tog) {
    constexpr int PER = NB / kThreads;
    const int tid = threadIdx.x;
    uint32_t c[PER];
    uint32_t sum = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        c[j] = hist[NB - 1 - (tid * PER + j)];
        sum += c[j];
    }
    uint32_t total;
    uint32_t above = scan2(s, sum, &total, tog);
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

// The bins holding the kk_hi-th and kk_lo-th largest keys of `hist`, in one
// scan: s.sel_digit (kBins0 - 1 if kk_hi == 0) and s.sel_digit2 (0 if
// kk_lo == 0).
template <int NB, class S>
__device__ __forceinline__ void find_digit2(S& s, const uint32_t* hist, uint32_t kk_hi, uint32_t kk_lo,
                                            int& tog) {
    constexpr int PER = NB / kThreads;
    const int tid = threadIdx.x;
    if (tid == 0) {
        s.sel_digit = NB - 1;
        s.sel_digit2 = 0;
    }
    uint32_t c[PER];
    uint32_t sum = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        c[j] = hist[NB - 1 - (tid * PER + j)];
        sum += c[j];
    }
    uint32_t total;
    uint32_t above = scan2(s, sum, &total, tog);
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const uint32_t d = (uint32_t)(NB - 1 - (tid * PER + j));
        if (above < kk_hi && above + c[j] >= kk_hi) s.sel_digit = d;
        if (above < kk_lo && above + c[j] >= kk_lo) s.sel_digit2 = d;
        above += c[j];
    }
    __syncthreads();
}

template <class S>
__device__ __forceinline__ void clear_hist(S& s, int nb) {
    for (int i = threadIdx.x; i < nb; i += kThreads) s.u.sel.hist[i] = 0;
    __syncthreads();
}

// Exact kk-th largest key (and the number of equal keys in the top kk)
// among the keys get(i, &key) yields for i in [0, M) on each thread, by
// three histogram passes of 12, 10 and 10 bits.
template <int M, class S, typename Get>
__device__ __forceinline__ void radix_select(S& s, uint32_t kk, Get get, uint32_t* thr_out,
                                             uint32_t* need_out, int& tog) {
    clear_hist(s, kBins0);
#pragma unroll
    for (int i = 0; i < M; ++i) {
        uint32_t key;
        if (get(i, &key)) atomicAdd(&s.u.sel.hist[bin0(key)], 1u);
    }
    __syncthreads();
    find_digit<kBins0>(s, s.u.sel.hist, kk, tog);
    uint32_t prefix = s.sel_digit << 20;
    kk = s.sel_need;
    uint32_t mask = 0xFFF00000u;
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
        find_digit<kBins1>(s, s.u.sel.hist, kk, tog);
        prefix |= s.sel_digit << shift;
        mask |= (uint32_t)(kBins1 - 1) << shift;
        kk = s.sel_need;
    }
    __syncthreads();
    *thr_out = prefix;
    *need_out = kk;
}

// k-th largest (1 <= k < n) of the n keys, thread t holding `mine` of them
// in key[0, mine).  s.h0 must be zero (the caller clears it before staging
// the list).
template <int P, class S>
__device__ __forceinline__ void select_kth(S& s, const uint32_t (&key)[P], int mine, int n, int k,
                                           uint32_t* thr_out, uint32_t* need_out, int& tog) {
    const int tid = threadIdx.x;
    const int per = keys_per_thread(n);
    const int samples = (n + per - 1) / per;        // threads holding a key
    // The candidate histograms live where the list was staged; clear them
    // now, under the sample histogram's barrier.
    for (int i = tid; i < kBins0; i += kThreads) {
        s.u.sel.hist[i] = 0u;
        s.u.sel.hist2[i] = 0u;
    }
    // 1. Sample histogram and the bracket of bins around rank k.
    if (mine > 0) atomicAdd(&s.h0[bin0(key[0])], 1u);
    __syncthreads();
    const float rho = (float)k * (float)samples / (float)n;
    const float sigma = sqrtf(fmaxf(rho * (1.0f - rho / (float)samples), 0.0f));
    const int delta = (int)ceilf(4.0f * sigma) + 4;
    const int r_hi = (int)rho - delta;
    const int r_lo = (int)ceilf(rho) + delta;
    // bracket bins, inclusive: [b_lo, b_hi] (the whole range when a rank falls
    // outside the sample)
    find_digit2<kBins0>(s, s.h0, r_hi >= 1 ? (uint32_t)r_hi : 0u, r_lo <= samples ? (uint32_t)r_lo : 0u, tog);
    uint32_t b_hi = s.sel_digit, b_lo = s.sel_digit2;
    // 2. Count keys above the bracket; compact the keys inside it in order.
    // Positions past a thread's share hold key 0 (bin 0); bin 0 is kept out
    // of the bracket, so they are never counted, and a real key of bin 0 (a
    // negative NaN pattern) only sends the selection to the fallback.
    b_lo = max(b_lo, 1u);
    uint32_t above = 0, inside = 0;
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const uint32_t b = bin0(key[i]);
        above += b > b_hi;
        inside += b >= b_lo && b <= b_hi;
    }
    // One scan of (above, inside) in 16-bit halves (each total <= 32768).
    uint32_t tot;
    const uint32_t both = scan2(s, (above << 16) | inside, &tot, tog);
    const uint32_t tot_above = tot >> 16, tot_inside = tot & 0xFFFFu;
    uint32_t at = both & 0xFFFFu;
    const bool fast = tot_above < (uint32_t)k && tot_above + tot_inside >= (uint32_t)k &&
                      tot_inside <= (uint32_t)kCandCap;
    if (fast) {
        // Branch-free: a key outside the bracket goes to the lane's dummy word.
        // The bounds are re-pinned so the compiler recomputes each key's test
        // here instead of keeping 32 of them live across the scan.
        pin(b_lo);
        pin(b_hi);
        const uint32_t dummy = (uint32_t)kCandCap + (threadIdx.x & (kWave - 1));
#pragma unroll
        for (int i = 0; i < P; ++i) {
            const uint32_t b = bin0(key[i]);
            const bool in = b >= b_lo && b <= b_hi;
            s.u.sel.cand_key[in ? at : dummy] = key[i];
            at += in;
        }
        __syncthreads();
        // 3. Exact rank among the compacted keys (4 per thread).
        const uint32_t nc = tot_inside;
        const uint32_t kk = (uint32_t)k - tot_above;
        if (b_hi - b_lo < 16u) {
            // Two 12-bit passes: (bin offset in the bracket, bits [19:12]),
            // then bits [11:0] among the keys sharing the first digit.
            constexpr int M = kCandCap / kThreads;
#pragma unroll
            for (int i = 0; i < M; ++i) {
                const uint32_t j = (uint32_t)tid + (uint32_t)(kThreads * i);
                if (j < nc) {
                    const uint32_t kv = s.u.sel.cand_key[j];
                    atomicAdd(&s.u.sel.hist[((bin0(kv) - b_lo) << 8) | ((kv >> 12) & 0xFFu)], 1u);
                }
            }
            __syncthreads();
            find_digit<kBins0>(s, s.u.sel.hist, kk, tog);
            const uint32_t d1 = s.sel_digit;
            const uint32_t kk2 = s.sel_need;
            const uint32_t top20 = ((b_lo + (d1 >> 8)) << 8) | (d1 & 0xFFu);   // key bits [31:12]
#pragma unroll
            for (int i = 0; i < M; ++i) {
                const uint32_t j = (uint32_t)tid + (uint32_t)(kThreads * i);
                if (j < nc) {
                    const uint32_t kv = s.u.sel.cand_key[j];
                    if ((kv >> 12) == top20) atomicAdd(&s.u.sel.hist2[kv & 0xFFFu], 1u);
                }
            }
            __syncthreads();
            find_digit<kBins0>(s, s.u.sel.hist2, kk2, tog);
            *thr_out = (top20 << 12) | s.sel_digit;
            *need_out = s.sel_need;
            return;
        }
        radix_select<kCandCap / kThreads>(
            s, kk,
            [&](int i, uint32_t* kv) {
                const uint32_t j = (uint32_t)tid + (uint32_t)(kThreads * i);
                if (j >= nc) return false;
                *kv = s.u.sel.cand_key[j];
                return true;
            },
            thr_out, need_out, tog);
        return;
    }
    radix_select<P>(
        s, (uint32_t)k,
        [&](int i, uint32_t* kv) {
            if (i >= mine) return false;
            *kv = key[i];
            return true;
        },
        thr_out, need_out, tog);
}

// LDS word of the emitted list positions (each k + one dummy per lane),
// inside the staging buffer, which is free once the keys are in registers;
// the keys follow at the layout's kEmitKey.
constexpr int kEmitPos = 0;
static_assert(2 * (kTopkMaxK + kWave) <= kTopkMaxList, "emission buffers fit the staging buffer");

// Selected keys in list order: a key is taken if it is above `thr`, or equal
// to it and among the first need_eq equal keys.  After one packed scan each
// thread's taken keys have consecutive ranks; their list positions (base +
// i) and keys are written to LDS at those ranks without branches (a key not
// taken goes to the lane's dummy word), for a coalesced copy out afterwards
// (after a barrier, by the caller).
template <int P, class S>
__device__ __forceinline__ void emit_to_lds(S& s, const uint32_t (&key)[P], int base,
                                            uint32_t thr, uint32_t need_eq, int k, int& tog) {
    // Positions past the thread's share hold key 0, which is never above a
    // threshold; equal keys are only counted for a nonzero threshold (a zero
    // one means NaN scores, an error the caller is told about).
    const uint32_t eq_key = thr != 0u ? thr : 0xFFFFFFFFu;
    const bool eq_ok = thr != 0u;
    uint32_t eq = 0, gt = 0;
#pragma unroll
    for (int i = 0; i < P; ++i) {
        eq += key[i] == eq_key && eq_ok;
        gt += key[i] > thr;
    }
    // One scan of (gt, eq) packed in 16-bit halves (each total <= 32768):
    // the equal keys taken before this thread are min(eq_before, need_eq).
    uint32_t tot;
    const uint32_t both = scan2(s, (gt << 16) | eq, &tot, tog);
    const uint32_t eq_before = both & 0xFFFFu;
    uint32_t eq_left = min(eq, need_eq > eq_before ? need_eq - eq_before : 0u);
    uint32_t rank = (both >> 16) + min(eq_before, need_eq);
    const uint32_t dummy = (uint32_t)k + (threadIdx.x & (kWave - 1));
    uint32_t thr2 = thr, eq_key2 = eq_key;   // recompute the per-key tests after the scan
    pin(thr2);
    pin(eq_key2);
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const bool is_eq = key[i] == eq_key2 && eq_ok;
        const bool take = key[i] > thr2 || (is_eq && eq_left > 0);
        eq_left -= (is_eq && take) ? 1u : 0u;
        const uint32_t slot = take ? min(rank, (uint32_t)k - 1u) : dummy;
        s.u.stage[kEmitPos + slot] = (uint32_t)(base + i);
        s.u.stage[S::kEmitKey + slot] = key[i];
        rank += take;
    }
}

// Direct emission (one split): the same selection as emit_to_lds, but each
// thread walks only the set bits of its taken-key mask and writes the list
// positions straight to `out` at their ranks.
template <int P, typename Out>
__device__ __forceinline__ void emit_direct(TopkSmem& s, const uint32_t (&key)[P], int base, uint32_t thr,
                                            uint32_t need_eq, int k, const Out& out, int lo, int& tog) {
    const uint32_t eq_key = thr != 0u ? thr : 0xFFFFFFFFu;
    const bool eq_ok = thr != 0u;
    uint32_t gtm = 0u, eqm = 0u;
#pragma unroll
    for (int i = 0; i < P; ++i) {
        gtm |= (key[i] > thr ? 1u : 0u) << i;
        eqm |= (key[i] == eq_key && eq_ok ? 1u : 0u) << i;
    }
    uint32_t tot;
    const uint32_t both = scan2(s, ((uint32_t)__popc(gtm) << 16) | (uint32_t)__popc(eqm), &tot, tog);
    const uint32_t eq_before = both & 0xFFFFu;
    uint32_t take_eq = min((uint32_t)__popc(eqm), need_eq > eq_before ? need_eq - eq_before : 0u);
    uint32_t tm = gtm;
    for (uint32_t em = eqm; take_eq > 0; --take_eq) {   // the lowest take_eq equal keys
        tm |= em & (0u - em);
        em &= em - 1u;
    }
    uint32_t rank = (both >> 16) + min(eq_before, need_eq);
    while (tm != 0u) {
        const int i = __ffs(tm) - 1;
        tm &= tm - 1u;
        if (rank < (uint32_t)k) out.put(rank, lo + base + i);
        ++rank;
    }
}

// Chunk swizzle of the vector staging buffer: chunk c (16 bytes) lives at
// c ^ ((c / 32) % 8).  32 consecutive chunks (a coalesced write) keep 32
// distinct 16-byte bank slots, and so do the chunks 8t + m (or 4t + m) that
// 32 consecutive threads read for their own contiguous keys.
__device__ __forceinline__ int chunk_swz(int c) { return c ^ ((c >> 5) & 7); }

// Keys of list positions [base, base + mine) into registers from a 16-byte
// aligned list (fp32 scores, turned into keys, or keys already), in 16-byte
// loads (coalesced across lanes, all issued before any use) and 16-byte LDS
// accesses.  Chunks past the list reload its last chunk and are never read
// back; positions past n in the last chunk are masked.  Sets `nan` if a
// listed score is NaN.  A stage smaller than the list takes it in rounds:
// round r holds chunks [r C, r C + C) (C chunks a round), and each thread
// reads its chunks in the rounds that hold them.
template <int P, bool kScores, class S>
__device__ __forceinline__ void load_list_vec(S& s, const void* src, int n, int base, int mine,
                                              uint32_t (&key)[P], bool& nan) {
    constexpr int kStageChunks = S::kStageWords / 4;
    constexpr int kRounds = (P / 4 * kThreads + kStageChunks - 1) / kStageChunks;
    constexpr int kPerRound = P / 4 / kRounds;   // loads (of kThreads chunks) a round stages
    static_assert(kRounds * kPerRound == P / 4 && kPerRound * kThreads <= kStageChunks, "whole rounds");
    const int nch = (n + 3) >> 2;
    uint4* stage4 = reinterpret_cast<uint4*>(s.u.stage);
    uint4 v[P / 4];   // keys of list chunk u * kThreads + thread
    if constexpr (kScores) {
        float4 f4[P / 4];
#pragma unroll
        for (int u = 0; u < P / 4; ++u)
            f4[u] = reinterpret_cast<const float4*>(src)[min(u * kThreads + (int)threadIdx.x, nch - 1)];
#pragma unroll
        for (int u = 0; u < P / 4; ++u) {
            const int q = u * kThreads + (int)threadIdx.x;
            const float f[4] = {f4[u].x, f4[u].y, f4[u].z, f4[u].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) nan |= (f[j] != f[j]) && 4 * q + j < n;
            v[u] = uint4{monotone_key(f[0]), monotone_key(f[1]), monotone_key(f[2]), monotone_key(f[3])};
        }
    } else {
#pragma unroll
        for (int u = 0; u < P / 4; ++u)
            v[u] = reinterpret_cast<const uint4*>(src)[min(u * kThreads + (int)threadIdx.x, nch - 1)];
    }
    if constexpr (kRounds == 1) {
#pragma unroll
        for (int u = 0; u < P / 4; ++u) stage4[chunk_swz(u * kThreads + (int)threadIdx.x)] = v[u];
        __syncthreads();
#pragma unroll
        for (int m = 0; m < P / 4; ++m) {
            const uint4 x = stage4[chunk_swz(min((base >> 2) + m, kStageChunks - 1))];
            key[4 * m + 0] = 4 * m + 0 < mine ? x.x : 0u;
            key[4 * m + 1] = 4 * m + 1 < mine ? x.y : 0u;
            key[4 * m + 2] = 4 * m + 2 < mine ? x.z : 0u;
            key[4 * m + 3] = 4 * m + 3 < mine ? x.w : 0u;
        }
    } else {
#pragma unroll
        for (int i = 0; i < P; ++i) key[i] = 0u;
#pragma unroll
        for (int r = 0; r < kRounds; ++r) {
            constexpr int kRound = kPerRound * kThreads;   // chunks a round holds
            const int c0 = r * kRound;
            if (r > 0) __syncthreads();   // every thread has read the previous round
#pragma unroll
            for (int uu = 0; uu < kPerRound; ++uu) {
                const int u = r * kPerRound + uu;
                stage4[chunk_swz(u * kThreads + (int)threadIdx.x - c0)] = v[u];
            }
            __syncthreads();
#pragma unroll
            for (int m = 0; m < P / 4; ++m) {
                const int c = (base >> 2) + m;
                if (4 * m < mine && c >= c0 && c < c0 + kRound) {
                    const uint4 x = stage4[chunk_swz(c - c0)];
                    key[4 * m + 0] = 4 * m + 0 < mine ? x.x : 0u;
                    key[4 * m + 1] = 4 * m + 1 < mine ? x.y : 0u;
                    key[4 * m + 2] = 4 * m + 2 < mine ? x.z : 0u;
                    key[4 * m + 3] = 4 * m + 3 < mine ? x.w : 0u;
                }
            }
        }
    }
    __syncthreads();
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
template <int P, typename Get>
__device__ __forceinline__ void load_list(TopkSmem& s, int n, int base, int mine, uint32_t (&key)[P], Get get) {
    // Positions past n load position n - 1 again and are never read back;
    // every index stays inside the 32768-word staging buffer.
    uint32_t v[P];
#pragma unroll
    for (int u = 0; u < P; ++u) {
        const int i = u * kThreads + (int)threadIdx.x;
        v[u] = get(min(i, n - 1));
    }
#pragma unroll
    for (int u = 0; u < P; ++u) s.u.stage[stage_index(u * kThreads + (int)threadIdx.x)] = v[u];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const uint32_t x = s.u.stage[stage_index(min(base + i, kTopkMaxList - 1))];
        key[i] = i < mine ? x : 0u;
    }
    __syncthreads();
}

__device__ __forceinline__ int checked_vis(const TopkArgs& a, int r) {
    const int v = a.row_vis[r];
    if (v < 0 || v > a.score_stride) {
        if (threadIdx.x == 0) flag(a.status, DSA_DEV_ROW_RANGE);
        return 0;
    }
    return v;
}

// Slots only: nothing but the output row.
template <>
struct OutRow<false> {
    static constexpr bool kHasRows = false;
    int32_t* idx;
    __device__ __forceinline__ void put(int rank, int slot) const { idx[rank] = slot; }
};

template <typename Out>
__device__ __forceinline__ void pad_tail(const Out& o, int from, int k) {
    for (int i = from + threadIdx.x; i < k; i += kThreads) {
        o.idx[i] = -1;
        if constexpr (Out::kHasRows) o.rows[i] = -1;
    }
}

// Split j of a row with `v` visible slots: [lo, hi) with split length
// ceil(v / n_splits) rounded up to whole 16-byte chunks.
struct SplitRange {
    int lo, hi;
};
__device__ __forceinline__ SplitRange split_range(int v, int ns, int j) {
    const int c = (((v + ns - 1) / ns) + 3) & ~3;
    const int lo = min(v, j * c);
    return {lo, min(v, lo + c)};
}

// Whole row, one split: grid (1, n_rows); no row is longer than P keys per
// thread.
template <int P, bool kRows>
__global__ __launch_bounds__(kThreads) void topk_direct_kernel(TopkArgs a) {
    __shared__ TopkSmem s;
    const int r = blockIdx.y;
    const int n = checked_vis(a, r);
    const int k = a.top_k;
    if (threadIdx.x == 0) a.topk_count[r] = min(n, k);
    const float* src = a.scores + (size_t)r * a.score_stride;
    const auto out_idx = make_out<kRows>(a, s, r, n);
    if (n <= k) {
        // Everything visible is selected.
        if constexpr (kRows) __syncthreads();   // the page ids are in LDS
        for (int i = threadIdx.x; i < n; i += kThreads) out_idx.put(i, i);
        pad_tail(out_idx, n, k);
        return;
    }
    const int per = keys_per_thread(n);
    if (per > P) {   // the launch bound the list length by score_stride
        if (threadIdx.x == 0) flag(a.status, DSA_DEV_ROW_RANGE);
        return;
    }
    const int base = threadIdx.x * per;
    const int mine = max(0, min(per, n - base));
    uint32_t key[P];
    bool nan = false;
    for (int i = threadIdx.x; i < kBins0; i += kThreads) s.h0[i] = 0u;   // under the staging barrier
    // 16-byte loads read whole chunks, so the last one may reach up to three
    // floats past the list: taken only where those stay inside the row.
    if ((reinterpret_cast<uintptr_t>(src) & 15) == 0 && ((n + 3) & ~3) <= a.score_stride) {
        load_list_vec<P, true>(s, src, n, base, mine, key, nan);
    } else {
        load_list<P>(s, n, base, mine, key, [&](int i) {
            const float f = src[i];
            nan |= (f != f);
            return monotone_key(f);
        });
    }
    if (__ballot(nan) != 0ull && (threadIdx.x & 63) == 0) flag(a.status, DSA_DEV_NAN);
    uint32_t thr, need;
    int tog = 0;
    select_kth<P>(s, key, mine, n, k, &thr, &need, tog);
    // A right selection takes exactly k keys; ranks are clamped below k so
    // that a wrong one could not write past the buffers.
    emit_direct<P>(s, key, base, thr, need, k, out_idx, 0, tog);
}

// ---------------------------------------------------------------------------
// Several workgroups per row: a filter pass and an exact merge.
//
// A row's top k is a small part of it, so each split of the row keeps only
// the keys at or above one row-wide cut, estimated from a strided sample of
// the whole row that every split of the row reads alike: sample position
// t_i = floor(i * v / S) for i < S = min(512, v).  With rho = k S / v the
// expected number of sample keys in the top k and sigma = sqrt(rho (1 -
// rho / S)), the cut is the floor of the 12-bit key bin holding the sample
// key of rank R = ceil(rho + 4 sigma + 4) from the top (no cut when R > S),
// so about R v / S keys of the row pass.  A split with more than k keys at
// or above the cut keeps its exact top k instead.  Every kept key is then
// at or above the cut, and every dropped key is below it or below k kept
// keys of its own split, so once at least k keys are kept in total, the top
// k of the kept keys is the row's top k.  The merge checks that count; when
// the cut was too high (fewer than k kept) it selects from the whole row,
// streamed in passes.
// ---------------------------------------------------------------------------

constexpr int kSample = 512;

// The filter's histogram of its kept keys: kHistBins bins linear in score
// value from the cut's value up to the top of the 12-bit key bin of the
// sample key of rank max(1, floor(rho - 4 sigma - 4)) (the other end of the
// sample's bracket around rank k); keys at or above that top go to the last
// bin.  Bins in value rather than in key bits: the kept range can straddle
// zero (a negative cut under a positive k-th key), and bins of key bits
// counted from the cut then spend themselves on the octaves around zero and
// put most of the top k in the last one.  Linear bins leave some ten kept
// keys in the k-th key's bin at long context and prefill.  The same
// arithmetic in the filter and the merge gives the same bin for a key, and
// the bin never decreases as the key grows.
constexpr int kHistBins = 512;

struct KeptBins {
    uint32_t top;      // keys at or above it: the last bin
    float lo, scale;   // the cut's value, and bins per unit of score
};

// The score a monotone key stands for.
__device__ __forceinline__ float key_value(uint32_t key) {
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

__device__ __forceinline__ KeptBins kept_bins(uint32_t cut, uint32_t top) {
    KeptBins b;
    b.top = top;
    b.lo = key_value(cut);
    const float hi = key_value(top);
    b.scale = hi > b.lo ? (float)(kHistBins - 1) / (hi - b.lo) : 0.0f;   // NaN or an empty range: one bin
    return b;
}

__device__ __forceinline__ int kept_bin(uint32_t key, const KeptBins& b) {
    if (key >= b.top) return kHistBins - 1;
    const float t = (key_value(key) - b.lo) * b.scale;
    return t > 0.0f ? (int)fminf(t, (float)(kHistBins - 1)) : 0;
}

// The ranks of the row sample's bracket around the k-th key: R (the cut's,
// kSample + 1 for "no cut") and the upper end's.
__device__ __forceinline__ int cut_rank(int v, int k, int S) {
    if (S <= 0) return kSample + 1;
    const float rho = (float)k * (float)S / (float)v;
    const float sigma = sqrtf(fmaxf(rho * (1.0f - rho / (float)S), 0.0f));
    const int R = (int)ceilf(rho + 4.0f * sigma + 4.0f);
    return R > S ? kSample + 1 : R;
}

__device__ __forceinline__ int top_rank(int v, int k, int S) {
    const float rho = (float)k * (float)S / (float)v;
    const float sigma = sqrtf(fmaxf(rho * (1.0f - rho / (float)S), 0.0f));
    return max(1, (int)floorf(rho - 4.0f * sigma - 4.0f));
}

// Filter pass: grid (n_splits, n_rows).  Split j of row r writes its kept
// keys and slots, in slot order, at the front of its own block of k entries
// of the workspace, and their number to cand_count[r][j].  kCompact: the
// compact LDS layout (P <= 16, k <= TopkSmemCompact::kMaxK, every split
// 16-byte aligned and read whole, which the launch checks).
template <int P, bool kCompact>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kCompact ? 8 : 1)))
void topk_filter_kernel(TopkArgs a) {
    using Smem = std::conditional_t<kCompact, TopkSmemCompact, TopkSmem>;
    static_assert(!kCompact || P <= 16, "compact layout: at most 16 keys a thread");
    __shared__ Smem s;
    const int r = blockIdx.y;
    const int j = blockIdx.x;
    const int tid = threadIdx.x;
    const int v = checked_vis(a, r);
    const SplitRange sr = split_range(v, a.n_splits, j);
    const int lo = sr.lo;
    const int n = sr.hi - sr.lo;
    const int k = a.top_k;
    const size_t seg = ((size_t)r * a.n_splits + j) * k;
    const size_t rj = (size_t)r * a.n_splits + j;
    uint32_t* hist_out = reinterpret_cast<uint32_t*>(a.cand_hist) + rj * kHistBins;
    const float* row = a.scores + (size_t)r * a.score_stride;
    const int per = keys_per_thread(n);
    if (n <= 0 || per > P) {   // an empty split (per > P cannot happen: the launch bounds the length)
        if (per > P && n > 0 && tid == 0) flag(a.status, DSA_DEV_ROW_RANGE);
        if (tid == 0) {
            a.cand_count[rj] = 0;
            a.cand_cut[rj] = 0;
            a.cand_top[rj] = 0;
        }
        for (int b = tid; b < kHistBins; b += kThreads) hist_out[b] = 0u;
        return;
    }
    // The row sample goes out first.
    const int S = min(kSample, v);
    float sf = 0.0f;
    if (tid < S) sf = row[(int)((int64_t)tid * v / S)];
    const int base = tid * per;
    const int mine = max(0, min(per, n - base));
    uint32_t key[P];
    bool nan = false;
    const float* src = row + lo;
    for (int i = tid; i < kBins0; i += kThreads) s.h0[i] = 0u;   // under the staging barrier
    for (int i = tid; i < kHistBins; i += kThreads) s.khist[i] = 0u;
    if constexpr (kCompact) {
        load_list_vec<P, true>(s, src, n, base, mine, key, nan);
    } else if ((reinterpret_cast<uintptr_t>(src) & 15) == 0 && lo + ((n + 3) & ~3) <= a.score_stride) {
        load_list_vec<P, true>(s, src, n, base, mine, key, nan);
    } else {
        load_list<P>(s, n, base, mine, key, [&](int i) {
            const float f = src[i];
            nan |= (f != f);
            return monotone_key(f);
        });
    }
    if (__ballot(nan) != 0ull && (tid & 63) == 0) flag(a.status, DSA_DEV_NAN);
    // The cut: bin of the sample key of rank R.
    int tog = 0;
    const int R = cut_rank(v, k, S);
    uint32_t cut = 0u;
    if (R <= S) {
        if (tid < S) atomicAdd(&s.h0[bin0(monotone_key(sf))], 1u);
        __syncthreads();
        find_digit2<kBins0>(s, s.h0, (uint32_t)min(top_rank(v, k, S), R), (uint32_t)R, tog);
        cut = s.sel_digit2 << 20;
    }
    // The histogram's top waits in LDS (read after later barriers): the
    // loops below run at the register limit.
    if (tid == 0) s.kept_top = R <= S ? (s.sel_digit << 20) | 0xFFFFFu : 0xFFFFFFFFu;
    uint32_t c = 0;
#pragma unroll
    for (int i = 0; i < P; ++i) c += (i < mine && key[i] >= cut) ? 1u : 0u;
    uint32_t total;
    uint32_t at = scan2(s, c, &total, tog);
    int32_t* cslot = a.cand_slot + seg;
    uint32_t* ckey = a.cand_key + seg;
    if (total <= (uint32_t)k) {
        // Kept keys in list order into the staging buffer (free: the keys
        // are in registers), then out in one coalesced pass.
        pin(cut);
        int pbase = base;   // pinned: else base + i for every key is computed early and spilled
        pin(pbase);
        const uint32_t dummy = (uint32_t)k + (uint32_t)(tid & (kWave - 1));
#pragma unroll
        for (int i = 0; i < P; ++i) {
            const bool in = i < mine && key[i] >= cut;
            const uint32_t d = in ? at : dummy;
            s.u.stage[kEmitPos + d] = (uint32_t)(pbase + i);
            s.u.stage[Smem::kEmitKey + d] = key[i];
            at += in ? 1u : 0u;
        }
        __syncthreads();
        // The histogram from the kept keys alone (a small part of the list).
        const KeptBins bins = kept_bins(cut, s.kept_top);
        for (int i = tid; i < (int)total; i += kThreads) {
            const uint32_t kk = s.u.stage[Smem::kEmitKey + i];
            cslot[i] = lo + (int)s.u.stage[kEmitPos + i];
            ckey[i] = kk;
            atomicAdd(&s.khist[kept_bin(kk, bins)], 1u);
        }
        __syncthreads();
        for (int b = tid; b < kHistBins; b += kThreads) hist_out[b] = s.khist[b];
        if (tid == 0) {
            a.cand_count[rj] = (int)total;
            a.cand_cut[rj] = (int)cut;
            a.cand_top[rj] = (int)s.kept_top;
        }
        return;
    }
    // More than k keys of this split at or above the cut: its exact top k.
    for (int i = tid; i < kBins0; i += kThreads) s.h0[i] = 0u;
    __syncthreads();
    uint32_t thr, need;
    select_kth<P>(s, key, mine, n, k, &thr, &need, tog);
    emit_to_lds<P>(s, key, base, thr, need, k, tog);
    __syncthreads();
    const KeptBins bins = kept_bins(cut, s.kept_top);
    for (int i = tid; i < k; i += kThreads) {
        const uint32_t kk = s.u.stage[Smem::kEmitKey + i];
        cslot[i] = lo + (int)s.u.stage[kEmitPos + i];
        ckey[i] = kk;
        atomicAdd(&s.khist[kept_bin(kk, bins)], 1u);
    }
    __syncthreads();
    for (int b = tid; b < kHistBins; b += kThreads) hist_out[b] = s.khist[b];
    if (tid == 0) {
        a.cand_count[rj] = k;
        a.cand_cut[rj] = (int)cut;
        a.cand_top[rj] = (int)s.kept_top;
    }
}

// Row r's exact top k straight from its scores [0, v), v > k, when the kept
// keys do not hold it: three radix passes of 12, 10 and 10 bits over the
// whole row, then the emission in rounds of kThreads positions, each round
// one scan.  Slow, and only for the rows whose cut missed.  The scan toggle comes
// by value (every caller returns right after), so the callers' own toggle
// stays in a register rather than in scratch memory.
template <typename Out>
__device__ void topk_row_streamed(TopkSmem& s, const float* row, int v, int k, const Out& out, int tog) {
    const int tid = threadIdx.x;
    uint32_t prefix = 0u, mask = 0u, kk = (uint32_t)k;
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = pass == 0 ? 20 : pass == 1 ? 10 : 0;
        const int nb = pass == 0 ? kBins0 : kBins1;
        __syncthreads();
        for (int i = tid; i < nb; i += kThreads) s.u.sel.hist[i] = 0u;
        __syncthreads();
        for (int i = tid; i < v; i += kThreads) {
            const uint32_t key = monotone_key(row[i]);
            if ((key & mask) == prefix) atomicAdd(&s.u.sel.hist[(key >> shift) & (uint32_t)(nb - 1)], 1u);
        }
        __syncthreads();
        if (pass == 0) find_digit<kBins0>(s, s.u.sel.hist, kk, tog);
        else find_digit<kBins1>(s, s.u.sel.hist, kk, tog);
        prefix |= s.sel_digit << shift;
        mask |= (uint32_t)(nb - 1) << shift;
        kk = s.sel_need;
    }
    const uint32_t thr = prefix, need_eq = kk;
    const bool eq_ok = thr != 0u;   // a zero threshold means NaN scores, reported elsewhere
    uint32_t taken_before = 0u, eq_before_round = 0u;
#pragma unroll 1
    for (int i0 = 0; i0 < v; i0 += kThreads) {
        const int i = i0 + tid;
        const uint32_t key = i < v ? monotone_key(row[i]) : 0u;
        const uint32_t gt = key > thr ? 1u : 0u;
        const uint32_t eq = (i < v && eq_ok && key == thr) ? 1u : 0u;
        uint32_t tot;
        const uint32_t both = scan2(s, (gt << 16) | eq, &tot, tog);
        const uint32_t eq_before = eq_before_round + (both & 0xFFFFu);
        const uint32_t eq_quota = need_eq > eq_before_round ? need_eq - eq_before_round : 0u;
        const bool take = gt || (eq && eq_before < need_eq);
        const uint32_t rank = taken_before + (both >> 16) + min(both & 0xFFFFu, eq_quota);
        if (take && rank < (uint32_t)k) out.put(rank, i);
        taken_before += (tot >> 16) + min(tot & 0xFFFFu, eq_quota);
        eq_before_round += tot & 0xFFFFu;
    }
}

// Merge pass: grid (n_rows).  The row's kept keys, split after split, form
// one list in slot order; its top k (the row's top k, see above) is emitted
// in that order.  The list is gathered into the staging buffer and selected
// with as few keys per thread (4, 8, 16 or 32) as its length allows.
template <int P, typename Out>
__device__ __forceinline__ void merge_select(const TopkArgs& a, TopkSmem& s, const int* off, int ns, int nc, int k,
                                             const Out& out_idx, int& tog) {
    const int tid = threadIdx.x;
    const int per = keys_per_thread(nc);
    const int base = tid * per;
    const int mine = max(0, min(per, nc - base));
    uint32_t key[P];
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const uint32_t x = s.u.stage[stage_index(min(base + i, kTopkMaxList - 1))];
        key[i] = i < mine ? x : 0u;
    }
    __syncthreads();
    for (int i = tid; i < kBins0; i += kThreads) s.h0[i] = 0u;
    __syncthreads();
    uint32_t thr, need;
    select_kth<P>(s, key, mine, nc, k, &thr, &need, tog);
    emit_to_lds<P>(s, key, base, thr, need, k, tog);
    __syncthreads();
    const size_t row_base = (size_t)blockIdx.x * ns * k;
    for (int i = tid; i < k; i += kThreads) {
        const int pos = min(max((int)s.u.stage[kEmitPos + i], 0), nc - 1);
        int lo_j = 0, hi_j = ns - 1;   // the split holding list position pos
        while (lo_j < hi_j) {
            const int mid = (lo_j + hi_j + 1) >> 1;
            if (off[mid] <= pos) lo_j = mid;
            else hi_j = mid - 1;
        }
        out_idx.put(i, a.cand_slot[row_base + (size_t)lo_j * k + (pos - off[lo_j])]);
    }
}

// Words of the staging buffer where the merge keeps the kept keys' slots
// (the keys sit at stage_index([0, nc)), which stays below kSlotBase when
// nc <= kSlotBase); the fast merge needs nc <= kSlotBase.
constexpr int kSlotBase = kTopkMaxList / 2;

template <int P, typename Out>
__device__ __forceinline__ void emit_slots(TopkSmem& s, const uint32_t (&key)[P], int base, int mine, uint32_t thr,
                                           uint32_t need_eq, int k, const Out& out_idx, int& tog);

// Keys of list positions [base, base + mine) of the staged candidates (keys
// at stage_index) into registers; per = keys_per_thread(nc).
template <int P>
__device__ __forceinline__ void load_staged(const TopkSmem& s, int nc, uint32_t (&key)[P], int& base, int& mine) {
    const int per = keys_per_thread(nc);
    base = (int)threadIdx.x * per;
    mine = max(0, min(per, nc - base));
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const uint32_t x = s.u.stage[stage_index(min(base + i, kSlotBase - 1))];
        key[i] = i < mine ? x : 0u;
    }
}

// The top k of the staged candidates, given a set of them (the keys for
// which inb holds, m <= 64 of them) that holds the k-th largest key as its
// need-th largest: one wavefront ranks the set exactly, then the selection
// is emitted in list order.
template <int P, typename InBin, typename Out>
__device__ __forceinline__ void rank_bin_emit(TopkSmem& s, const uint32_t (&key)[P], int base, int mine, int k,
                                              uint32_t need, uint32_t m, InBin inb, const Out& out_idx, int& tog) {
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    if (tid == 0) s.bcount = 0u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < P; ++i) {
        if (i < mine && inb(key[i])) {
            const uint32_t at = atomicAdd(&s.bcount, 1u);
            s.bkey[min(at, (uint32_t)kWave - 1)] = key[i];
        }
    }
    __syncthreads();
    if (tid < kWave) {
        const uint32_t mk = lane < (int)m ? s.bkey[lane] : 0u;
        uint32_t gt = 0, ge = 0;
        for (uint32_t j = 0; j < m; ++j) {
            const uint32_t x = s.bkey[j];
            gt += x > mk ? 1u : 0u;
            ge += x >= mk ? 1u : 0u;
        }
        if (lane < (int)m && gt < need && need <= ge) {
            s.sel_thr = mk;
            s.sel_need_eq = need - gt;
        }
    }
    __syncthreads();
    emit_slots<P>(s, key, base, mine, s.sel_thr, s.sel_need_eq, k, out_idx, tog);
}

// Fast merge, given the threshold bin b of the summed kept-key histograms
// (need = how many keys of bin b belong to the top k, m = keys in bin b <=
// 64): thread t holds list positions [t*per, t*per + per) of the kept keys
// (in the staging buffer, slots at kSlotBase); one wavefront ranks bin b's
// keys exactly and the selection is emitted in list order.
template <int P, typename Out>
__device__ __forceinline__ void merge_fast(TopkSmem& s, int nc, int k, uint32_t cut, const KeptBins& bins, int bstar,
                                           uint32_t need, uint32_t m, const Out& out_idx, int& tog) {
    uint32_t key[P];
    int base, mine;
    load_staged<P>(s, nc, key, base, mine);
    rank_bin_emit<P>(s, key, base, mine, k, need, m,
                     [&](uint32_t x) { return x >= cut && kept_bin(x, bins) == bstar; }, out_idx, tog);
}

// Emission as in the direct selection (keys above thr, then the first
// need_eq keys equal to it, in list order), each position's slot read from
// the staging buffer at kSlotBase.
template <int P, typename Out>
__device__ __forceinline__ void emit_slots(TopkSmem& s, const uint32_t (&key)[P], int base, int mine, uint32_t thr,
                                           uint32_t need_eq, int k, const Out& out_idx, int& tog) {
    uint32_t gtm = 0u, eqm = 0u;
#pragma unroll
    for (int i = 0; i < P; ++i) {
        gtm |= (i < mine && key[i] > thr ? 1u : 0u) << i;
        eqm |= (i < mine && key[i] == thr ? 1u : 0u) << i;
    }
    uint32_t tot;
    const uint32_t both = scan2(s, ((uint32_t)__popc(gtm) << 16) | (uint32_t)__popc(eqm), &tot, tog);
    const uint32_t eq_before = both & 0xFFFFu;
    uint32_t take_eq = min((uint32_t)__popc(eqm), need_eq > eq_before ? need_eq - eq_before : 0u);
    uint32_t tm = gtm;
    for (uint32_t em = eqm; take_eq > 0; --take_eq) {
        tm |= em & (0u - em);
        em &= em - 1u;
    }
    uint32_t rank = (both >> 16) + min(eq_before, need_eq);
    while (tm != 0u) {
        const int i = __ffs(tm) - 1;
        tm &= tm - 1u;
        if (rank < (uint32_t)k) out_idx.put(rank, (int32_t)s.u.stage[kSlotBase + base + i]);
        ++rank;
    }
}

// Merge pass: grid (n_rows).  The row's kept keys, split after split, form
// one list in slot order, gathered into the staging buffer; its top k is
// the row's top k (see above).  The splits' histograms, summed, give the bin
// of the k-th largest kept key, and one wavefront ranks that bin's keys;
// rows whose bin holds more than 64 keys (or without a cut) take the general
// selection instead.
template <bool kRows>
__global__ __launch_bounds__(kThreads) void topk_merge_kernel(TopkArgs a) {
    __shared__ TopkSmem s;
    __shared__ int off[kMaxSplits + 1];
    __shared__ uint32_t hsum[kHistBins];
    const int r = blockIdx.x;
    const int tid = threadIdx.x;
    const int k = a.top_k;
    const int ns = a.n_splits;
    const size_t rb = (size_t)r * ns;
    const int v = checked_vis(a, r);
    const auto out_idx = make_out<kRows>(a, s, r, v);
    const int want = min(v, k);
    if (tid == 0) a.topk_count[r] = want;
    // Everything this row needs goes out at once: the splits' counts, the
    // cut, the summed histograms, and the first kSpec entries of each
    // split's kept list (kept lists are usually that short).
    const int tps = kThreads / ns;            // threads per split for the speculative loads
    constexpr int kSpec = 8;
    const int sj = tid / tps, si = tid - sj * tps;
    int cnt_lane = 0;
    if (tid < kWave) cnt_lane = tid < ns ? min(max(a.cand_count[rb + tid], 0), k) : 0;
    const uint32_t cut = (uint32_t)a.cand_cut[rb];
    const uint32_t top = (uint32_t)a.cand_top[rb];
    uint32_t hs = 0u;
    if (tid < kHistBins) {
        const uint32_t* h = reinterpret_cast<const uint32_t*>(a.cand_hist) + rb * kHistBins + tid;
        for (int j = 0; j < ns; ++j) hs += h[(size_t)j * kHistBins];
    }
    uint32_t sk[kSpec];
    int32_t ss[kSpec];
#pragma unroll
    for (int q = 0; q < kSpec; ++q) {
        const int i = si + q * tps;
        const bool ok = sj < ns && i < k;
        const size_t at = (rb + (size_t)(ok ? sj : 0)) * k + (size_t)(ok ? i : 0);
        sk[q] = a.cand_key[at];
        ss[q] = a.cand_slot[at];
    }
    if (tid < kWave) {
        const uint32_t inc = wave_inclusive_scan((uint32_t)cnt_lane);
        if (tid < ns) off[tid + 1] = (int)inc;
        if (tid == 0) off[0] = 0;
    }
    if (tid < kHistBins) hsum[tid] = hs;
    __syncthreads();
    const int nc = off[ns];
    int tog = 0;
    if (nc < want) {
        // The cut kept fewer than k keys: select from the whole row.
        topk_row_streamed(s, a.scores + (size_t)r * a.score_stride, v, k, out_idx, tog);
        return;
    }
    // The kept keys (and, when they fit, their slots) into the staging
    // buffer at their list positions.
    const bool slots_fit = nc <= kSlotBase;
    if (sj < ns) {
        const int c = off[sj + 1] - off[sj];
#pragma unroll
        for (int q = 0; q < kSpec; ++q) {
            const int i = si + q * tps;
            if (i < c) {
                s.u.stage[stage_index(off[sj] + i)] = sk[q];
                if (slots_fit) s.u.stage[kSlotBase + off[sj] + i] = (uint32_t)ss[q];
            }
        }
        for (int i = si + kSpec * tps; i < c; i += tps) {   // longer kept lists
            s.u.stage[stage_index(off[sj] + i)] = a.cand_key[(rb + sj) * k + i];
            if (slots_fit) s.u.stage[kSlotBase + off[sj] + i] = (uint32_t)a.cand_slot[(rb + sj) * k + i];
        }
    }
    __syncthreads();
    if (nc <= k) {
        // Every kept key is selected (nc == want), in list order.
        for (int i = tid; i < nc; i += kThreads) {
            if (slots_fit) {
                out_idx.put(i, (int32_t)s.u.stage[kSlotBase + i]);
            } else {
                int lo_j = 0, hi_j = ns - 1;
                while (lo_j < hi_j) {
                    const int mid = (lo_j + hi_j + 1) >> 1;
                    if (off[mid] <= i) lo_j = mid;
                    else hi_j = mid - 1;
                }
                out_idx.put(i, a.cand_slot[(rb + lo_j) * k + (i - off[lo_j])]);
            }
        }
        pad_tail(out_idx, nc, k);
        return;
    }
    // Threshold bin: thread t holds bin kHistBins - 1 - t, so its exclusive
    // prefix counts the keys in the bins above.
    const uint32_t hb = tid < kHistBins ? hsum[kHistBins - 1 - tid] : 0u;
    if (tid == 0) {
        s.sel_digit = 0u;
        s.sel_need = 0u;
    }
    uint32_t total;
    const uint32_t above = scan2(s, hb, &total, tog);
    if (tid < kHistBins && above < (uint32_t)k && above + hb >= (uint32_t)k) {
        s.sel_digit = (uint32_t)(kHistBins - 1 - tid);
        s.sel_need = (uint32_t)k - above;
    }
    __syncthreads();
    const int bstar = min((int)s.sel_digit, kHistBins - 1);
    const uint32_t need = s.sel_need;
    const uint32_t m = hsum[bstar];
    if (cut != 0u && slots_fit && total == (uint32_t)nc && m <= (uint32_t)kWave && need >= 1u) {
        const KeptBins bins = kept_bins(cut, top);
        if (nc <= 4 * kThreads) merge_fast<4>(s, nc, k, cut, bins, bstar, need, m, out_idx, tog);
        else if (nc <= 8 * kThreads) merge_fast<8>(s, nc, k, cut, bins, bstar, need, m, out_idx, tog);
        else merge_fast<16>(s, nc, k, cut, bins, bstar, need, m, out_idx, tog);
        return;
    }
    if (nc <= 4 * kThreads) merge_select<4>(a, s, off, ns, nc, k, out_idx, tog);
    else if (nc <= 8 * kThreads) merge_select<8>(a, s, off, ns, nc, k, out_idx, tog);
    else if (nc <= 16 * kThreads) merge_select<16>(a, s, off, ns, nc, k, out_idx, tog);
    else merge_select<32>(a, s, off, ns, nc, k, out_idx, tog);
}


// Merge of the candidates that the decode indexer kept (dsa_index_topk):
// grid (n_rows).  Chunk j of the row kept every visible key at or above its
// own cut c_j (up to cand_cap of them, else count -1).  With C = max_j c_j,
// every key of the row at or above C is a candidate; so when at least k
// candidates are >= C, the row's k-th largest key T is >= C, every key >= T
// is a candidate, and the top k of the candidates (in slot order, ties to
// the lower slot) is the row's top k.  Rows where that does not hold, or
// whose candidates do not fit the staging buffer, are selected from their
// scores.  Candidates at or above C are binned by their top 16 key bits
// relative to C; the bin of the k-th largest is ranked by one wavefront when
// it holds at most 64 keys, else the general selection runs over all
// candidates.
constexpr int kMaxCutSplits = 1024;

// The bin of 512 (scanned from the largest) that holds the need-th largest
// counted key: s.sel_digit, and s.sel_need = need minus the keys in the bins
// above (0 and 0 when fewer than need keys are counted); *total = all counted.
__device__ __forceinline__ void find_bin512(TopkSmem& s, const uint32_t* hist, uint32_t need, uint32_t* total,
                                            int& tog) {
    const int tid = threadIdx.x;
    const uint32_t h = tid < kHistBins ? hist[kHistBins - 1 - tid] : 0u;
    if (tid == 0) {
        s.sel_digit = 0u;
        s.sel_need = 0u;
    }
    const uint32_t above = scan2(s, h, total, tog);
    if (tid < kHistBins && above < need && above + h >= need) {
        s.sel_digit = (uint32_t)(kHistBins - 1 - tid);
        s.sel_need = need - above;
    }
    __syncthreads();
}

__global__ __launch_bounds__(kThreads) void topk_merge_cuts_kernel(TopkArgs a) {
    __shared__ TopkSmem s;
    __shared__ int off[kMaxCutSplits + 1];
    __shared__ uint32_t kmax_s;   // the largest candidate
    const int r = blockIdx.x;
    const int tid = threadIdx.x;
    const int k = a.top_k;
    const int ns = a.n_splits;
    const int cap = a.cand_cap;
    const size_t rb = (size_t)r * ns;
    const int v = checked_vis(a, r);
    const auto out_idx = make_out<false>(a, s, r, v);
    if (tid == 0) a.topk_count[r] = min(v, k);
    if (v <= k) {
        for (int i = tid; i < v; i += kThreads) out_idx.put(i, i);
        pad_tail(out_idx, v, k);
        return;
    }
    // Counts, cuts and the first kSpec candidates of every chunk go out at
    // once (kept lists are usually that short).
    const int tps = kThreads / ns;   // threads per chunk for the speculative loads (ns <= kThreads)
    constexpr int kSpec = 8;
    const int sj = tid / tps, si = tid - sj * tps;
    int cnt = 0;
    uint32_t cut = 0u;
    if (tid < ns) {
        cnt = a.cand_count[rb + tid];
        cut = (uint32_t)a.cand_cut[rb + tid];
    }
    uint32_t sk[kSpec];
    int32_t ss[kSpec];
#pragma unroll
    for (int q = 0; q < kSpec; ++q) {
        const int i = si + q * tps;
        const bool ok = sj < ns && i < cap;
        const size_t at = (rb + (size_t)(ok ? sj : 0)) * cap + (size_t)(ok ? i : 0);
        sk[q] = a.cand_key[at];
        ss[q] = a.cand_slot[at];
    }
    for (int b = tid; b < kHistBins; b += kThreads) s.khist[b] = 0u;
    for (int b = tid; b < kBins0; b += kThreads) s.h0[b] = 0u;
    if (tid == 0) {
        s.sel_thr = 0u;   // C
        s.bcount = 0u;    // a chunk overflowed
        kmax_s = 0u;
    }
    __syncthreads();
    const bool over = tid < ns && (cnt < 0 || cnt > cap);
    if (tid < ns) atomicMax(&s.sel_thr, cut);
    if (over) s.bcount = 1u;
    int tog = 0;
    uint32_t nc_u;
    const uint32_t ex = scan2(s, over ? 0u : (uint32_t)max(cnt, 0), &nc_u, tog);
    if (tid < ns) off[tid] = (int)ex;
    if (tid == 0) off[ns] = (int)nc_u;
    const uint32_t C = s.sel_thr;
    const bool fall = s.bcount != 0u || nc_u < (uint32_t)k || nc_u > (uint32_t)kSlotBase;
    __syncthreads();
    const float* row = a.scores + (size_t)r * a.score_stride;
    if (fall) {
        topk_row_streamed(s, row, v, k, out_idx, tog);
        return;
    }
    const int nc = (int)nc_u;
    // Candidates (keys at stage_index, slots at kSlotBase) in list order, and
    // the largest of them.
    uint32_t kmax = 0u;
    auto put = [&](int at, uint32_t key, int32_t slot) {
        s.u.stage[stage_index(at)] = key;
        s.u.stage[kSlotBase + at] = (uint32_t)slot;
        kmax = max(kmax, key);
    };
    if (sj < ns) {
        const int o = off[sj];
        const int c = off[sj + 1] - o;
#pragma unroll
        for (int q = 0; q < kSpec; ++q) {
            const int i = si + q * tps;
            if (i < c) put(o + i, sk[q], ss[q]);
        }
        for (int i = si + kSpec * tps; i < c; i += tps)
            put(o + i, a.cand_key[(rb + sj) * cap + i], a.cand_slot[(rb + sj) * cap + i]);
    }
    kmax = wave_max_u32(kmax);
    if ((tid & (kWave - 1)) == 0) atomicMax(&kmax_s, kmax);
    __syncthreads();
    // Keys >= C in 512 bins of 2^s1 key values from C up, s1 the smallest
    // shift that fits the largest candidate; the bin of the k-th largest;
    // inside it, if it holds more than 64 keys, 512 bins of 2^s2 values.
    const uint32_t range = kmax_s >= C ? kmax_s - C : 0u;
    const int s1 = range == 0u ? 0 : max(0, 32 - __clz(range) - 9);
    const int s2 = max(0, s1 - 9);
    auto select = [&](auto pc) {
        constexpr int P = decltype(pc)::value;
        uint32_t key[P];
        int base, mine;
        load_staged<P>(s, nc, key, base, mine);
        auto in_b0 = [&](uint32_t x) { return x >= C; };
#pragma unroll
        for (int i = 0; i < P; ++i)
            if (i < mine && in_b0(key[i])) atomicAdd(&s.khist[(key[i] - C) >> s1], 1u);
        __syncthreads();
        uint32_t ge_c;
        find_bin512(s, s.khist, (uint32_t)k, &ge_c, tog);
        if (ge_c < (uint32_t)k) {   // fewer than k candidates >= C: the row's top k may lie below C
            topk_row_streamed(s, row, v, k, out_idx, tog);
            return;
        }
        if (nc == k) {   // every candidate is >= C and selected
            for (int i = tid; i < nc; i += kThreads) out_idx.put(i, (int32_t)s.u.stage[kSlotBase + i]);
            return;
        }
        const uint32_t bstar = s.sel_digit, need = s.sel_need, m = s.khist[bstar];
        auto in_b = [&](uint32_t x) { return x >= C && ((x - C) >> s1) == bstar; };
        if (m <= (uint32_t)kWave) {
            rank_bin_emit<P>(s, key, base, mine, k, need, m, in_b, out_idx, tog);
            return;
        }
        if (s1 > 0) {
            // s.h0 is still zero.
#pragma unroll
            for (int i = 0; i < P; ++i)
                if (i < mine && in_b(key[i])) atomicAdd(&s.h0[((key[i] - C) >> s2) & (kHistBins - 1)], 1u);
            __syncthreads();
            uint32_t tot;
            find_bin512(s, s.h0, need, &tot, tog);
            const uint32_t sb = s.sel_digit, need2 = s.sel_need, m2 = s.h0[sb];
            if (tot == m && m2 <= (uint32_t)kWave) {
                rank_bin_emit<P>(s, key, base, mine, k, need2, m2,
                                 [&](uint32_t x) { return in_b(x) && (((x - C) >> s2) & (kHistBins - 1)) == sb; },
                                 out_idx, tog);
                return;
            }
            for (int b = tid; b < kHistBins; b += kThreads) s.h0[b] = 0u;
        }
        // General selection over every candidate (many equal keys).
        __syncthreads();   // its histograms overwrite the staged keys (not the slots); s.h0 is zero
        uint32_t thr, need_eq;
        select_kth<P>(s, key, mine, nc, k, &thr, &need_eq, tog);
        emit_slots<P>(s, key, base, mine, thr, need_eq, k, out_idx, tog);
    };
    if (nc <= 4 * kThreads) select(std::integral_constant<int, 4>{});
    else if (nc <= 8 * kThreads) select(std::integral_constant<int, 8>{});
    else select(std::integral_constant<int, 16>{});
}
}  // namespace

namespace {

// Keys per thread a launch is compiled for: the smallest of 4, 8, 16, 32
// that holds a list of up to `longest` entries.
int keys_class(int64_t longest) {
    const int64_t per = (longest + 4 * kThreads - 1) / (4 * kThreads) * 4;
    return per <= 4 ? 4 : per <= 8 ? 8 : per <= 16 ? 16 : 32;
}

template <typename F>
hipError_t by_class(int cls, F f) {
    switch (cls) {
        case 4: return f(std::integral_constant<int, 4>{});
        case 8: return f(std::integral_constant<int, 8>{});
        case 16: return f(std::integral_constant<int, 16>{});
        default: return f(std::integral_constant<int, 32>{});
    }
}

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t stream) {
    if (a.n_rows == 0) return hipSuccess;
    // Longest split: ceil(score_stride / n_splits) rounded up to whole chunks
    // (row_vis <= score_stride is checked on the device).
    const int64_t split_max = (((int64_t)a.score_stride + a.n_splits - 1) / a.n_splits + 3) & ~int64_t{3};
    if (a.n_splits == 1) {
        return by_class(keys_class(split_max), [&](auto pc) {
            if (a.topk_rows != nullptr)
                topk_direct_kernel<decltype(pc)::value, true><<<dim3(1, a.n_rows), kThreads, 0, stream>>>(a);
            else
                topk_direct_kernel<decltype(pc)::value, false><<<dim3(1, a.n_rows), kThreads, 0, stream>>>(a);
            return hipGetLastError();
        });
    }
    // The compact filter layout (two workgroups per CU) when there are more
    // workgroups than CUs to run, every split is a whole 16-byte aligned run
    // of at most 16 keys a thread (rows 16-byte aligned, score_stride a
    // multiple of 4: the splits start on multiples of 4) and k fits it.
    const bool compact = (int64_t)a.n_splits * a.n_rows > kComputeUnits && keys_class(split_max) <= 16 &&
                         a.top_k <= TopkSmemCompact::kMaxK &&
                         (reinterpret_cast<uintptr_t>(a.scores) & 15) == 0 && (a.score_stride & 3) == 0;
    hipError_t e = by_class(keys_class(split_max), [&](auto pc) {
        constexpr int P = decltype(pc)::value;
        if constexpr (P <= 16) {
            if (compact) {
                topk_filter_kernel<P, true><<<dim3(a.n_splits, a.n_rows), kThreads, 0, stream>>>(a);
                return hipGetLastError();
            }
        }
        topk_filter_kernel<P, false><<<dim3(a.n_splits, a.n_rows), kThreads, 0, stream>>>(a);
        return hipGetLastError();
    });
    if (e != hipSuccess) return e;
    if (a.topk_rows != nullptr) topk_merge_kernel<true><<<a.n_rows, kThreads, 0, stream>>>(a);
    else topk_merge_kernel<false><<<a.n_rows, kThreads, 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_topk_merge_cuts(const TopkArgs& a, hipStream_t stream) {
    if (a.n_rows == 0) return hipSuccess;
    if (a.n_splits < 1 || a.n_splits > kMaxCutSplits || a.cand_cap < 1) return hipErrorInvalidValue;
    topk_merge_cuts_kernel<<<a.n_rows, kThreads, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace dsa
