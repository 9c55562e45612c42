// Split-K sparse absorbed-MLA decode on gfx950.
//
// A workgroup (four wavefronts per 16 heads) owns one (row, split): the
// split's entries of the row's selected list, walked in tiles of 64 tokens
// with an online softmax.  Per tile:
//   gather  the 64 selected 576-byte fp8 rows through the block table into
//           LDS (rows padded to 592 bytes), with their fp32 scales;
//   QK      on fp8 matrix cores: the keys' codes as stored (A, M = tokens)
//           against the bf16 query split into two E4M3 terms with one
//           power-of-two scale per head (B, N = heads), four 128-deep steps
//           over the 512 latent values and two 32-deep steps over the 64
//           rope values per term, on two accumulator chains.  The query
//           terms stay in registers for the whole split.  Wavefront w owns
//           head block w % HB and token block w / HB (16 tokens);
//   softmax a lane holds 4 tokens of one head, so the per-head maximum and
//           sum reduce in-lane and then across the four 16-lane rows with two
//           permlane swaps; P' = 2^(l - m) * token scale (logits in base-2
//           units) goes to LDS in bf16, 4 tokens per 8-byte store, against
//           the running max m of the tiles before, which every wavefront
//           holds; the tile maxima per head go through LDS with P', and the
//           output is rescaled when the running max moves (the loop has the
//           details);
//   PV      wavefront w owns output columns [CW w, CW w + CW) for all heads:
//           A = P' (heads x tokens), B = the fp8 rows read transposed by
//           ds_read_b64_tr_b8 (8 tokens of one column per lane), converted
//           exactly to bf16.
// The value rows are the first 512 entries of the same rows (absorbed MLA),
// so a tile is read from HBM once for both products.
//
// Latency hiding: the bf16 query goes out first, as LDS-direct loads into
// the last tile buffer (free until the first tile's barrier); a split's
// range of the selected list depends only on top_k, so its entries are
// loaded together with the row's metadata; the block table is then walked
// once for the whole split (slot -> page -> physical row, kept in LDS) and
// the first gathers go out right after it.  Tiles are gathered by LDS-direct loads
// (global_load_lds_dwordx4: each lane's 16 bytes land at the wavefront's LDS
// base + 16 * lane), which need no registers: with four tile buffers, three
// tiles are in flight while the fourth is computed.  Each wavefront waits
// with an explicit count for its own loads of the tile it needs next, and
// barriers order LDS only, so loads of later tiles stay in flight.
//
// LDS banking (gfx950: 16-byte reads are served 32 lanes at a time, 8-byte
// accesses 64 lanes at a time, over 512 bytes of banks): rows are 592 bytes
// apart (37 chunks of 16), so 16 consecutive rows fall on 16 distinct odd
// multiples of 16 bytes and the next 16 rows on the other half.  QK's K
// order therefore gives lane groups g = 0..3 the 16-byte chunks
// c + {0, 16, 8, 24} of a row: the two groups served together differ by
// 256 bytes and never collide.  Lane group g reads chunks
// {2p + h + 16 (g & 1) + 8 (g >> 1) : h < 2} (its 32 codes of 128-deep step
// p) and 32 + g (its 16 rope codes); the query takes the same element
// positions, so the sums are the plain dot products.  P' is laid
// out as [token group of 8][head][8 tokens] with 768 bytes per token group,
// which makes both its 8-byte stores and its 16-byte A-operand reads
// conflict-free.  ds_read_b64_tr_b8 over 32 rows of 592 bytes is
// conflict-free as it is.
#include "device_common.h"
#include "launch.h"
#include "query_quant.h"

namespace dsa {

namespace {

constexpr int kT = 64;            // tokens per tile
constexpr int kRowBytes = 576;    // elements of a query head / code bytes of a cache row
constexpr int kKvRow = 640;       // bytes of a cache row: 576 codes, fp32 scale at 576, pad
constexpr int kScaleAt = 576;     // byte of the scale within a (cache or LDS) row
constexpr int kXStride = 592;     // LDS bytes per gathered row
constexpr int kPGroup = 768;      // LDS bytes per group of 8 tokens of P' (up to 32 heads x 16 B + pad)
constexpr int kDv = 512;
constexpr int kRowChunks = kXStride / 16;        // 37: 36 data chunks + 1 pad chunk
constexpr int kTileChunks = kT * kRowChunks;       // 2368 chunks of 16 bytes
constexpr int kDmaInsts = kTileChunks / kWave;     // 37 wavefront-wide LDS-direct loads
constexpr float kSlack = 11.5f;  // P = 2^(l - running max) < 2^11.5 (about e^8) without the exchange (see the loop)
constexpr float kLazy = 8.0f;    // the running max moves only when a tile's exceeds it by more (base 2)
constexpr float kLog2e = 1.44269504088896341f;
constexpr float kLn2 = 0.693147180559945309f;

typedef __attribute__((address_space(3))) v2i lds_v2i;
typedef __attribute__((address_space(3))) void lds_void;

// LDS-direct loads of one tile: the first 592 bytes (37 chunks: codes,
// scale, 12 pad bytes) of each of the 64 rows, 37 loads of 64 chunks that go
// round-robin over the NW wavefronts (load j by wavefront j % NW).
template <int NW>
struct DmaPlan {
    static constexpr int kPer = (kDmaInsts + NW - 1) / NW;   // loads per wavefront, at most
    static constexpr int count(int w) { return (kDmaInsts - w + NW - 1) / NW; }
};
static_assert(DmaPlan<4>::count(0) == 10 && DmaPlan<4>::count(1) == 9 && DmaPlan<4>::count(3) == 9,
              "per-wavefront load counts, 4 wavefronts");
static_assert(DmaPlan<8>::count(0) == 5 && DmaPlan<8>::count(4) == 5 && DmaPlan<8>::count(5) == 4 &&
              DmaPlan<8>::count(7) == 4, "per-wavefront load counts, 8 wavefronts");

// s_waitcnt immediate for "at most n vector-memory operations outstanding"
// (expcnt and lgkmcnt left at their no-wait maxima).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Wait until at most this wavefront's loads of the `younger` tiles issued
// after the one needed now are outstanding (0 <= younger <= 2).  A
// wavefront issues kPer or kPer - 1 loads per tile.
template <int NW, int N>
__device__ __forceinline__ void wait_tiles_n(int wv) {
    constexpr int kPer = DmaPlan<NW>::kPer;
    if (DmaPlan<NW>::count(wv) == kPer) wait_vm<N * kPer>();
    else wait_vm<N * (kPer - 1)>();
}
template <int NW>
__device__ __forceinline__ void wait_tiles(int wv, int younger) {
    if (younger <= 0) wait_vm<0>();
    else if (younger == 1) wait_tiles_n<NW, 1>(wv);
    else wait_tiles_n<NW, 2>(wv);
}

// NB tile buffers: 4 (three tiles in flight while one is computed) when a
// split holds at most 1024 entries, else 2, which leaves LDS for the physical
// rows of a split of up to top_k = 8192 entries.
template <int NB>
struct MlaGeom {
    static_assert(NB == 2 || NB == 4, "tile buffers");
    static constexpr int kRowsCap = NB == 4 ? 1024 : kTopkMaxK;  // split entries kept in LDS
};

// 16-byte chunk of a 592-byte LDS row that lane group g reads for half h
// of the 128-wide K step p (see the banking note above).
__device__ __forceinline__ int qk_chunk(int p, int h, int g) {
    return 2 * p + h + ((g & 1) << 4) + ((g >> 1) << 3);
}

// kNt: the tiles are gathered with the non-temporal hint (rows that no
// other workgroup reads again).
template <int HB, int NB, bool kNt>
__global__ __launch_bounds__(256 * HB) void sparse_mla_kernel(MlaArgs a) {
    constexpr int H = 16 * HB;
    constexpr int NW = 4 * HB;          // wavefronts: one per (token block, head block) in QK
    constexpr int NT = 64 * NW;
    constexpr int CW = kDv / NW;        // output columns per wavefront in PV
    constexpr int NCB = CW / 16;
    constexpr int kDmaPer = DmaPlan<NW>::kPer;
    constexpr int kRowsCap = MlaGeom<NB>::kRowsCap;
    constexpr int kTileBytes = kT * kXStride;
    // Tile buffers; the loads into them are issued as inline assembly and
    // waited for with explicit counts, so the compiler never waits for them.
    __shared__ __attribute__((aligned(16))) uint8_t s_x[NB][kTileBytes];
    __shared__ __attribute__((aligned(16))) uint8_t s_p[8 * kPGroup];
    __shared__ int32_t s_rows[kRowsCap];
    __shared__ __attribute__((aligned(16))) float s_red[H][4];           // per-head values of the wavefronts
    // Rescale factors per head, with a flag per head block (some factor is
    // not 1): pending ones (a tile's, applied before the next tile's PV) and
    // the exact path's (applied before the same tile's PV).
    __shared__ __attribute__((aligned(16))) float s_alpha[H];
    __shared__ __attribute__((aligned(16))) float s_alpha_x[H];
    __shared__ __attribute__((aligned(16))) float s_m[H];
    __shared__ int s_moved[HB];
    __shared__ int s_moved_x[HB];
    __shared__ __attribute__((aligned(16))) int s_big[NW];   // per wavefront: a logit far above the running max
    __shared__ int s_bad[NW];   // per wavefront: an entry of the split is invalid
    // The bf16 query is staged in the last tile buffer: head h at row h,
    // kQRow bytes apart (72 chunks of 16 bytes and a pad chunk).
    constexpr int kQRow = 2 * kRowBytes + 16;
    constexpr int kQChunks = kQRow / 16;
    static_assert(H * kQRow <= kTileBytes, "the query fits one tile buffer");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar branches
    if (tid < HB) s_moved[tid] = 0;   // no rescale pending before the first tile (barriers follow)
    const int nn = lane & 15;
    const int g = lane >> 4;
    const int hb = wv % HB;         // head block of this wavefront in QK
    const int tbk = wv / HB;        // its token block: tokens [16 tbk, 16 tbk + 16) of a tile
    const int ns = a.n_splits;
    // Chains on XCDs: workgroup L runs on XCD L % 8 (the dispatcher deals
    // workgroups out to the XCDs in turn); XCD x takes chains x, x + 8, ...
    // one after the other, all (row, split) units of a chain in a row.  A
    // chain is `chain` consecutive rows sharing one list (one row when
    // nothing is shared), so the chain's shared rows and each row's query,
    // which every split of the row loads, are fetched into that XCD's L2
    // once.  Padding units past the last chain do nothing.
    int r, sp;
    {
        const int L = blockIdx.x;
        const int per_chain = a.chain * ns;
        const int j = L >> 3;
        const int c = ((j / per_chain) << 3) | (L & 7);
        const int u = j % per_chain;
        if (c * a.chain >= a.n_rows) return;
        r = c * a.chain + u / ns;
        sp = u % ns;
    }

    // The bf16 query of the row, gathered like a tile (lane i of load j
    // fills chunk 64 j + i of the staging rows; the pad chunk rereads chunk
    // 0 of its row).  These are the oldest loads of every wavefront, so the
    // waits for any later load cover them.
    {
        const uint8_t* qrow = reinterpret_cast<const uint8_t*>(a.q + (size_t)r * H * kRowBytes);
        const uint32_t xl = lds_offset(s_x[NB - 1]);
        constexpr int kQInsts = (H * kQChunks + kWave - 1) / kWave;
        for (int j = wv; j < kQInsts; j += NW) {
            const int c = min(64 * j + lane, H * kQChunks - 1);
            const int t = c / kQChunks, part = c - t * kQChunks;
            lds_dma16(qrow + (size_t)t * (2 * kRowBytes) + (part < kQChunks - 1 ? part * 16 : 0), xl + j * 1024);
        }
    }

    // Row metadata (uniform loads) and the split's range of the selected
    // list.  The range depends only on top_k, so the list entries can be
    // loaded together with the metadata.
    // rows: the list holds physical rows (no request, no block table).
    const bool rows = a.topk_rows != nullptr;
    const int b_raw = rows ? 0 : a.row_req[r];
    const int v_raw = a.row_vis[r];
    // The list this row attends: its own, or the shared one row_list names.
    const int list_raw = a.row_list != nullptr ? a.row_list[r] : r;
    const bool list_ok = list_raw >= 0 && list_raw < a.n_lists;
    const int list = list_ok ? list_raw : 0;
    const int c_raw = a.topk_count[list];
    const int chunk = (a.top_k + ns - 1) / ns;
    const int lo = min(a.top_k, sp * chunk);
    const int hi_list = min(a.top_k, lo + chunk);
    const int32_t* sel = (rows ? a.topk_rows : a.topk_idx) + (size_t)list * a.top_k;

    // First batch of list entries (8 per thread), issued before anything
    // else; indexes are clamped into the list.
    constexpr int kBatch = 8 * NT;
    int slot[8];
    auto load_slots = [&](int base) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (base + NT * u < hi_list) slot[u] = sel[min(base + NT * u + tid, hi_list - 1)];
    };
    load_slots(lo);

    bool ok = (rows || (b_raw >= 0 && b_raw < a.batch && v_raw <= a.max_pages * a.page_size)) && v_raw >= 0 &&
              list_ok;
    if (!ok && tid == 0) flag(a.status, DSA_DEV_ROW_RANGE);
    if (ok && (c_raw < 0 || c_raw > a.top_k || c_raw > v_raw)) {
        if (tid == 0) flag(a.status, DSA_DEV_TOPK_OOB);
        ok = false;
    }
    const int vis = ok ? v_raw : 0;
    const int hi = ok ? min(hi_list, c_raw) : lo;    // entries [lo, hi) of the list are ours
    const int n_tiles = hi > lo ? (hi - lo + kT - 1) / kT : 0;
    const int32_t* pt = a.page_table + (size_t)(ok ? b_raw : 0) * a.max_pages;
    const int pmask = a.page_size - 1;
    // Block-table walk for the whole split, once: selected slot -> page ->
    // physical row, kept in LDS (-1 for invalid entries, which are reported).
    // All page-table loads of a batch go out before any result is used;
    // their indexes are clamped into the table so that they need no branch,
    // and validity is decided afterwards.
    bool bad = false;
    const int64_t pool_rows = (int64_t)a.num_pages * a.page_size;
    auto walk = [&](int base) {
        if (rows) {   // physical rows given: -1 (left out by the top-k) stays out quietly
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int e = base + NT * u + tid;
                if (base + NT * u < hi && e < hi) {
                    int32_t row = slot[u];
                    if (row < -1 || (int64_t)row >= pool_rows) flag(a.status, DSA_DEV_TOPK_OOB);
                    if (row < 0 || (int64_t)row >= pool_rows) row = -1;
                    bad |= row < 0;
                    s_rows[e - lo] = row;
                }
            }
            return;
        }
        int page[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (base + NT * u < hi) page[u] = pt[min(max(slot[u], 0) >> a.log2_page, a.max_pages - 1)];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int e = base + NT * u + tid;
            if (base + NT * u < hi && e < hi) {
                int32_t row = -1;
                if (slot[u] < 0 || slot[u] >= vis) {
                    flag(a.status, DSA_DEV_TOPK_OOB);
                } else if (page[u] < 0 || page[u] >= a.num_pages) {
                    flag(a.status, DSA_DEV_PAGE_OOB);
                } else {
                    row = page[u] * a.page_size + (slot[u] & pmask);
                }
                bad |= row < 0;
                s_rows[e - lo] = row;
            }
        }
    };
    walk(lo);
    if constexpr (NB == 2) {   // splits longer than one batch
        for (int base = lo + kBatch; base < hi; base += kBatch) {
            load_slots(base);
            walk(base);
        }
    }
    static_assert(MlaGeom<4>::kRowsCap <= 2048, "a four-buffer split is one batch (kBatch >= 2048)");
    // The row list padded to whole tiles with row 0 (n_tiles * kT <= kRowsCap:
    // a split holds at most kRowsCap entries and kRowsCap is a multiple of
    // kT), so the gathers need no bound check; dead rows are zeroed in LDS
    // before they are used.
    static_assert(MlaGeom<4>::kRowsCap % kT == 0 && MlaGeom<2>::kRowsCap % kT == 0, "whole tiles");
    for (int e = hi - lo + tid; e < n_tiles * kT; e += NT) s_rows[e] = 0;
    const bool wave_bad = __ballot(bad) != 0ull;
    if (lane == 0) s_bad[wv] = wave_bad;
    // Every load of the wavefronts done (the query included, which the
    // compiler does not track), so the query is in LDS after the barrier and
    // no load the compiler tracks is outstanding once the gathers go out.
    wait_vm<0>();
    __syncthreads();
    bool any_bad = false;
#pragma unroll
    for (int w = 0; w < NW; ++w) any_bad |= s_bad[w] != 0;

    const float cq = a.sm_scale;

    // Row of tile-local token t of the tile starting at split entry `base`.
    // The read is clamped into the array and its value discarded past the end,
    // so it needs no branch.
    auto row_at = [&](int base, int t) -> int32_t {
        const int32_t v = s_rows[min(base + t - lo, kRowsCap - 1)];
        return base + t < hi ? v : -1;
    };

    // LDS-direct gather.  Wavefront wv issues the loads j = wv, wv+NW, ... of
    // a tile; lane i of load j fills tile chunk 64j + i, i.e. row t =
    // chunk / 37, part chunk % 37 (part 36 holds the scale).  Dead rows read
    // row 0 of page 0 and are zeroed afterwards.  All row ids are read from
    // LDS before the first load is issued.
    // Tile row and byte offset of lane `lane` in load j (recomputed at each
    // issue rather than kept in registers).
    auto dma_geo = [&](int j, int& t, int& off) {
        const int c = 64 * j + lane;
        t = c / kRowChunks;
        off = (c - t * kRowChunks) * 16;
    };
    auto gather = [&](const void* src, uint32_t lds) {
        if constexpr (kNt) lds_dma16_nt(src, lds);
        else lds_dma16(src, lds);
    };
    auto issue = [&](int buf, int base) {
        const uint32_t xl = lds_offset(s_x[buf]);
        const int32_t* tile_rows = s_rows + (base - lo);   // padded to whole tiles
        int32_t row[kDmaPer], off[kDmaPer];
#pragma unroll
        for (int jj = 0; jj < kDmaPer; ++jj) {
            int t;
            dma_geo(min(wv + NW * jj, kDmaInsts - 1), t, off[jj]);
            row[jj] = max(tile_rows[t], 0);
        }
        // Loads j = wv + NW jj; the last one exists only while j < 37.
#pragma unroll
        for (int jj = 0; jj < kDmaPer - 1; ++jj)
            gather(a.kv_cache + (size_t)row[jj] * kKvRow + off[jj], xl + (wv + NW * jj) * 1024);
        if (wv + NW * (kDmaPer - 1) < kDmaInsts)
            gather(a.kv_cache + (size_t)row[kDmaPer - 1] * kKvRow + off[kDmaPer - 1],
                      xl + (wv + NW * (kDmaPer - 1)) * 1024);
    };
    // Tiles with dead rows (past the split's end, or invalid entries) have
    // those rows zeroed, so no stale or garbage bytes reach the PV product.
    auto zero_dead = [&](uint8_t* xb, int base) {
        for (int c = tid; c < kT * kRowChunks; c += NT) {
            const int t = c / kRowChunks, part = c - t * kRowChunks;
            if (row_at(base, t) < 0) *reinterpret_cast<uint4*>(xb + t * kXStride + part * 16) = uint4{0u, 0u, 0u, 0u};
        }
    };

    // Prologue: the first NB-1 tiles in flight.
#pragma unroll
    for (int j = 0; j < NB - 1; ++j)
        if (j < n_tiles) issue(j, lo + j * kT);

    // The query as two E4M3 terms, while those tiles load.  Head h's bf16
    // values q (exact fp32) are scaled by 2^-e_h, e_h the smallest exponent
    // with max|q| <= 448 * 2^e_h (the indexer query's rule); hi = RNE(q 2^-e)
    // in E4M3, lo = RNE(q 2^-e - hi).  A bf16 value has 8 significant bits and
    // hi keeps the top 4, so lo is exact except where it falls below E4M3's
    // smallest subnormal (values under 2^-7 of the head's largest, where the
    // lost part is at most 2^-10 of the scaled unit): q . k = 2^e (hi . k +
    // lo . k) with every fp8 product exact, on fp8 matrix cores with the
    // keys' codes as they are stored.  Sixteen threads per head (36 values
    // each) split the query in place in its staging buffer: each head's row
    // becomes 576 hi codes then 576 lo codes.
    __shared__ float s_qs[H];   // 2^e per head
    {
        constexpr int kPart = kRowBytes / 16;   // 36 values per thread
        static_assert(NT == 16 * H, "sixteen threads per head");
        const int qh = tid >> 4, part = tid & 15;
        uint8_t* hrow = s_x[NB - 1] + qh * kQRow;
        float v[kPart];
        float amax = 0.0f;
#pragma unroll
        for (int k = 0; k < kPart / 4; ++k) {
            const uint2 w = *reinterpret_cast<const uint2*>(hrow + 2 * (kPart * part + 4 * k));
            v[4 * k + 0] = __uint_as_float(w.x << 16);
            v[4 * k + 1] = __uint_as_float(w.x & 0xFFFF0000u);
            v[4 * k + 2] = __uint_as_float(w.y << 16);
            v[4 * k + 3] = __uint_as_float(w.y & 0xFFFF0000u);
        }
#pragma unroll
        for (int k = 0; k < kPart; ++k) amax = fmaxf(amax, fabsf(v[k]));
        amax = row16_max(amax);   // the head's sixteen threads are one 16-lane row
        const int e = idx_q_exponent(amax);
        uint32_t hw[kPart / 4], lw[kPart / 4];
#pragma unroll
        for (int k = 0; k < kPart / 4; ++k) {
            float y[4], rr[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) y[j] = __builtin_amdgcn_ldexpf(v[4 * k + j], -e);
            const int h01 = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
            const int h23 = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], h01, true);
            const auto d01 = __builtin_amdgcn_cvt_pk_f32_fp8(h23, false);
            const auto d23 = __builtin_amdgcn_cvt_pk_f32_fp8(h23, true);
            rr[0] = y[0] - d01[0];
            rr[1] = y[1] - d01[1];
            rr[2] = y[2] - d23[0];
            rr[3] = y[3] - d23[1];
            const int l01 = __builtin_amdgcn_cvt_pk_fp8_f32(rr[0], rr[1], 0, false);
            hw[k] = (uint32_t)h23;
            lw[k] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(rr[2], rr[3], l01, true);
        }
        // LDS-only barriers: the tiles just issued stay in flight (a
        // __syncthreads() would wait for all of them).
        lds_sync();   // every bf16 value of the buffer has been read
#pragma unroll
        for (int k = 0; k < kPart / 4; ++k) {
            *reinterpret_cast<uint32_t*>(hrow + kPart * part + 4 * k) = hw[k];
            *reinterpret_cast<uint32_t*>(hrow + kRowBytes + kPart * part + 4 * k) = lw[k];
        }
        if (part == 0) s_qs[qh] = __builtin_amdgcn_ldexpf(1.0f, e);
        lds_sync();
    }
    // This lane's operands (head 16 hb + nn, lane group g) for the whole
    // split: for 128-element MFMA step m the 32 codes at elements
    // [16 c, 16 c + 32), c = qk_chunk(m, 0, g), the same 32 bytes of every
    // key row; for the rope, the 16 codes [512 + 16 g, +16) as two 8-code
    // steps.  Both terms.
    v8i qh8[4], ql8[4];
    v4i qrh, qrl;
    float qsc;
    {
        const uint8_t* hr = s_x[NB - 1] + (16 * hb + nn) * kQRow;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int c = qk_chunk(m, 0, g);
            const v4i h0 = *reinterpret_cast<const v4i*>(hr + 16 * c);
            const v4i h1 = *reinterpret_cast<const v4i*>(hr + 16 * c + 16);
            const v4i l0 = *reinterpret_cast<const v4i*>(hr + kRowBytes + 16 * c);
            const v4i l1 = *reinterpret_cast<const v4i*>(hr + kRowBytes + 16 * c + 16);
            qh8[m] = v8i{h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
            ql8[m] = v8i{l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
        }
        qrh = *reinterpret_cast<const v4i*>(hr + 16 * (32 + g));
        qrl = *reinterpret_cast<const v4i*>(hr + kRowBytes + 16 * (32 + g));
        qsc = cq * kLog2e * s_qs[16 * hb + nn];   // logits in base-2 units
    }

    // Softmax state, with logits l in base-2 units (the softmax scale times
    // log2 e, folded into the query scale), so P = 2^(l - m): in the QK
    // layout a lane owns head 16 hb + nn (m_run, and l_run: this
    // wavefront's share of the denominator, relative to m_run); in the PV
    // layout accumulator row i of lane group g is head 16 h2 + 4g + i.
    //
    // A tile's probabilities are taken against m_run as it stood before the
    // tile (every wavefront holds the same value for a head), so they need
    // no exchange of the tile's maxima first: P = 2^(l - m_run) stays
    // below 2^kSlack unless the tile holds a logit more than kSlack above
    // m_run.  The maxima are exchanged at the barrier that publishes P', and
    // the rescale to the new maximum is applied to the output before the
    // next tile's PV.  A tile where some logit exceeds m_run + kSlack (every
    // first tile with a live token, where m_run is -inf) takes the exact
    // path instead: P against the new maximum, one more barrier.
    float m_run = -INFINITY, l_run = 0.0f;
    v4f o_acc[HB][NCB];
#pragma unroll
    for (int h2 = 0; h2 < HB; ++h2)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) o_acc[h2][cb] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    bool scale_bad = false;   // a live token of this lane had a bad scale

    // Per tile: wait for its data, start the gather NB-1 tiles ahead into the
    // buffer freed by the previous tile, then QK, softmax and PV.
    for (int it = 0, buf = 0; it < n_tiles; ++it, buf = buf == NB - 1 ? 0 : buf + 1) {
        uint8_t* xb = s_x[buf];
        const int tile = lo + it * kT;
        const int nt = min(kT, hi - tile);
        wait_tiles<NW>(wv, min(NB - 2, n_tiles - 1 - it));
        lds_sync();   // tile `it` is in LDS; every wavefront is done with tile it-1
        if (it + NB - 1 < n_tiles) issue(buf == 0 ? NB - 1 : buf - 1, tile + (NB - 1) * kT);
        // The previous tile's pending rescale, read now (the factors are
        // rewritten after this tile's second barrier) and applied before PV.
        int pend[HB];
        float4 pend_a[HB];
#pragma unroll
        for (int h2 = 0; h2 < HB; ++h2) {
            pend[h2] = s_moved[h2];
            pend_a[h2] = *reinterpret_cast<const float4*>(&s_alpha[16 * h2 + 4 * g]);
        }
        if (nt < kT || any_bad) {
            zero_dead(xb, tile);
            lds_sync();
        }

        // QK: token block tbk (A, rows), head block hb (B), on fp8 matrix
        // cores: the keys' codes as stored against the two query terms, the
        // 512 latent values in four 128-deep steps, the 64 rope values in two
        // 32-deep steps.
        v4f ah = v4f{0.0f, 0.0f, 0.0f, 0.0f}, al = ah;
        {
            const uint8_t* xr = xb + (16 * tbk + nn) * kXStride;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int c = qk_chunk(m, 0, g);
                const v4i x0 = *reinterpret_cast<const v4i*>(xr + 16 * c);
                const v4i x1 = *reinterpret_cast<const v4i*>(xr + 16 * c + 16);
                const v8i ka = v8i{x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
                ah = mfma_fp8_16x16x128(ka, qh8[m], ah);
                al = mfma_fp8_16x16x128(ka, ql8[m], al);
            }
            const v4i xq = *reinterpret_cast<const v4i*>(xr + 16 * (32 + g));
            ah = mfma_fp8_16x16x32(v2i{xq.x, xq.y}, v2i{qrh.x, qrh.y}, ah);
            al = mfma_fp8_16x16x32(v2i{xq.x, xq.y}, v2i{qrl.x, qrl.y}, al);
            ah = mfma_fp8_16x16x32(v2i{xq.z, xq.w}, v2i{qrh.z, qrh.w}, ah);
            al = mfma_fp8_16x16x32(v2i{xq.z, xq.w}, v2i{qrl.z, qrl.w}, al);
        }

        // Logits of this lane's tokens tk0 + i (tk0 = 16 tbk + 4g) for head
        // 16 hb + nn, and this wavefront's maximum.
        const int tk0 = 16 * tbk + 4 * g;
        float ts[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) ts[i] = *reinterpret_cast<const float*>(xb + (tk0 + i) * kXStride + kScaleAt);
        bool live[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) live[i] = tk0 + i < nt;
        if (any_bad) {
#pragma unroll
            for (int i = 0; i < 4; ++i) live[i] = live[i] && row_at(tile, tk0 + i) >= 0;
        }
        // A selected row whose scale is not a positive finite number is left
        // out of the attention, and reported once the loop is done.
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool ok = scale_ok(ts[i]);
            scale_bad |= live[i] && !ok;
            live[i] = live[i] && ok;
        }
        float lg[4];
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            lg[i] = live[i] ? (ah[i] + al[i]) * (qsc * ts[i]) : -INFINITY;
            mx = fmaxf(mx, lg[i]);
        }
        mx = rows4_max(mx);
        const int h = 16 * hb + nn;
        const bool big = mx > m_run + kSlack;   // false for mx = -inf; true for m_run = -inf < mx

        // Probabilities against m_run; P' to LDS.
        // tokens t = 16 tbk + 4g + i: group t / 8 = 2 tbk + g / 2, slot 4 (g & 1) + i
        uint2* const p_dst = reinterpret_cast<uint2*>(s_p + (2 * tbk + (g >> 1)) * kPGroup + h * 16 + 8 * (g & 1));
        auto probs = [&](float ref) -> float {
            float pv[4], ps = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pv[i] = live[i] ? __builtin_amdgcn_exp2f(lg[i] - ref) : 0.0f;
                ps += pv[i];
            }
            float pt4[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) pt4[i] = live[i] ? pv[i] * ts[i] : 0.0f;   // no 0 * (bad scale)
            const v2bf p01 = v2bf{(__bf16)pt4[0], (__bf16)pt4[1]};
            const v2bf p23 = v2bf{(__bf16)pt4[2], (__bf16)pt4[3]};
            *p_dst = uint2{__builtin_bit_cast(uint32_t, p01), __builtin_bit_cast(uint32_t, p23)};
            return rows4_sum(ps);
        };
        const float psum = probs(m_run);
        if (g == 0) s_red[h][tbk] = mx;
        s_big[wv] = __ballot(big) != 0ull;   // the same value from every lane
        lds_sync();

        // New running max (over the four token blocks) and its rescale.  The
        // running max moves only when the tile's exceeds it by more than
        // kLazy, so most tiles after the first need no rescale (P stays below
        // 2^kLazy against it, 2^kSlack on the tile that moves it).
        const float4 r4 = *reinterpret_cast<const float4*>(&s_red[h][0]);
        const float tmax = fmaxf(fmaxf(r4.x, r4.y), fmaxf(r4.z, r4.w));
        const float mn = tmax > m_run + kLazy ? tmax : m_run;   // tmax when m_run is -inf
        const bool moved = mn != m_run;
        const float alpha = (m_run == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_run - mn);
        const bool any_moved = __ballot(moved) != 0ull;   // same in the 4 wavefronts of head block hb
        bool exact = false;
#pragma unroll
        for (int w = 0; w < NW; ++w) exact |= s_big[w] != 0;
        m_run = mn;
        if (!exact) {
            l_run = (l_run + psum) * alpha;
            if (tbk == 0) {   // pending: applied before the next tile's PV
                if (g == 0) s_alpha[h] = alpha;
                if (lane == 0) s_moved[hb] = any_moved;
            }
        } else {
            // Exact path: P against the new maximum, rescale now, nothing pending.
            l_run = l_run * alpha + probs(mn);
            if (tbk == 0) {
                if (g == 0) s_alpha_x[h] = alpha;
                if (lane == 0) {
                    s_moved_x[hb] = any_moved;
                    s_moved[hb] = 0;
                }
            }
            lds_sync();
#pragma unroll
            for (int h2 = 0; h2 < HB; ++h2) {
                if (s_moved_x[h2]) {
                    const float4 al4 = *reinterpret_cast<const float4*>(&s_alpha_x[16 * h2 + 4 * g]);
                    if (pend[h2]) {
                        pend_a[h2].x *= al4.x; pend_a[h2].y *= al4.y; pend_a[h2].z *= al4.z; pend_a[h2].w *= al4.w;
                    } else {
                        pend_a[h2] = al4;
                    }
                    pend[h2] = 1;
                }
            }
        }

        // Rescales before PV; alpha is exactly 1 for every head whose max did not move.
#pragma unroll
        for (int h2 = 0; h2 < HB; ++h2) {
            if (pend[h2]) {
                const float av[4] = {pend_a[h2].x, pend_a[h2].y, pend_a[h2].z, pend_a[h2].w};
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb) o_acc[h2][cb][i] *= av[i];
            }
        }

        // PV for columns [CW wv, CW wv + CW), all heads.  Lane group g's
        // 8 K values are tokens 32 ks + 8 g + [0, 8) in both operands.
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            v8bf pa[HB];
#pragma unroll
            for (int h2 = 0; h2 < HB; ++h2)
                pa[h2] = *reinterpret_cast<const v8bf*>(s_p + (4 * ks + g) * kPGroup + (16 * h2 + nn) * 16);
            const uint8_t* trow = xb + (32 * ks + 8 * g + (nn >> 1)) * kXStride + CW * wv + 8 * (nn & 1);
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                const v2i t = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(trow + 16 * cb));
                const v8bf bx = fp8x8_to_bf16x8((uint32_t)t.x, (uint32_t)t.y);
#pragma unroll
                for (int h2 = 0; h2 < HB; ++h2) o_acc[h2][cb] = mfma_bf16_16x16x32(pa[h2], bx, o_acc[h2][cb]);
            }
        }
    }

    if (__ballot(scale_bad) != 0ull && lane == 0) flag(a.status, DSA_DEV_SCALE);

    // The last tile's pending rescale; the barrier also ends every read of
    // the last tile's maxima, so s_red and s_m are free below.
    lds_sync();
#pragma unroll
    for (int h2 = 0; h2 < HB; ++h2) {
        if (s_moved[h2]) {
            const float4 al4 = *reinterpret_cast<const float4*>(&s_alpha[16 * h2 + 4 * g]);
            const float av[4] = {al4.x, al4.y, al4.z, al4.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) o_acc[h2][cb][i] *= av[i];
        }
    }

    // Denominators (sum of the wavefronts' shares) and the running max,
    // moved to the PV layout through LDS.
    if (g == 0) s_red[16 * hb + nn][tbk] = l_run;
    if (tbk == 0 && g == 0) s_m[16 * hb + nn] = m_run;
    __syncthreads();
#pragma unroll
    for (int h2 = 0; h2 < HB; ++h2) {
        const float4 m4 = *reinterpret_cast<const float4*>(&s_m[16 * h2 + 4 * g]);
        const float mv[4] = {m4.x, m4.y, m4.z, m4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int hh = h2 * 16 + 4 * g + i;
            const float4 l4 = *reinterpret_cast<const float4*>(&s_red[hh][0]);
            const float l = (l4.x + l4.y) + (l4.z + l4.w);
            const float inv = l > 0.0f ? 1.0f / l : 0.0f;
            const float lse = l > 0.0f ? mv[i] * kLn2 + __logf(l) : -INFINITY;   // natural log
            const size_t rh = (size_t)r * H + hh;
            if (ns == 1) {
                uint16_t* dst = a.out + rh * kDv + CW * wv + nn;
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) dst[16 * cb] = f32_to_bf16_rne(o_acc[h2][cb][i] * inv);
                if (a.out_lse != nullptr && wv == 0 && nn == 0) a.out_lse[rh] = lse;
            } else {
                // bf16 partials, two columns a lane: lanes nn and nn ^ 1
                // swap one value of a block pair, so the even lane writes
                // columns (nn, nn + 1) of block cb and the odd lane those of
                // block cb + 1.
                static_assert(NCB % 2 == 0, "column blocks in pairs");
                const bool odd = (nn & 1) != 0;
                uint16_t* dst = a.part_o + (rh * ns + sp) * kDv + CW * wv + (nn & ~1);
#pragma unroll
                for (int cb = 0; cb < NCB; cb += 2) {
                    const uint32_t v0 = f32_to_bf16_rne(o_acc[h2][cb][i] * inv);
                    const uint32_t v1 = f32_to_bf16_rne(o_acc[h2][cb + 1][i] * inv);
                    const uint32_t got =
                        (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(odd ? v0 : v1), 0xB1, 0xF, 0xF, false);
                    *reinterpret_cast<uint32_t*>(dst + 16 * (cb + (odd ? 1 : 0))) =
                        odd ? (got | (v1 << 16)) : (v0 | (got << 16));
                }
                if (wv == 0 && nn == 0) a.part_lse[rh * ns + sp] = lse;
            }
        }
    }
}

template <int HB, int NB>
hipError_t launch_hb(const MlaArgs& a, hipStream_t stream) {
    // Whole groups of eight chains (one per XCD), padded.
    const int64_t chains = (a.n_rows / a.chain + 7) / 8 * 8;
    const int64_t wgs = chains * a.chain * a.n_splits;
    if (wgs > INT32_MAX) return hipErrorInvalidValue;
    // Decode and MTP verify (at most 8 query rows a request) gather rows
    // that hardly any other workgroup reads, with the non-temporal hint:
    // bulk decode alone 31.8 -> 27.5 us cold, MTP verify's step 181.6 ->
    // 178.9 us.  Prefill's thousands of rows of one request read the same
    // cache rows many times over, and the hint cost it 18% (916 -> 1081 us).
    if ((int64_t)a.n_rows <= 8 * (int64_t)a.batch)
        sparse_mla_kernel<HB, NB, true><<<(unsigned)wgs, 256 * HB, 0, stream>>>(a);
    else
        sparse_mla_kernel<HB, NB, false><<<(unsigned)wgs, 256 * HB, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_mla(const MlaArgs& a, hipStream_t stream) {
    if (a.n_rows == 0) return hipSuccess;
    const int chunk = (a.top_k + a.n_splits - 1) / a.n_splits;
    const bool ring4 = chunk <= MlaGeom<4>::kRowsCap;
    switch (a.n_heads) {
        case 16: return ring4 ? launch_hb<1, 4>(a, stream) : launch_hb<1, 2>(a, stream);
        case 32: return ring4 ? launch_hb<2, 4>(a, stream) : launch_hb<2, 2>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace dsa
