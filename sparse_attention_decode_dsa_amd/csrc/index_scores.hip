// fp8 lightning-indexer scores on gfx950 MFMA.
//
// For one query row the score of token t is
//     s_t = k_scale[t] * sum_h wq[h] * relu(qcode[h] . kcode[t]),  wq = w * q_scale,
// i.e. a 64 x 128 by 128 x N fp8 contraction followed by a ReLU-weighted sum
// over the 64 heads.  The heads are the MFMA M dimension (4 blocks of 16), a
// 16-token block is N, and one v_mfma_f32_16x16x128_f8f6f4 covers the whole
// 128-wide key, so a token block costs 4 MFMAs per row.  The head reduction
// happens on the accumulator: each lane holds 16 of a token's 64 head dots
// (rows 4*(l/16)+i of 4 blocks), ReLU-weights and adds them, and two
// cross-lane adds finish the sum.
//
// K ordering: the MFMA pairs byte j of lane group g in A with byte j of lane
// group g in B, so any byte order shared by both operands is valid.  Lane
// group g takes key bytes [16g, 16g+16) and [64+16g, 64+16g+16): each of the
// two 16-byte loads of a wavefront then reads one contiguous 64-byte half of
// 16 consecutive 128-byte key rows.
//
// Work split, decode (G = 1): a workgroup (4 wavefronts) owns a chunk of
// a.chunk tokens of one row; wavefronts take 64-token groups in turn.  The
// chunk (a multiple of 256, at most kMaxChunk) is picked at launch so that the
// grid is about two workgroups per compute unit, all resident at once: a
// second, partial round of workgroups would run with most of the chip idle.
// With G > 1 (MTP verify, prefill) the keys of a 64-token group are loaded
// once and reused for every row of the group, whose queries sit in LDS; one
// 12-wavefront workgroup per compute unit takes an equal share of all groups'
// tiles, and its wavefronts claim the 64-token groups of that share as they go
// (the launch shapes are described above the kernels).
//
// Latency hiding: the chunk's page ids are read once into LDS, so key
// addresses never wait on a block-table load; each wavefront issues the
// loads of its next 64-token group before computing the current one.
#include "device_common.h"
#include "launch.h"
#include "query_quant.h"

#include <climits>

namespace dsa {

namespace {

constexpr int kMaxChunk = 8192;  // most tokens per workgroup
constexpr int kMinChunk = 1024;
constexpr int kQStride = 144;   // LDS bytes per query head row (128 + 16 pad: conflict-free b128 reads)

constexpr int kMaxChunkPages = kMaxChunk / 16;  // pages of one chunk at the smallest page size

// A read-only value at a wavefront-uniform address, through the scalar
// cache: it does not queue behind the wavefront's vector loads, so reading
// it never waits for them.
template <typename T>
__device__ __forceinline__ T load_uniform(const T* p) {
    return *(const __attribute__((address_space(4))) T*)p;
}

__device__ __forceinline__ v8i load_q_operand(const uint8_t* head_row, int g) {
    const uint4 lo = *reinterpret_cast<const uint4*>(head_row + 16 * g);
    const uint4 hi = *reinterpret_cast<const uint4*>(head_row + 64 + 16 * g);
    v8i r;
    r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
    r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
    return r;
}

// Whole-row key loads of a 16-token block (kWhole): load A reads rows 0-7
// of the block, load B rows 8-15, each 8 whole 128-byte rows.  Lane (n, g)
// with n < 8 gets (row n, bytes 16g) in A and (row n + 8, bytes 64 + 16g) in
// B; with n >= 8 it gets (row n - 8, bytes 64 + 16g) in A and (row n, bytes
// 16g) in B.  Lanes n and n ^ 8 trade the piece that belongs to the other's
// row (a DPP rotation of each 16-lane row by 8), which leaves every lane the
// operand of the half-row loads: bytes [16g, 16g + 16) and [64 + 16g, + 16)
// of row n.  x holds A in [0, 4) and B in [4, 8) as loaded.
__device__ __forceinline__ v8i trade_whole_rows(const v8i& x, int n) {
    const bool low = n < 8;
    v8i r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r[i] = low ? x[i] : x[4 + i];
        r[4 + i] = __builtin_amdgcn_update_dpp(0, low ? x[4 + i] : x[i], 0x128, 0xF, 0xF, false);   // row_ror:8
    }
    return r;
}

// The keys of one 64-token group in MFMA B layout: block j (tokens
// 16j..16j+15) in b[j]; lane l holds the scale of token l of the group and
// whether that token is scored at all (inside the span, on a valid page).
struct KeyGroup {
    v8i b[4];
    float scale;
    bool ok;
};

// max(x, 0) as one integer max on the bit pattern: every negative float
// (sign bit set) is a negative int32 and becomes +0, every other one is kept.
// (fmaxf costs a second, NaN-quieting instruction.)
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Scores of one 64-token group for one row, before the key scale: lane l
// gets the ReLU-weighted head sum of token l.  All 16 MFMAs (4 token blocks
// x 4 head blocks) are issued before any result is used.  Lane (n, g) of
// block j holds heads 16hb + 4g + i of token 16j + n; p[j] is its share of
// the head sum, and a transpose-reduce over the four lane rows gives row g
// the total of block g: two 32-lane swaps pair rows {0,2} and {1,3} of two
// blocks at once, one 16-lane swap then folds rows 0 and 1.
__device__ __forceinline__ float group_dot(const v8i (&qa)[4], const float (&wq)[4][4], const v8i (&kb)[4]) {
    v4f acc[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) acc[j][hb] = mfma_fp8_16x16x128(qa[hb], kb[j], v4f{0.0f, 0.0f, 0.0f, 0.0f});
    float p[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float t = 0.0f;
#pragma unroll
        for (int hb = 0; hb < 4; ++hb)
#pragma unroll
            for (int i = 0; i < 4; ++i) t = fmaf(wq[hb][i], relu(acc[j][hb][i]), t);
        p[j] = t;
    }
    // After the 32-lane swaps u (v) holds block 0 (1) in rows 0-1 and block
    // 2 (3) in rows 2-3, each as the sum of two rows.
    const auto s02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[0]), __float_as_uint(p[2]), false, false);
    const auto s13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[1]), __float_as_uint(p[3]), false, false);
    const float u = __uint_as_float(s02[0]) + __uint_as_float(s02[1]);
    const float v = __uint_as_float(s13[0]) + __uint_as_float(s13[1]);
    const auto w = __builtin_amdgcn_permlane16_swap(__float_as_uint(u), __float_as_uint(v), false, false);
    return __uint_as_float(w[0]) + __uint_as_float(w[1]);
}

// Row-groups a balanced launch can schedule (their tile counts live in LDS;
// fewer at eight rows a group, whose query codes take most of the LDS).
template <int G>
constexpr int max_balanced_groups() { return G > 4 ? 512 : 1024; }

template <int G, int NT>
struct IndexSmem {
    int vok[G];   // the rows' checked spans (0 for an invalid row)
    int page[kMaxChunkPages];
    __attribute__((aligned(16))) uint8_t q[G * 64 * kQStride];   // fp8 query codes
    __attribute__((aligned(16))) float wq[G * 64];              // head weight * query scale
    // One row (decode): a range's scores collect here and go out in one
    // burst after its keys are read (HBM reads slow down markedly when
    // writes are mixed in).  Several rows write as they go.
    __attribute__((aligned(16))) float sc[G == 1 ? kMaxChunk : 4];
    int pre[max_balanced_groups<G>() + 1];   // balanced launch: first tile of each group
    uint32_t scan[NT / kWave + 1];
    int next;     // balanced launch: the range's next unclaimed 64-token group
};

// Scores of rows [r0, r0 + G) at tokens [t0, t_end) (t0 a multiple of 64;
// -inf where a row's span ends) and -inf over [fill_lo, fill_hi), by a
// workgroup of NT threads.  The range's pages must fit the LDS page array
// (kMaxChunkPages).  `report`: this call reports the rows' geometry errors
// (one call per row does).  `quantize`: the group's queries are not in LDS
// yet (the previous call, if any, was for another group).  kDynamic (the
// balanced launch): the wavefronts claim the range's 64-token groups from an
// LDS counter, so a wavefront that the compute unit serves first also does
// more of them, and the rows' geometry comes checked and reported from the
// caller (geo_vis: the rows' checked spans, geo_b: their request); otherwise
// wavefront w takes groups w, w + NT/64, ... and the geometry is read here.
// kWhole: whole-row key loads with the non-temporal hint (see
// trade_whole_rows), for launches whose rows all stream most of the stride.
template <int G, int NT, bool kDynamic, bool kWhole = false>
__device__ __forceinline__ void score_range(const IndexArgs& a, IndexSmem<G, NT>& s, int r0, int t0, int t_end,
                                            int fill_lo, int fill_hi, bool report, bool quantize,
                                            const int* geo_vis = nullptr, int geo_b = 0) {
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int n = lane & 15;
    const int g = lane >> 4;
    lds_sync();   // the previous range is done with the shared arrays
    if (kDynamic && threadIdx.x == 0) s.next = 0;

    // The group's bf16 queries and head weights, loaded first (nothing waits
    // for them until the first keys are about to go out) and quantized once
    // those keys are in flight: four threads per head, elements [32 c,
    // 32 c + 32) each, c = threadIdx % 4; 256 threads cover the 64 heads of
    // one row, and the rows (passes) go round the NT / 256 sets of them.
    constexpr int kSets = NT / 256;
    constexpr int kPasses = (G + kSets - 1) / kSets;
    const int qc = threadIdx.x & 3;
    const int qh = (threadIdx.x >> 2) & 63;
    const int qset = threadIdx.x >> 8;
    uint4 qraw[kPasses][4];
    float hw[kPasses];   // head weight of this thread's head in each pass (used by qc == 0)
    if (quantize) {
#pragma unroll
        for (int j = 0; j < kPasses; ++j) {
            const int p = min(qset + kSets * j, G - 1);   // a set past the last row repeats it
#pragma unroll
            for (int k = 0; k < 4; ++k)
                qraw[j][k] = reinterpret_cast<const uint4*>(a.q + ((size_t)r0 * 64 + p * 64 + qh) * 128 + 32 * qc)[k];
            hw[j] = a.head_w[(size_t)r0 * 64 + p * 64 + qh];
        }
    }

    int b, vmax, vchk;
    int vrow[G];   // checked spans
    if constexpr (kDynamic) {
        b = geo_b;
        vmax = 0;
#pragma unroll
        for (int j = 0; j < G; ++j) {
            vrow[j] = geo_vis[j];
            vmax = max(vmax, vrow[j]);
        }
        vchk = vmax;
    } else {
        // Row geometry, the same in every thread (uniform loads, no LDS
        // round trip): the request and span against the launch's bounds, the
        // group's rows against its first row's request, then the spans
        // against that request's kv_len.  Thread j reports row j.  vis[j] =
        // -1 marks a row already reported.  vmax, the longest span before
        // the kv_len check, lets the block-table loads go out without
        // waiting for kv_len.
        int req[G], vis[G];
#pragma unroll
        for (int j = 0; j < G; ++j) {   // all loads first, then the checks
            req[j] = load_uniform(a.row_req + r0 + j);
            vis[j] = load_uniform(a.row_vis + r0 + j);
        }
        const int b0 = req[0];
        b = b0 >= 0 && b0 < a.batch ? b0 : 0;
        vmax = 0;
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const int bj = req[j];
            int v = vis[j];
            const bool ok = (bj >= 0) & (bj < a.batch) & (v >= 0) & (v <= a.score_stride) &
                            (v <= a.max_pages * a.page_size);
            if (!ok) {
                if (report && (int)threadIdx.x == j) flag(a.status, DSA_DEV_ROW_RANGE);
                v = -1;
            } else if (bj != b0) {
                if (report && (int)threadIdx.x == j) flag(a.status, DSA_DEV_GROUP);
                v = -1;
            }
            vis[j] = v;
            vmax = max(vmax, v);
        }
        const int kv = load_uniform(a.kv_lens + b);
        const bool kv_ok = kv <= a.max_pages * a.page_size;
        vchk = 0;
#pragma unroll
        for (int j = 0; j < G; ++j) {
            int v = vis[j];
            if (v >= 0 && (v > kv || !kv_ok)) {
                if (report && (int)threadIdx.x == j) flag(a.status, DSA_DEV_ROW_RANGE);
                v = 0;
            }
            vrow[j] = max(v, 0);
            vchk = max(vchk, vrow[j]);
        }
    }
#pragma unroll
    for (int j = 0; j < G; ++j)
        if ((int)threadIdx.x == j) s.vok[j] = vrow[j];   // for the row loop below
    const int pmask = a.page_size - 1;
    // Tokens [t0, t_comp) are computed in 64-token groups; the rest of the
    // range only needs -inf.
    const int t_comp = min(t_end, t0 + ((max(vmax - t0, 0) + 63) & ~63));

    // Block table of the range, once: page ids of the pages [t0, t_comp)
    // touches (-1 for invalid ones).  An invalid page is reported only if it
    // lies inside a checked span.
    const int p0 = t0 >> a.log2_page;
    {
        int bad_from = INT_MAX;   // first token of an invalid page this thread saw
        const int np = t_comp > t0 ? ((t_comp - 1) >> a.log2_page) - p0 + 1 : 0;
        const int* pt = a.page_table + (size_t)b * a.max_pages;
        for (int i = threadIdx.x; i < np; i += NT) {
            int page = -1;
            if (((p0 + i) << a.log2_page) < vmax) {
                page = pt[p0 + i];
                if (page < 0 || page >= a.num_pages) {
                    bad_from = min(bad_from, (p0 + i) << a.log2_page);
                    page = -1;
                }
            }
            s.page[i] = page;
        }
        if (bad_from < vchk) flag(a.status, DSA_DEV_PAGE_OOB);
    }
    lds_sync();   // page ids and the claim counter are in place

    v8i qa[4];
    float wq[4][4];

    // Loads of the group starting at token tg, branch-free: a block past
    // vmax or on an invalid page reads row n of page 0 instead (always
    // inside the cache) and its tokens are masked out of the scores.
    // Keeping every path's loads identical lets the compiler wait for
    // exactly the group it needs.
    auto load_group = [&](int tg, KeyGroup& kg) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int tb = tg + 16 * j;
            const int page = tb < vmax ? s.page[(tb >> a.log2_page) - p0] : -1;
            if constexpr (kWhole) {
                typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
                const size_t base = page >= 0 ? (size_t)page * a.page_size + (tb & pmask) : 0;
                const int lo_row = n & 7, lo_chunk = n < 8 ? g : 4 + g;
                const int hi_row = (n & 7) + 8, hi_chunk = n < 8 ? 4 + g : g;
                const i32x4 x = __builtin_nontemporal_load(
                    reinterpret_cast<const i32x4*>(a.k_code + (base + lo_row) * 128 + 16 * lo_chunk));
                const i32x4 y = __builtin_nontemporal_load(
                    reinterpret_cast<const i32x4*>(a.k_code + (base + hi_row) * 128 + 16 * hi_chunk));
                kg.b[j] = v8i{x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
            } else {
                const size_t row = page >= 0 ? (size_t)page * a.page_size + (tb & pmask) + n : (size_t)n;
                kg.b[j] = load_q_operand(a.k_code + row * 128, g);
            }
        }
        const int t = tg + lane;
        const int page = t < vmax ? s.page[(t >> a.log2_page) - p0] : -1;
        kg.ok = page >= 0;
        kg.scale = a.k_scale[page >= 0 ? (size_t)page * a.page_size + (t & pmask) : 0];
    };

    bool scale_bad = false;   // a checked key of this lane had a bad scale

    // Scores of the group at tg for every row of the group.
    auto process = [&](KeyGroup& kg, int tg) {
        // Every path consumes the group's loads here, so none is left
        // pending across the loop's back edge when a path skips the rows.
#pragma unroll
        for (int j = 0; j < 4; ++j) pin(kg.b[j]);
        pin(kg.scale);
        if constexpr (kWhole) {
#pragma unroll
            for (int j = 0; j < 4; ++j) kg.b[j] = trade_whole_rows(kg.b[j], n);
        }
        const int t = tg + lane;
        // A key whose scale is not a positive finite number is not scored
        // (the head reduction relies on a positive scale); one inside a
        // checked span is reported once the range is done.
        const bool sok = scale_ok(kg.scale);
        scale_bad |= kg.ok && !sok && t < vchk;
        kg.ok = kg.ok && sok;
#pragma unroll 1
        for (int rr = 0; rr < G; ++rr) {
            const int r = r0 + rr;
            const int v = s.vok[rr];
            float mine = -INFINITY;
            if (tg < v) {
                if constexpr (G > 1) {
#pragma unroll
                    for (int hb = 0; hb < 4; ++hb) {
                        qa[hb] = load_q_operand(s.q + (rr * 64 + hb * 16 + n) * kQStride, g);
#pragma unroll
                        for (int i = 0; i < 4; ++i) wq[hb][i] = s.wq[rr * 64 + hb * 16 + 4 * g + i];
                    }
                }
                const float sc = group_dot(qa, wq, kg.b) * kg.scale;
                if (kg.ok && t < v) mine = sc;
            }
            if constexpr (G == 1) {
                if (t < t_end) s.sc[t - t0] = mine;
            } else {
                if (t < t_end) a.scores[(size_t)r * a.score_stride + t] = mine;
            }
        }
    };

    // The wavefront's first 64-token group, and the one after tg.
    constexpr int kStride = NT;   // static order: the workgroup's wavefronts cover NT tokens a round
    auto claim = [&]() -> int {
        int i = 0;
        if (lane == 0) i = atomicAdd(&s.next, 1);
        return t0 + 64 * __builtin_amdgcn_readfirstlane(i);
    };
    auto after = [&](int tg) -> int {
        if constexpr (kDynamic) return claim();
        else return tg + kStride;
    };

    KeyGroup ka, kb;
    int tg = kDynamic ? claim() : t0 + wv * 64;
    if (quantize) {
        // The query loads are long done; consuming them here, before any key
        // load goes out, keeps the compiler from waiting for keys as well
        // when the quantization below first reads them.
#pragma unroll
        for (int j = 0; j < kPasses; ++j) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                pin(qraw[j][k].x); pin(qraw[j][k].y); pin(qraw[j][k].z); pin(qraw[j][k].w);
            }
            pin(hw[j]);
        }
    }
    if (tg < t_comp) load_group(tg, ka);

    if (quantize) {
        // Query quantization (the same arithmetic as dsa_quantize_q) into LDS
        // while the first keys load: the head's amax over its four threads,
        // one power-of-two scale, fp8 codes.
#pragma unroll
        for (int j = 0; j < kPasses; ++j) {
            const int p = qset + kSets * j;
            float v[32];
            float amax = 0.0f;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                float x[8];
                bf16x8_to_f32(qraw[j][k], x);
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    v[8 * k + u] = x[u];
                    amax = fmaxf(amax, fabsf(x[u]));
                }
            }
            amax = fmaxf(amax, dpp<0xB1>(amax));   // the head's four threads are one quad
            amax = fmaxf(amax, dpp<0x4E>(amax));
            const int e = idx_q_exponent(amax);
            const IdxQFactors f = idx_q_factors(e);
            uint32_t w[8];
#pragma unroll
            for (int k = 0; k < 8; ++k)
                w[k] = idx_q_code2(v[4 * k], v[4 * k + 1], f) | (idx_q_code2(v[4 * k + 2], v[4 * k + 3], f) << 16);
            if (p < G) {
                const int hr = p * 64 + qh;
                uint4* dst = reinterpret_cast<uint4*>(s.q + hr * kQStride + 32 * qc);
                dst[0] = uint4{w[0], w[1], w[2], w[3]};
                dst[1] = uint4{w[4], w[5], w[6], w[7]};
                if (qc == 0) s.wq[hr] = hw[j] * ldexpf(1.0f, e);
            }
        }
        lds_sync();
    }
    if constexpr (G == 1) {
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) {
            qa[hb] = load_q_operand(s.q + (hb * 16 + n) * kQStride, g);
#pragma unroll
            for (int i = 0; i < 4; ++i) wq[hb][i] = s.wq[hb * 16 + 4 * g + i];
        }
    }

    // Two key buffers in turn: the loads of the next group are in flight
    // while the current one is computed, and no register copy forces a wait
    // on them before the next loads go out.  The last prefetch of a
    // wavefront re-reads its current group (an L2 hit) rather than
    // branching around the loads.
    if (tg < t_comp) {
        while (true) {
            const int t1 = after(tg);
            const bool m1 = t1 < t_comp;
            load_group(m1 ? t1 : tg, kb);
            process(ka, tg);
            if (!m1) break;
            tg = t1;
            const int t2 = after(tg);
            const bool m2 = t2 < t_comp;
            load_group(m2 ? t2 : tg, ka);
            process(kb, tg);
            if (!m2) break;
            tg = t2;
        }
    }
    if (__ballot(scale_bad) != 0ull && lane == 0) flag(a.status, DSA_DEV_SCALE);

    if constexpr (G == 1) {
        // -inf past the span, then the whole range out: 16-byte stores where
        // the row's range is 16-byte aligned, else one float per lane.
        for (int t = t_comp + threadIdx.x; t < t_end; t += NT) s.sc[t - t0] = -INFINITY;
        __syncthreads();
        float* dst = a.scores + (size_t)r0 * a.score_stride + t0;
        const int cnt = t_end - t0;
        if ((reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
            for (int i = 4 * threadIdx.x; i + 3 < cnt; i += 4 * NT)
                *reinterpret_cast<float4*>(dst + i) = *reinterpret_cast<const float4*>(&s.sc[i]);
            for (int i = (cnt & ~3) + threadIdx.x; i < cnt; i += NT) dst[i] = s.sc[i];
        } else {
            for (int i = threadIdx.x; i < cnt; i += NT) dst[i] = s.sc[i];
        }
    } else {
        // -inf for the part of the range past every row's span.
        for (int rr = 0; rr < G; ++rr) {
            float* srow = a.scores + (size_t)(r0 + rr) * a.score_stride;
            for (int t = t_comp + threadIdx.x; t < t_end; t += NT) srow[t] = -INFINITY;
        }
    }
    // This range's share of the rows' tail past their tiles.
    for (int rr = 0; rr < G; ++rr) {
        float* srow = a.scores + (size_t)(r0 + rr) * a.score_stride;
        for (int t = fill_lo + threadIdx.x; t < fill_hi; t += NT) srow[t] = -INFINITY;
    }
}

// ---------------------------------------------------------------------------
// Top-k candidates in the decode epilogue (dsa_index_topk).
//
// The row's top k is a small part of it, and a chunk's scores are still in
// LDS when they have gone out, so the chunk keeps its likely share of the top
// k right there: every visible score at or above a cut of its own, as keys
// and slots in slot order, for a merge that selects the row's top k from them.
// Thread t holds the chunk's positions [t L, t L + L) in registers, and its
// first key is one of S evenly spaced samples.  The chunk holds n of the
// row's v visible tokens, so about mu = k S / v samples fall in the row's top
// k; the cut is the sample of rank rho = ceil(mu + 4 sqrt(mu) + 4) from the
// top, rounded down to 14 bits below the highest bit in which the samples
// differ, or 0 (keep all) when rho > S, and about rho n / S keys pass it.  Keeping more than cand_cap
// keys (only when many scores are equal) is reported as a count of -1.  None
// of this decides the result: the merge checks that the candidates hold the
// row's top k and otherwise selects from the scores.
// ---------------------------------------------------------------------------

constexpr int kKeepMax = kMaxChunk / 256;   // most keys per thread

// Chunk j = [t0, t0 + cnt) of row r: its candidates into the workspace
// block of (r, j).  Called by every thread after score_range, whose scores
// stay in s.sc; the query codes are no longer needed, and their LDS holds the
// samples.
template <int NT>
__device__ void keep_candidates(const IndexArgs& a, IndexSmem<1, NT>& s, int r, int j, int t0, int cnt) {
    static_assert(NT == 256 && sizeof(s.q) >= NT * sizeof(uint32_t), "the samples fit the query codes' LDS");
    constexpr int NW = NT / kWave;
    // The compute unit's other workgroup is usually still in its main loop;
    // this short tail goes first.
    __builtin_amdgcn_s_setprio(3);
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = tid / kWave;
    const int v = s.vok[0];
    const int n = min(max(v - t0, 0), cnt);   // the chunk's visible tokens
    const size_t rj = (size_t)r * gridDim.x + j;
    uint32_t* smp = reinterpret_cast<uint32_t*>(s.q);
    int* tab = s.pre;   // kept keys per wavefront

    // Keys per thread: a multiple of 4 (whole 16-byte LDS reads), so that
    // NT L covers the chunk (L <= kKeepMax since cnt <= kMaxChunk).
    const int L = (((cnt + NT - 1) / NT) + 3) & ~3;
    const int base = tid * L;
    const int mine = max(0, min(L, n - base));
    uint32_t key[kKeepMax];
    bool nan = false;
#pragma unroll
    for (int m = 0; m < kKeepMax / 4; ++m) {
        float4 f = float4{0.0f, 0.0f, 0.0f, 0.0f};
        if (4 * m < mine) f = *reinterpret_cast<const float4*>(&s.sc[base + 4 * m]);
        const float fv[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            nan |= (fv[e] != fv[e]) && 4 * m + e < mine;
            key[4 * m + e] = monotone_key(fv[e]);
        }
    }
    if (__ballot(nan) != 0ull && lane == 0) flag(a.status, DSA_DEV_NAN);
    // Samples: thread t's first key, for the S threads that hold any; the
    // rest read as key 0, which never rises above a real sample.
    const int S = (n + L - 1) / L;
    smp[tid] = mine > 0 ? key[0] : 0u;
    __syncthreads();
    const float mu = n > 0 ? (float)a.top_k * (float)S / (float)v : 0.0f;
    const int rho = (int)ceilf(mu + 4.0f * sqrtf(mu) + 4.0f);
    uint32_t cut = 0u;
    if (rho <= S) {
        // Every wavefront finds the rho-th largest sample on its own (no
        // barrier), lane l holding samples l + 64 i.  Below the bits that
        // all samples share, two bits a step: the largest t on the step's
        // grid with at least rho samples >= t (counted with ballots) becomes
        // the cut.  Fourteen bits below the first one that differs, the cut
        // sits at or below the rho-th largest sample, so at least rho
        // samples pass it.
        uint32_t x[NT / kWave];
        uint32_t hi = 0u, lo = ~0u;
#pragma unroll
        for (int i = 0; i < NT / kWave; ++i) {
            x[i] = smp[lane + kWave * i];
            hi = max(hi, x[i]);
            lo = min(lo, x[i]);
        }
        hi = wave_max_u32(hi);
        lo = wave_min_u32(lo);
        const int top = hi == lo ? -1 : 31 - __clz(hi ^ lo);   // highest bit the samples differ in
        cut = top < 0 ? hi : hi & ~((2u << top) - 1u);
        auto count_ge = [&](uint32_t t) {
            uint32_t c = 0;
#pragma unroll
            for (int i = 0; i < NT / kWave; ++i) c += (uint32_t)__popcll(__ballot(x[i] >= t));
            return c;
        };
#pragma unroll 1
        for (int b = top; b >= max(top - 13, 0); b -= 2) {
            const int sh = max(b - 1, 0);   // the step's lowest bit (one bit when b == 0)
            const uint32_t t3 = cut | (3u << sh), t2 = cut | (2u << sh), t1 = cut | (1u << sh);
            const uint32_t c3 = b > 0 ? count_ge(t3) : 0u;
            const uint32_t c2 = b > 0 ? count_ge(t2) : 0u;
            const uint32_t c1 = count_ge(t1);
            cut = c3 >= (uint32_t)rho ? t3 : c2 >= (uint32_t)rho ? t2 : c1 >= (uint32_t)rho ? t1 : cut;
        }
    }

    // Kept keys in slot order: a mask per thread, one wavefront scan, and the
    // wavefronts' totals in LDS.
    uint32_t km = 0u;
#pragma unroll
    for (int i = 0; i < kKeepMax; ++i) km |= (i < mine && key[i] >= cut ? 1u : 0u) << i;
    const uint32_t c = (uint32_t)__popc(km);
    const uint32_t inc = wave_inclusive_scan(c);
    if (lane == kWave - 1) tab[w] = (int)inc;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int q = 0; q < NW; ++q) {
        before += q < w ? tab[q] : 0;
        total += tab[q];
    }
    if (total > a.cand_cap) {
        if (tid == 0) {
            a.cand_count[rj] = -1;
            a.cand_cut[rj] = (int)cut;
        }
        return;
    }
    // The kept keys and their positions go to LDS in order (the scores there
    // are in registers by now), then out in coalesced stores; a list too
    // long for that goes out directly.
    uint32_t* ckey = a.cand_key + rj * a.cand_cap;
    int32_t* cslot = a.cand_slot + rj * a.cand_cap;
    uint32_t* stk = reinterpret_cast<uint32_t*>(s.sc);
    constexpr int kHalf = kMaxChunk / 2;
    const bool staged = total <= kHalf;
    uint32_t at = (uint32_t)before + inc - c;
#pragma unroll
    for (int i = 0; i < kKeepMax; ++i) {
        if ((km >> i) & 1u) {
            if (staged) {
                stk[at] = key[i];
                stk[kHalf + at] = (uint32_t)(base + i);
            } else {
                ckey[at] = key[i];
                cslot[at] = t0 + base + i;
            }
            ++at;
        }
    }
    if (staged) {
        __syncthreads();
        for (int i = tid; i < total; i += NT) {
            ckey[i] = stk[i];
            cslot[i] = t0 + (int)stk[kHalf + i];
        }
    }
    if (tid == 0) {
        a.cand_count[rj] = total;
        a.cand_cut[rj] = (int)cut;
    }
}

// Two launch shapes:
//   chunked:  grid (chunks, groups) of 256-thread workgroups; a workgroup
//             scores one chunk of a.chunk tokens of one group of G rows;
//   balanced: one 768-thread workgroup per compute unit (three wavefronts
//             per SIMD, as many as 168 VGPRs allow); every workgroup
//             counts the live 64-token tiles of every group (max(1,
//             ceil(vmax / 64)), vmax the group's longest row, so that a dead
//             group still owns one tile), and takes an equal share of the
//             concatenated tiles, group by group, in ranges whose pages fit
//             the LDS page array.  A group's tail past its tiles, [64 T,
//             score_stride), is cut in proportion to the tiles, so every
//             position of every row is written exactly once.  Rows of very
//             different lengths then cost each workgroup the same.
// Groups of several rows (MTP verify, prefill) use the balanced shape; one
// row per group (decode) the chunked one, whose workgroups start sooner
// (measured faster for decode batches, ragged ones included).
//
// The balanced shape is compute-bound, and a compute unit serves its oldest
// wavefronts first.  Two workgroups per unit with fixed shares measured a
// long tail in which the younger one ran alone, one wavefront per SIMD; one
// workgroup whose wavefronts claim tiles as they go ends them together, and
// quantizes each group's queries once per unit instead of twice.
// kKeep (one row a group): the chunk's top-k candidates are kept as well.
template <int G, bool kKeep, bool kWhole = false>
__global__ __launch_bounds__(256) void index_scores_kernel(IndexArgs a) {
    __shared__ IndexSmem<G, 256> s;
    const int t0 = blockIdx.x * a.chunk;
    const int t_end = min(t0 + a.chunk, a.score_stride);
    score_range<G, 256, false, kWhole>(a, s, blockIdx.y * G, t0, t_end, 0, 0, blockIdx.x == 0, true);
    if constexpr (kKeep) keep_candidates<256>(a, s, blockIdx.y, blockIdx.x, t0, t_end - t0);
}

constexpr int kBalancedThreads = 768;

template <int G>
__global__ __launch_bounds__(kBalancedThreads) void index_scores_balanced_kernel(IndexArgs a) {
    constexpr int NT = kBalancedThreads;
    __shared__ IndexSmem<G, NT> s;
    constexpr int kPer = (max_balanced_groups<G>() + NT - 1) / NT;   // groups per thread in the scan
    // A workgroup pays a prologue (query loads and quantization, block
    // table) for every group it works on, about as long as kPrologue tiles
    // of that group.  Each group therefore starts with kPrologue virtual
    // tiles in the concatenation that the shares cut: a share that runs
    // into a second group gets that many fewer real tiles.
    constexpr int kPrologue = 2 * G + 2;
    const int ng = a.n_rows / G;
    const int cap = min(a.score_stride, a.max_pages * a.page_size);
    // The groups' row geometry, read and checked once here for the whole
    // launch (the first workgroup reports): each row's request and span
    // against the launch's bounds, its request against its group's first
    // row's, its span against that request's kv_len.  rvis holds the checked
    // spans (0 for an invalid row), greq each group's request.  The kv_len
    // loads complete while the tile counts are scanned.
    __shared__ int rvis[max_balanced_groups<G>() * G];
    __shared__ int greq[max_balanced_groups<G>()];
    const bool report = blockIdx.x == 0;
    int req[kPer][G], vis[kPer][G], kv[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int gi = kPer * (int)threadIdx.x + k;
#pragma unroll
        for (int j = 0; j < G; ++j) {
            req[k][j] = gi < ng ? a.row_req[gi * G + j] : 0;
            vis[k][j] = gi < ng ? a.row_vis[gi * G + j] : 0;
        }
    }
    int cnt[kPer];
    int sum = 0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int gi = kPer * (int)threadIdx.x + k;
        const int b0 = req[k][0];
        kv[k] = gi < ng && b0 >= 0 && b0 < a.batch ? a.kv_lens[b0] : 0;
        int vm = 0;
#pragma unroll
        for (int j = 0; j < G; ++j) vm = max(vm, min(max(vis[k][j], 0), cap));
        cnt[k] = gi < ng ? kPrologue + max(1, (vm + 63) >> 6) : 0;
        sum += cnt[k];
    }
    uint32_t total;
    int ex = (int)block_exclusive_scan<NT>((uint32_t)sum, s.scan, &total);
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int gi = kPer * (int)threadIdx.x + k;
        if (gi < ng) {
            s.pre[gi] = ex;
            const int b0 = req[k][0];
            const bool kv_ok = kv[k] <= a.max_pages * a.page_size;
#pragma unroll
            for (int j = 0; j < G; ++j) {
                const int bj = req[k][j];
                int v = vis[k][j];
                const bool ok = (bj >= 0) & (bj < a.batch) & (v >= 0) & (v <= a.score_stride) &
                                (v <= a.max_pages * a.page_size);
                if (!ok) {
                    if (report) flag(a.status, DSA_DEV_ROW_RANGE);
                    v = 0;
                } else if (bj != b0) {
                    if (report) flag(a.status, DSA_DEV_GROUP);
                    v = 0;
                } else if (v > kv[k] || !kv_ok) {
                    if (report) flag(a.status, DSA_DEV_ROW_RANGE);
                    v = 0;
                }
                rvis[gi * G + j] = v;
            }
            greq[gi] = b0 >= 0 && b0 < a.batch ? b0 : 0;
        }
        ex += cnt[k];
    }
    if (threadIdx.x == 0) s.pre[ng] = (int)total;
    __syncthreads();
    const int T = s.pre[ng];
    const int A = (int)((int64_t)blockIdx.x * T / gridDim.x);
    const int B = (int)((int64_t)(blockIdx.x + 1) * T / gridDim.x);
    if (A >= B) return;
    // First group: the last one starting at or before position A.
    int lo = 0, hi = ng - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s.pre[mid] <= A) lo = mid;
        else hi = mid - 1;
    }
    // Tiles per range: its pages (one more where it starts inside a page)
    // must fit the page array.
    const int max_tiles = (int)min<int64_t>(
        INT_MAX / 64, max<int64_t>(kMaxChunk / 64, ((int64_t)(kMaxChunkPages - 1) << a.log2_page) / 64));
    int last = -1;
    for (int gi = lo; gi < ng && s.pre[gi] < B; ++gi) {
        const int base = s.pre[gi] + kPrologue;   // position of the group's first real tile
        const int tiles = s.pre[gi + 1] - base;
        const int j0 = max(A, base) - base, j1 = min(B, base + tiles) - base;   // j1 <= j0: none here
        const int tail = max(0, a.score_stride - 64 * tiles);
        for (int js = j0; js < j1; js += max_tiles) {
            const int je = min(j1, js + max_tiles);
            const int f_lo = 64 * tiles + (int)((int64_t)tail * js / tiles);
            const int f_hi = 64 * tiles + (int)((int64_t)tail * je / tiles);
            score_range<G, NT, true>(a, s, gi * G, 64 * js, min(64 * je, a.score_stride), f_lo, f_hi, js == 0,
                                     gi != last, &rvis[gi * G], greq[gi]);
            last = gi;
        }
    }
}

// Chunked grid size: two workgroups per compute unit (256 units).  Registers
// would allow three at G = 1, but two larger chunks each measure faster.
constexpr int kResidentWgs = 512;
constexpr int kComputeUnits = 256;

template <int G>
hipError_t launch_g(IndexArgs a, hipStream_t stream) {
    const int groups = a.n_rows / G;
    if constexpr (G > 1) {
        if (groups <= max_balanced_groups<G>()) {
            index_scores_balanced_kernel<G><<<kComputeUnits, kBalancedThreads, 0, stream>>>(a);
            return hipGetLastError();
        }
    }
    a.chunk = index_chunk(groups, a.score_stride);
    dim3 grid((a.score_stride + a.chunk - 1) / a.chunk, groups);
    if constexpr (G == 1) {
        if (a.cand_key != nullptr) {
            index_scores_kernel<1, true><<<grid, 256, 0, stream>>>(a);
            return hipGetLastError();
        }
        if (a.whole_rows) {
            index_scores_kernel<1, false, true><<<grid, 256, 0, stream>>>(a);
            return hipGetLastError();
        }
    }
    index_scores_kernel<G, false><<<grid, 256, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace

int index_chunk(int groups, int score_stride) {
    const int per_group = max(1, kResidentWgs / max(groups, 1));
    const int chunk = (int)(((int64_t)score_stride + per_group - 1) / per_group);
    return min(kMaxChunk, max(kMinChunk, (chunk + 255) & ~255));
}

hipError_t launch_index_scores(const IndexArgs& a, hipStream_t stream) {
    if (a.n_rows == 0) return hipSuccess;
    switch (a.group_rows) {
        case 1: return launch_g<1>(a, stream);
        case 2: return launch_g<2>(a, stream);
        case 3: return launch_g<3>(a, stream);
        case 4: return launch_g<4>(a, stream);
        case 5: return launch_g<5>(a, stream);
        case 6: return launch_g<6>(a, stream);
        case 7: return launch_g<7>(a, stream);
        case 8: return launch_g<8>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace dsa
