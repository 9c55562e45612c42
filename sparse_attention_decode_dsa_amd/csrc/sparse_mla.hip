// Split-K sparse absorbed-MLA decode on gfx950.
//
// A workgroup (4 wavefronts) owns one (row, split): the split's entries of
// the row's selected list, walked in tiles of 64 tokens with an online
// softmax.  Per tile:
//   gather  the 64 selected 576-byte fp8 rows through the block table into
//           LDS (rows padded to 592 bytes so 16 consecutive rows start on 16
//           distinct bank groups), with their fp32 scales;
//   QK      wavefront w computes the logits of tokens [16w, 16w+16) for all
//           heads: heads are the M dimension of v_mfma_f32_16x16x32_bf16 (one
//           chain per block of 16 heads sharing the token operand), tokens N,
//           the 576 latent+rope dims K.  The query sits in LDS for the whole
//           split (rows padded to 1168 bytes: conflict-free 16-byte reads);
//           each fp8 byte converts exactly to bf16 once; the token scale and
//           sm_scale multiply the fp32 logits;
//   softmax the tile maximum per head goes through LDS, every wavefront
//           keeps the same running max (the output is rescaled only when it
//           moved); P' = exp(l - m) * token scale is written to LDS in bf16;
//   PV      wavefront w owns output columns [128w, 128w+128) for all heads:
//           A = P' (heads x tokens), B = the fp8 rows read transposed by
//           ds_read_b64_tr_b8 (8 tokens of one column per lane), in bf16.
// The value rows are the first 512 entries of the same rows (absorbed MLA),
// so a tile is read from HBM once for both products.
//
// Latency hiding: the block table is walked once for the whole split (slot ->
// page -> physical row, kept in LDS).  Tiles are gathered by LDS-direct
// loads (global_load_lds_dwordx4: each lane's 16 bytes land at the
// wavefront's LDS base + 16 * lane), so the gather of tile i+1 needs no
// registers and runs while tile i is computed from the other buffer.
//
// K ordering in QK: lane group g supplies, for the MFMA pair p, dims
// [64p + 16g, 64p + 16g + 8) and then [64p + 16g + 8, 64p + 16g + 16), so one
// 16-byte LDS read of a row feeds two MFMAs; the query operand uses the same
// dims.  Accumulator rows 4*(l/16)+i of a lane are the same heads in the QK
// and PV layouts, so the running max and sum are per-lane state.
#include "device_common.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kT = 64;            // tokens per tile
constexpr int kRowBytes = 576;
constexpr int kXStride = 592;     // LDS bytes per gathered row
constexpr int kPStride = 144;     // LDS bytes per head of P' (64 bf16 + 16 pad)
constexpr int kQStride = 1168;    // LDS bytes per query head (576 bf16 + 16 pad)
constexpr int kDv = 512;
constexpr int kRowChunks = kXStride / 16;        // 37: 36 data chunks + 1 pad chunk
constexpr int kTileChunks = kT * kRowChunks;       // 2368 chunks of 16 bytes
constexpr int kDmaInsts = kTileChunks / kWave;     // 37 wavefront-wide LDS-direct loads
constexpr int kDmaPerWave = (kDmaInsts + 3) / 4;   // 10
constexpr int kMaxSplitLen = kTopkMaxK;  // selected entries one workgroup may own

typedef __attribute__((address_space(3))) v2i lds_v2i;
typedef __attribute__((address_space(3))) void lds_void;

template <int HB>
__global__ __launch_bounds__(256) void sparse_mla_kernel(MlaArgs a) {
    constexpr int H = 16 * HB;
    __shared__ __attribute__((aligned(16))) uint8_t s_x[2][kT * kXStride];
    __shared__ __attribute__((aligned(16))) uint8_t s_p[H * kPStride];
    __shared__ __attribute__((aligned(16))) uint8_t s_q[H * kQStride];
    __shared__ int32_t s_rows[kMaxSplitLen];
    __shared__ float s_scale[2][kT];
    __shared__ float s_red[4][H];
    __shared__ int s_geo[4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int nn = lane & 15;
    const int g = lane >> 4;
    const int r = blockIdx.y;
    const int sp = blockIdx.x;
    const int ns = gridDim.x;

    if (tid == 0) {
        const int b = a.row_req[r];
        const int v = a.row_vis[r];
        const int cnt = a.topk_count[r];
        bool ok = b >= 0 && b < a.batch && v >= 0 && v <= a.max_pages * a.page_size;
        if (!ok) flag(a.status, DSA_DEV_ROW_RANGE);
        if (ok && (cnt < 0 || cnt > a.top_k || cnt > v)) {
            flag(a.status, DSA_DEV_TOPK_OOB);
            ok = false;
        }
        s_geo[0] = ok ? b : 0;
        s_geo[1] = ok ? v : 0;
        s_geo[2] = ok ? cnt : 0;
        s_geo[3] = 0;
    }

    // Query of all heads into LDS.
    {
        const uint8_t* qsrc = reinterpret_cast<const uint8_t*>(a.q + (size_t)r * H * kRowBytes);
        for (int c = tid; c < H * 72; c += 256) {
            const int h = c / 72, part = c - h * 72;
            *reinterpret_cast<uint4*>(s_q + h * kQStride + part * 16) =
                *reinterpret_cast<const uint4*>(qsrc + (size_t)h * kRowBytes * 2 + part * 16);
        }
    }
    __syncthreads();
    const int vis = s_geo[1];
    const int cnt = s_geo[2];
    const int chunk = (cnt + ns - 1) / ns;
    const int lo = min(cnt, sp * chunk);
    const int hi = min(cnt, lo + chunk);
    const int n_tiles = (hi - lo + kT - 1) / kT;
    const int32_t* sel = a.topk_idx + (size_t)r * a.top_k;
    const int32_t* pt = a.page_table + (size_t)s_geo[0] * a.max_pages;
    const int pmask = a.page_size - 1;

    // Block-table walk for the whole split, once: selected slot -> page ->
    // physical row, kept in LDS (-1 for invalid entries, which are reported).
    // Loads go out in batches of 8 per thread before their results are used.
    for (int base = lo; base < hi; base += 256 * 8) {
        int slot[8], page[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int e = base + 256 * u + tid;
            slot[u] = e < hi ? sel[e] : -1;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int e = base + 256 * u + tid;
            page[u] = -1;
            if (e < hi) {
                if (slot[u] < 0 || slot[u] >= vis) flag(a.status, DSA_DEV_TOPK_OOB);
                else page[u] = pt[slot[u] >> a.log2_page];
            }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int e = base + 256 * u + tid;
            if (e < hi) {
                int32_t row = -1;
                if (page[u] >= a.num_pages || (page[u] < 0 && slot[u] >= 0 && slot[u] < vis)) {
                    flag(a.status, DSA_DEV_PAGE_OOB);
                } else if (page[u] >= 0) {
                    row = page[u] * a.page_size + (slot[u] & pmask);
                }
                if (row < 0) s_geo[3] = 1;
                s_rows[e - lo] = row;
            }
        }
    }

    // Row of tile-local token t of the tile starting at split entry `base`.
    auto row_at = [&](int base, int t) -> int32_t { return base + t < hi ? s_rows[base + t - lo] : -1; };

    // LDS-direct gather.  Wavefront wv issues the loads j = wv, wv+4, ... of
    // a tile; lane i of load j fills tile chunk 64j + i, i.e. row t =
    // chunk / 37, part chunk % 37 (part 36 is the row's pad and repeats part
    // 35).  Dead rows read row 0 of page 0 and are zeroed afterwards.
    int dma_t[kDmaPerWave], dma_off[kDmaPerWave];
#pragma unroll
    for (int jj = 0; jj < kDmaPerWave; ++jj) {
        const int c = 64 * (wv + 4 * jj) + lane;
        const int t = c / kRowChunks;
        const int part = min(c - t * kRowChunks, 35);
        dma_t[jj] = t;
        dma_off[jj] = part * 16;
    }
    auto gather_issue = [&](int buf, int base) {
#pragma unroll
        for (int jj = 0; jj < kDmaPerWave; ++jj) {
            const int j = wv + 4 * jj;
            if (j < kDmaInsts) {
                const int32_t row = max(row_at(base, dma_t[jj]), 0);
                const uint8_t* gp = a.kv_code + (size_t)row * kRowBytes + dma_off[jj];
                __builtin_amdgcn_global_load_lds(gp, (lds_void*)&s_x[buf][j * 1024], 16, 0, 0);
            }
        }
        if (wv == 0) {
            const int32_t row = max(row_at(base, lane), 0);
            __builtin_amdgcn_global_load_lds(a.kv_scale + row, (lds_void*)&s_scale[buf][0], 4, 0, 0);
        }
    };
    // Tiles that may hold dead rows: a partial last tile, or any invalid entry.
    auto zero_dead = [&](int buf, int base) {
        for (int c = tid; c < kT * 36; c += 256) {
            const int t = c / 36, part = c - t * 36;
            if (row_at(base, t) < 0) *reinterpret_cast<uint4*>(&s_x[buf][t * kXStride + part * 16]) = uint4{0u, 0u, 0u, 0u};
        }
    };

    // Prologue: tile 0.
    __syncthreads();
    const bool maybe_dead = ((hi - lo) % kT) != 0 || s_geo[3] != 0;
    if (n_tiles > 0) {
        gather_issue(0, lo);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (maybe_dead) zero_dead(0, lo);
    }
    __syncthreads();

    float m_run[HB][4], l_run[HB][4];
    v4f o_acc[HB][8];
#pragma unroll
    for (int h2 = 0; h2 < HB; ++h2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            m_run[h2][i] = -INFINITY;
            l_run[h2][i] = 0.0f;
        }
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) o_acc[h2][cb] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    }

    for (int it = 0; it < n_tiles; ++it) {
        const int cur = it & 1, nxt = cur ^ 1;
        const int tile = lo + it * kT;
        const int nt = min(kT, hi - tile);
        if (it + 1 < n_tiles) gather_issue(nxt, tile + kT);

        // QK for tokens [16 wv, 16 wv + 16), all heads.
        v4f s_acc[HB];
#pragma unroll
        for (int h2 = 0; h2 < HB; ++h2) s_acc[h2] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        const uint8_t* xrow = &s_x[cur][(16 * wv + nn) * kXStride + 16 * g];
#pragma unroll
        for (int p = 0; p < 9; ++p) {
            const uint4 xv = *reinterpret_cast<const uint4*>(xrow + 64 * p);
            const v8bf b0 = fp8x8_to_bf16x8(xv.x, xv.y);
            const v8bf b1 = fp8x8_to_bf16x8(xv.z, xv.w);
#pragma unroll
            for (int h2 = 0; h2 < HB; ++h2) {
                const uint8_t* qrow = s_q + (h2 * 16 + nn) * kQStride + (64 * p + 16 * g) * 2;
                s_acc[h2] = mfma_bf16_16x16x32(*reinterpret_cast<const v8bf*>(qrow), b0, s_acc[h2]);
                s_acc[h2] = mfma_bf16_16x16x32(*reinterpret_cast<const v8bf*>(qrow + 16), b1, s_acc[h2]);
            }
        }

        // Logits and this wavefront's maximum per head.
        const int tk = 16 * wv + nn;
        const bool live = tk < nt && row_at(tile, tk) >= 0;
        const float tsc = s_scale[cur][tk];
        const float lsc = live ? a.sm_scale * tsc : 0.0f;
        float lg[HB][4];
#pragma unroll
        for (int h2 = 0; h2 < HB; ++h2) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                lg[h2][i] = live ? s_acc[h2][i] * lsc : -INFINITY;
                const float mx = row16_max(lg[h2][i]);
                if (nn == 0) s_red[wv][h2 * 16 + 4 * g + i] = mx;
            }
        }
        __syncthreads();

        // Running max; probabilities of this wavefront's token.
        float alpha[HB][4];
        bool moved = false;
#pragma unroll
        for (int h2 = 0; h2 < HB; ++h2) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int h = h2 * 16 + 4 * g + i;
                const float mt = fmaxf(fmaxf(s_red[0][h], s_red[1][h]), fmaxf(s_red[2][h], s_red[3][h]));
                const float mn = fmaxf(m_run[h2][i], mt);
                moved |= mn != m_run[h2][i];
                alpha[h2][i] = (m_run[h2][i] == -INFINITY) ? 0.0f : __expf(m_run[h2][i] - mn);
                m_run[h2][i] = mn;
                const float pv = live ? __expf(lg[h2][i] - mn) : 0.0f;
                l_run[h2][i] = l_run[h2][i] * alpha[h2][i] + row16_sum(pv);
                *reinterpret_cast<uint16_t*>(s_p + h * kPStride + tk * 2) = f32_to_bf16_rne(live ? pv * tsc : 0.0f);
            }
        }
        // alpha is exactly 1 for every head whose max did not move.
        if (__ballot(moved) != 0ull) {
#pragma unroll
            for (int h2 = 0; h2 < HB; ++h2)
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int cb = 0; cb < 8; ++cb) o_acc[h2][cb][i] *= alpha[h2][i];
        }
        __syncthreads();

        // PV for columns [128 wv, 128 wv + 128), all heads.
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            v8bf pa[HB];
#pragma unroll
            for (int h2 = 0; h2 < HB; ++h2)
                pa[h2] = *reinterpret_cast<const v8bf*>(s_p + (h2 * 16 + nn) * kPStride + (32 * ks + 8 * g) * 2);
            const uint8_t* trow = &s_x[cur][(32 * ks + 8 * g + (nn >> 1)) * kXStride + 128 * wv + 8 * (nn & 1)];
#pragma unroll
            for (int cb = 0; cb < 8; ++cb) {
                const v2i t = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(trow + 16 * cb));
                const v8bf bx = fp8x8_to_bf16x8((uint32_t)t.x, (uint32_t)t.y);
#pragma unroll
                for (int h2 = 0; h2 < HB; ++h2) o_acc[h2][cb] = mfma_bf16_16x16x32(pa[h2], bx, o_acc[h2][cb]);
            }
        }
        // The next tile's loads were this wavefront's only memory traffic.
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (it + 1 < n_tiles && maybe_dead) {
            zero_dead(nxt, tile + kT);
            __syncthreads();
        }
    }

    // Softmax denominators: sum of the four wavefronts' partial sums.
#pragma unroll
    for (int h2 = 0; h2 < HB; ++h2)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (nn == 0) s_red[wv][h2 * 16 + 4 * g + i] = l_run[h2][i];
    __syncthreads();
#pragma unroll
    for (int h2 = 0; h2 < HB; ++h2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int h = h2 * 16 + 4 * g + i;
            const float l = s_red[0][h] + s_red[1][h] + s_red[2][h] + s_red[3][h];
            const float inv = l > 0.0f ? 1.0f / l : 0.0f;
            const float lse = l > 0.0f ? m_run[h2][i] + __logf(l) : -INFINITY;
            const size_t rh = (size_t)r * H + h;
            if (ns == 1) {
                uint16_t* dst = a.out + rh * kDv + 128 * wv + nn;
#pragma unroll
                for (int cb = 0; cb < 8; ++cb) dst[16 * cb] = f32_to_bf16_rne(o_acc[h2][cb][i] * inv);
                if (a.out_lse != nullptr && wv == 0 && nn == 0) a.out_lse[rh] = lse;
            } else {
                float* dst = a.part_o + (rh * ns + sp) * kDv + 128 * wv + nn;
#pragma unroll
                for (int cb = 0; cb < 8; ++cb) dst[16 * cb] = o_acc[h2][cb][i] * inv;
                if (wv == 0 && nn == 0) a.part_lse[rh * ns + sp] = lse;
            }
        }
    }
}

template <int HB>
hipError_t launch_hb(const MlaArgs& a, hipStream_t stream) {
    sparse_mla_kernel<HB><<<dim3(a.n_splits, a.n_rows), 256, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_mla(const MlaArgs& a, hipStream_t stream) {
    if (a.n_rows == 0) return hipSuccess;
    switch (a.n_heads) {
        case 16: return launch_hb<1>(a, stream);
        case 32: return launch_hb<2>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace dsa
