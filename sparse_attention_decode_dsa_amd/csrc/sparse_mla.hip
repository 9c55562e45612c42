// Split-K sparse absorbed-MLA decode on gfx950.
//
// A workgroup (4 wavefronts) owns one (row, split): the split's entries of
// the row's selected list, walked in tiles of 64 tokens with an online
// softmax.  Per tile:
//   gather  the 64 selected 576-byte fp8 rows through the block table into
//           LDS (rows padded to 592 bytes so 16 consecutive rows start on 16
//           distinct bank groups), with their fp32 scales;
//   QK      wavefront w computes the logits of tokens [16w, 16w+16) for all
//           heads: heads are the M dimension of v_mfma_f32_16x16x32_bf16,
//           tokens N, and the 576 latent+rope dims K.  The fp8 bytes convert
//           exactly to bf16; the token scale and sm_scale multiply the fp32
//           logits;
//   softmax the tile maximum per head goes through LDS, every wavefront
//           keeps the same running max; P' = exp(l - m) * token scale is
//           written to LDS in bf16;
//   PV      wavefront w owns output columns [128w, 128w+128): A = P' (heads x
//           tokens), B = the fp8 rows read transposed by ds_read_b64_tr_b8
//           (8 tokens of one column per lane), converted to bf16.
// The value rows are the first 512 entries of the same rows (absorbed MLA),
// so the tile is read from HBM once for both products.
//
// K ordering in QK: lane group g supplies, for the MFMA pair p, dims
// [64p + 16g, 64p + 16g + 8) and then [64p + 16g + 8, 64p + 16g + 16), so one
// 16-byte LDS read of a row feeds two MFMAs; the query operand uses the same
// dims.  The accumulator rows 4*(l/16)+i of a lane are the same heads in the
// QK and PV layouts, so running max and sum are per-lane state.
#include "device_common.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kT = 64;            // tokens per tile
constexpr int kRowBytes = 576;
constexpr int kXStride = 592;     // LDS bytes per gathered row
constexpr int kQStride = 1168;    // LDS bytes per query head (576 bf16 + 16 pad)
constexpr int kPStride = 144;     // LDS bytes per head of P' (64 bf16 + 16 pad)
constexpr int kDv = 512;

typedef __attribute__((address_space(3))) v2i lds_v2i;

template <int HB>
__global__ __launch_bounds__(256) void sparse_mla_kernel(MlaArgs a) {
    constexpr int H = 16 * HB;
    __shared__ __attribute__((aligned(16))) uint8_t s_x[kT * kXStride];
    __shared__ __attribute__((aligned(16))) uint8_t s_q[H * kQStride];
    __shared__ __attribute__((aligned(16))) uint8_t s_p[H * kPStride];
    __shared__ int64_t s_row[kT];
    __shared__ float s_scale[kT];
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
    }
    // Query of the row into LDS.
    {
        const uint8_t* qsrc = reinterpret_cast<const uint8_t*>(a.q + (size_t)r * H * kRowBytes);
        for (int c = tid; c < H * 72; c += 256) {
            const int h = c / 72, part = c - h * 72;
            *reinterpret_cast<uint4*>(s_q + h * kQStride + part * 16) =
                *reinterpret_cast<const uint4*>(qsrc + (size_t)h * kRowBytes * 2 + part * 16);
        }
    }
    __syncthreads();
    const int b = s_geo[0];
    const int vis = s_geo[1];
    const int cnt = s_geo[2];
    const int chunk = (cnt + ns - 1) / ns;
    const int lo = min(cnt, sp * chunk);
    const int hi = min(cnt, lo + chunk);
    const int32_t* sel = a.topk_idx + (size_t)r * a.top_k;
    const int32_t* pt = a.page_table + (size_t)b * a.max_pages;

    float m_run[HB][4], l_run[HB][4];
    v4f o_acc[HB][8];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) { m_run[hb][i] = -INFINITY; l_run[hb][i] = 0.0f; }
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) o_acc[hb][cb] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    }

    for (int tile = lo; tile < hi; tile += kT) {
        const int nt = min(kT, hi - tile);
        if (tid < kT) {
            int64_t row = -1;
            float sc = 0.0f;
            if (tid < nt) {
                const int slot = sel[tile + tid];
                if (slot < 0 || slot >= vis) {
                    flag(a.status, DSA_DEV_TOPK_OOB);
                } else {
                    const int page = pt[slot >> a.log2_page];
                    if (page < 0 || page >= a.num_pages) {
                        flag(a.status, DSA_DEV_PAGE_OOB);
                    } else {
                        row = (int64_t)page * a.page_size + (slot & (a.page_size - 1));
                        sc = a.kv_scale[row];
                    }
                }
            }
            s_row[tid] = row;
            s_scale[tid] = sc;
        }
        __syncthreads();
        // Gather: 64 rows x 36 chunks of 16 bytes; dead rows become zeros.
        for (int c = tid; c < kT * 36; c += 256) {
            const int t = c / 36, part = c - t * 36;
            const int64_t row = s_row[t];
            uint4 v = {0u, 0u, 0u, 0u};
            if (row >= 0) v = *reinterpret_cast<const uint4*>(a.kv_code + row * kRowBytes + part * 16);
            *reinterpret_cast<uint4*>(s_x + t * kXStride + part * 16) = v;
        }
        __syncthreads();

        // QK for tokens [16 wv, 16 wv + 16).
        v4f s_acc[HB];
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) s_acc[hb] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        const uint8_t* xrow = s_x + (16 * wv + nn) * kXStride + 16 * g;
#pragma unroll 3
        for (int p = 0; p < 9; ++p) {
            const uint4 xv = *reinterpret_cast<const uint4*>(xrow + 64 * p);
            const v8bf b0 = fp8x8_to_bf16x8(xv.x, xv.y);
            const v8bf b1 = fp8x8_to_bf16x8(xv.z, xv.w);
#pragma unroll
            for (int hb = 0; hb < HB; ++hb) {
                const uint8_t* qrow = s_q + (hb * 16 + nn) * kQStride + (64 * p + 16 * g) * 2;
                const v8bf a0 = *reinterpret_cast<const v8bf*>(qrow);
                const v8bf a1 = *reinterpret_cast<const v8bf*>(qrow + 16);
                s_acc[hb] = mfma_bf16_16x16x32(a0, b0, s_acc[hb]);
                s_acc[hb] = mfma_bf16_16x16x32(a1, b1, s_acc[hb]);
            }
        }

        // Logits and the tile max per head.
        const int tk = 16 * wv + nn;
        const bool live = tk < nt && s_row[tk] >= 0;
        const float tscale = s_scale[tk];
        const float lsc = a.sm_scale * tscale;
        float lg[HB][4];
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                lg[hb][i] = live ? s_acc[hb][i] * lsc : -INFINITY;
                const float mx = row16_max(lg[hb][i]);
                if (nn == 0) s_red[wv][hb * 16 + 4 * g + i] = mx;
            }
        }
        __syncthreads();
        float alpha[HB][4];
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int h = hb * 16 + 4 * g + i;
                const float mt = fmaxf(fmaxf(s_red[0][h], s_red[1][h]), fmaxf(s_red[2][h], s_red[3][h]));
                const float mn = fmaxf(m_run[hb][i], mt);
                alpha[hb][i] = (m_run[hb][i] == -INFINITY) ? 0.0f : __expf(m_run[hb][i] - mn);
                m_run[hb][i] = mn;
                const float pv = live ? __expf(lg[hb][i] - mn) : 0.0f;
                l_run[hb][i] = l_run[hb][i] * alpha[hb][i] + row16_sum(pv);
                const float pw = pv * tscale;
                *reinterpret_cast<uint16_t*>(s_p + h * kPStride + tk * 2) = f32_to_bf16_rne(pw);
#pragma unroll
                for (int cb = 0; cb < 8; ++cb) o_acc[hb][cb][i] *= alpha[hb][i];
            }
        }
        __syncthreads();

        // PV for columns [128 wv, 128 wv + 128).
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            v8bf pa[HB];
#pragma unroll
            for (int hb = 0; hb < HB; ++hb)
                pa[hb] = *reinterpret_cast<const v8bf*>(s_p + (hb * 16 + nn) * kPStride + (32 * ks + 8 * g) * 2);
            const uint8_t* trow = s_x + (32 * ks + 8 * g + (nn >> 1)) * kXStride + 128 * wv + 8 * (nn & 1);
#pragma unroll
            for (int cb = 0; cb < 8; ++cb) {
                const v2i t = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(trow + 16 * cb));
                const v8bf bx = fp8x8_to_bf16x8((uint32_t)t.x, (uint32_t)t.y);
#pragma unroll
                for (int hb = 0; hb < HB; ++hb) o_acc[hb][cb] = mfma_bf16_16x16x32(pa[hb], bx, o_acc[hb][cb]);
            }
        }
        __syncthreads();
    }

    // Sum of the per-wavefront softmax denominators.
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (nn == 0) s_red[wv][hb * 16 + 4 * g + i] = l_run[hb][i];
    }
    __syncthreads();
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int h = hb * 16 + 4 * g + i;
            const float l = s_red[0][h] + s_red[1][h] + s_red[2][h] + s_red[3][h];
            const float inv = l > 0.0f ? 1.0f / l : 0.0f;
            const float lse = l > 0.0f ? m_run[hb][i] + __logf(l) : -INFINITY;
            const size_t rh = (size_t)r * H + h;
            if (ns == 1) {
                uint16_t* dst = a.out + rh * kDv + 128 * wv + nn;
#pragma unroll
                for (int cb = 0; cb < 8; ++cb) dst[16 * cb] = f32_to_bf16_rne(o_acc[hb][cb][i] * inv);
                if (a.out_lse != nullptr && wv == 0 && nn == 0) a.out_lse[rh] = lse;
            } else {
                float* dst = a.part_o + (rh * ns + sp) * kDv + 128 * wv + nn;
#pragma unroll
                for (int cb = 0; cb < 8; ++cb) dst[16 * cb] = o_acc[hb][cb][i] * inv;
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
