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
// Work split: a workgroup (4 wavefronts) owns a chunk of kChunk tokens of a
// group of G rows of one request; wavefronts take 64-token groups in turn.
// With G > 1 (MTP verify, prefill) the keys of a 64-token group are loaded
// once and reused for every row of the group, whose queries sit in LDS.
#include "device_common.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kChunk = 2048;    // tokens per workgroup
constexpr int kQStride = 144;   // LDS bytes per query head row (128 + 16 pad: conflict-free b128 reads)

struct KeyBlock {
    v8i b;
    float scale;
    bool live;
};

__device__ __forceinline__ v8i load_q_operand(const uint8_t* head_row, int g) {
    const uint4 lo = *reinterpret_cast<const uint4*>(head_row + 16 * g);
    const uint4 hi = *reinterpret_cast<const uint4*>(head_row + 64 + 16 * g);
    v8i r;
    r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
    r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
    return r;
}

// Score of this lane's token column (lane % 16) for one row: 4 MFMAs over
// the head blocks, ReLU-weighted head sum, then the key scale.
__device__ __forceinline__ float score_block(const v8i (&qa)[4], const float (&wq)[4][4],
                                             const KeyBlock& kb) {
    float part = 0.0f;
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
        v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
        acc = mfma_fp8_16x16x128(qa[hb], kb.b, acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) part += wq[hb][i] * fmaxf(acc[i], 0.0f);
    }
    part += __shfl_xor(part, 16);
    part += __shfl_xor(part, 32);
    return part * kb.scale;
}

template <int G>
__global__ __launch_bounds__(256) void index_scores_kernel(IndexArgs a) {
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int n = lane & 15;
    const int g = lane >> 4;
    const int r0 = blockIdx.y * G;
    const int t0 = blockIdx.x * kChunk;
    const int t_end = min(t0 + kChunk, a.score_stride);

    __shared__ int s_req[G];
    __shared__ int s_vis[G];
    __shared__ __attribute__((aligned(16))) uint8_t s_q[G > 1 ? G * 64 * kQStride : 16];
    __shared__ __attribute__((aligned(16))) float s_wq[G > 1 ? G * 64 : 4];

    // Row geometry, checked once per row.
    if (threadIdx.x < G) {
        const int r = r0 + threadIdx.x;
        const int b = a.row_req[r];
        int v = a.row_vis[r];
        const int b0 = a.row_req[r0];
        bool ok = b >= 0 && b < a.batch;
        if (ok) {
            const int kv = a.kv_lens[b];
            ok = v >= 0 && v <= kv && kv <= a.max_pages * a.page_size && v <= a.score_stride;
        }
        if (!ok) {
            if (blockIdx.x == 0) flag(a.status, DSA_DEV_ROW_RANGE);
            v = 0;
        } else if (b != b0) {
            if (blockIdx.x == 0) flag(a.status, DSA_DEV_GROUP);
            v = 0;
        }
        s_req[threadIdx.x] = ok ? b : 0;
        s_vis[threadIdx.x] = v;
    }
    if constexpr (G > 1) {
        // Queries of the group into LDS (rows padded to kQStride bytes).
        for (int c = threadIdx.x; c < G * 64 * 8; c += 256) {
            const int hr = c >> 3, part = c & 7;   // head row (g*64+h), 16-byte part
            const uint4 v = *reinterpret_cast<const uint4*>(a.q_code + (size_t)(r0 * 64 + hr) * 128 + part * 16);
            *reinterpret_cast<uint4*>(s_q + hr * kQStride + part * 16) = v;
        }
        for (int c = threadIdx.x; c < G * 64; c += 256) {
            const size_t i = (size_t)r0 * 64 + c;
            s_wq[c] = a.head_w[i] * a.q_scale[i];
        }
    }
    __syncthreads();

    const int b = s_req[0];
    int vmax = 0;
#pragma unroll
    for (int j = 0; j < G; ++j) vmax = max(vmax, s_vis[j]);
    const int* pt = a.page_table + (size_t)b * a.max_pages;
    const int pmask = a.page_size - 1;

    // Tokens [t0, t_comp) are computed in 64-token groups; the rest of the
    // chunk only needs -inf.
    const int t_comp = min(t_end, t0 + ((max(vmax - t0, 0) + 63) & ~63));

    v8i qa[4];
    float wq[4][4];
    if constexpr (G == 1) {
        const int r = r0;
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) {
            qa[hb] = load_q_operand(a.q_code + ((size_t)r * 64 + hb * 16 + n) * 128, g);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const size_t hi = (size_t)r * 64 + hb * 16 + 4 * g + i;
                wq[hb][i] = a.head_w[hi] * a.q_scale[hi];
            }
        }
    }

    for (int tg = t0 + wv * 64; tg < t_comp; tg += 256) {
        KeyBlock kb[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int tb = tg + 16 * j;
            kb[j].live = tb < vmax;
            kb[j].scale = 0.0f;
            if (kb[j].live) {
                const int page = pt[tb >> a.log2_page];
                if (page < 0 || page >= a.num_pages) {
                    if (lane == 0) flag(a.status, DSA_DEV_PAGE_OOB);
                    kb[j].live = false;
                } else {
                    const size_t row = (size_t)page * a.page_size + (tb & pmask) + n;
                    kb[j].b = load_q_operand(a.k_code + row * 128, g);
                    kb[j].scale = a.k_scale[row];
                }
            }
        }
#pragma unroll 1
        for (int rr = 0; rr < G; ++rr) {
            const int r = r0 + rr;
            const int v = s_vis[rr];
            if constexpr (G > 1) {
#pragma unroll
                for (int hb = 0; hb < 4; ++hb) {
                    qa[hb] = load_q_operand(s_q + (rr * 64 + hb * 16 + n) * kQStride, g);
#pragma unroll
                    for (int i = 0; i < 4; ++i) wq[hb][i] = s_wq[rr * 64 + hb * 16 + 4 * g + i];
                }
            }
            float mine = -INFINITY;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int tb = tg + 16 * j;
                if (kb[j].live && tb < v) {
                    const float s = score_block(qa, wq, kb[j]);
                    if (g == j && tb + n < v) mine = s;
                }
            }
            const int t = tg + lane;
            if (t < t_end) a.scores[(size_t)r * a.score_stride + t] = mine;
        }
    }

    // -inf for the part of the chunk past every row's span.
    for (int rr = 0; rr < G; ++rr) {
        float* srow = a.scores + (size_t)(r0 + rr) * a.score_stride;
        for (int t = t_comp + threadIdx.x; t < t_end; t += 256) srow[t] = -INFINITY;
    }
}

template <int G>
hipError_t launch_g(const IndexArgs& a, hipStream_t stream) {
    dim3 grid((a.score_stride + kChunk - 1) / kChunk, a.n_rows / G);
    index_scores_kernel<G><<<grid, 256, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace

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
