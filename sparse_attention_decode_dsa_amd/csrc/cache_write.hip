// Cache write: new tokens into the paged caches, the step before the decode
// path (page "[ROCm] Support decode context parallel (DCP) for GLM-5 /
// DeepSeek-V3.2", Modifications: writes, the fused rope + KV-cache write;
// Future work: the write location computed once and fused into the write).
//
// One wavefront per token.  Lane l holds latent entries [8l, 8l + 8), lanes
// l < 32 the rope pair (2l, 2l + 1), every lane index-key entries
// (2l, 2l + 1).  The rope pair is rotated with the caller's cos/sin at the
// token's position, each product and the sum or difference rounded on its
// own (contraction into fused multiply-adds is switched off there), so the
// rotated values are fixed to the bit.
// The row's max |x| (a wavefront reduction) gives the scale max|x| / 448;
// each entry is divided by it (IEEE division), clamped to +-448 and rounded
// to E4M3FN by the hardware's round-to-nearest-even conversion.  The latent
// codes leave as one 8-byte store per lane, the rope and index codes as 2
// bytes per lane, the scales from lane 0.  Bytes 580..639 of an MLA row are
// not written.
#include "device_common.h"
#include "launch.h"
#include "query_quant.h"

namespace dsa {

namespace {

constexpr int kKvRowBytes = 640;
constexpr int kLatent = 512;
constexpr int kRopeAt = 512;    // first rope byte of an MLA row
constexpr int kScaleAt = 576;   // fp32 scale of an MLA row

__device__ __forceinline__ float scale_of(float amax) { return amax > 0.0f ? amax / 448.0f : 1.0f; }

// Two entries divided by the scale, clamped and rounded to E4M3FN (low 16 bits).
__device__ __forceinline__ uint32_t code2(float x0, float x1, float scale) {
    const float y0 = fminf(fmaxf(x0 / scale, -448.0f), 448.0f);
    const float y1 = fminf(fmaxf(x1 / scale, -448.0f), 448.0f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false) & 0xFFFFu;
}

__global__ __launch_bounds__(256) void cache_write_kernel(CacheWriteArgs a) {
    const int tok = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (tok >= a.n_tok) return;   // whole wavefront leaves together
    const int lane = threadIdx.x & 63;
    const int b = a.tok_req[tok];
    const int t = a.tok_slot[tok];
    if (b < 0 || b >= a.batch || t < 0 || t >= a.max_pages * a.page_size ||
        (a.rope_cos != nullptr && t >= a.max_pos)) {
        if (lane == 0) flag(a.status, DSA_DEV_WRITE);
        return;
    }
    const int page = a.page_table[(size_t)b * a.max_pages + (t >> a.log2_page)];
    if (page < 0 || page >= a.num_pages) {
        if (lane == 0) flag(a.status, DSA_DEV_PAGE_OOB);
        return;
    }
    const size_t row = (size_t)page * a.page_size + (t & (a.page_size - 1));

    // Inputs: 8 latent entries, a rope pair (lanes < 32), 2 index entries.
    float lat[8];
    bf16x8_to_f32(reinterpret_cast<const uint4*>(a.latent + (size_t)tok * kLatent)[lane], lat);
    float r0 = 0.0f, r1 = 0.0f;
    if (lane < 32) {
        const uint32_t w = reinterpret_cast<const uint32_t*>(a.rope + (size_t)tok * 64)[lane];
        const float x0 = __uint_as_float(w << 16), x1 = __uint_as_float(w & 0xFFFF0000u);
        if (a.rope_cos != nullptr) {
            // Each product rounded on its own: the compiler contracts a*b - c*d
            // into a fused multiply-add unless told not to.
#pragma clang fp contract(off)
            const float c = a.rope_cos[(size_t)t * 32 + lane];
            const float s = a.rope_sin[(size_t)t * 32 + lane];
            r0 = x0 * c - x1 * s;
            r1 = x0 * s + x1 * c;
        } else {
            r0 = x0;
            r1 = x1;
        }
    }
    const uint32_t wi = reinterpret_cast<const uint32_t*>(a.index_k + (size_t)tok * 128)[lane];
    const float i0 = __uint_as_float(wi << 16), i1 = __uint_as_float(wi & 0xFFFF0000u);

    // Scales.
    float am = fmaxf(fabsf(r0), fabsf(r1));
#pragma unroll
    for (int k = 0; k < 8; ++k) am = fmaxf(am, fabsf(lat[k]));
    const float s_mla = scale_of(wave_max(am));
    const float s_idx = scale_of(wave_max(fmaxf(fabsf(i0), fabsf(i1))));

    // Codes out.
    uint8_t* dst = a.kv_cache + row * kKvRowBytes;
    const uint32_t c01 = code2(lat[0], lat[1], s_mla), c23 = code2(lat[2], lat[3], s_mla);
    const uint32_t c45 = code2(lat[4], lat[5], s_mla), c67 = code2(lat[6], lat[7], s_mla);
    *reinterpret_cast<uint2*>(dst + 8 * lane) = uint2{c01 | (c23 << 16), c45 | (c67 << 16)};
    if (lane < 32) *reinterpret_cast<uint16_t*>(dst + kRopeAt + 2 * lane) = (uint16_t)code2(r0, r1, s_mla);
    *reinterpret_cast<uint16_t*>(a.k_code + row * 128 + 2 * lane) = (uint16_t)code2(i0, i1, s_idx);
    if (lane == 0) {
        *reinterpret_cast<float*>(dst + kScaleAt) = s_mla;
        a.k_scale[row] = s_idx;
    }
}

}  // namespace

hipError_t launch_cache_write(const CacheWriteArgs& a, hipStream_t stream) {
    if (a.n_tok == 0) return hipSuccess;
    cache_write_kernel<<<(a.n_tok + 3) / 4, 256, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace dsa
