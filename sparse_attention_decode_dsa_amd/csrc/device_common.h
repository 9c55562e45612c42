// Device helpers shared by the gfx950 kernels: vector types, MFMA wrappers,
// fp8 / bf16 conversions, wavefront reductions and a workgroup scan.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsa.h"

namespace dsa {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// D(16x16 f32) += A(16x128 fp8) * B(128x16 fp8).  Lane l holds row/column
// l % 16 of A/B and 32 K-bytes for lane group l / 16; D lane l holds rows
// 4*(l/16) + i of column l % 16.  Zero scale operands select the unscaled
// v_mfma_f32_16x16x128_f8f6f4 (format 0 = E4M3 for both operands).
__device__ __forceinline__ v4f mfma_fp8_16x16x128(const v8i& a, const v8i& b, const v4f& c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// D(16x16 f32) += A(16x32 fp8) * B(32x16 fp8) (v_mfma_f32_16x16x32_fp8_fp8,
// E4M3 both); lane l holds row/column l % 16 and 8 K-bytes for lane group
// l / 16.
__device__ __forceinline__ v4f mfma_fp8_16x16x32(const v2i& a, const v2i& b, const v4f& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(__builtin_bit_cast(long, a), __builtin_bit_cast(long, b),
                                                     c, 0, 0, 0);
}

// D(16x16 f32) += A(16x32 bf16) * B(32x16 bf16); lane l holds row/column
// l % 16 and the 8 K-values of lane group l / 16.
__device__ __forceinline__ v4f mfma_bf16_16x16x32(const v8bf& a, const v8bf& b, const v4f& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Two E4M3FN bytes (the low or, with HIGH, the high half of `w`) to two
// bf16; exact, since every E4M3FN value is a bf16 value.
template <bool HIGH>
__device__ __forceinline__ v2bf fp8x2_to_bf16x2(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HIGH);
}

// Eight E4M3FN bytes (two dwords) to eight bf16.
__device__ __forceinline__ v8bf fp8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
    v2bf a = fp8x2_to_bf16x2<false>(lo), b = fp8x2_to_bf16x2<true>(lo);
    v2bf c = fp8x2_to_bf16x2<false>(hi), d = fp8x2_to_bf16x2<true>(hi);
    v8bf r;
    r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
    r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
    return r;
}

// fp32 -> bf16 bits, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Order-preserving map of an fp32 onto uint32: a < b  <=>  key(a) < key(b)
// for non-NaN values, and -0.0 and +0.0 share one key (they are equal
// scores); -inf maps to 0x007FFFFF.
__device__ __forceinline__ uint32_t monotone_key(float f) {
    uint32_t u = (f == 0.0f) ? 0u : __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_to_float(uint32_t k) {
    uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(u);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}
// Lane exchange inside rows of 16 lanes by DPP (a VALU operand modifier,
// no LDS round trip).  0xB1 / 0x4E: quad_perm [1,0,3,2] / [2,3,0,1];
// 0x141: mirror within each half row; 0x140: mirror within the row.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// All-reductions over the 16 lanes that share l / 16: after the two quad
// steps every lane holds its quad's result, the half-row mirror pairs the
// two quads of a half row, the row mirror pairs the two half rows.
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp<0xB1>(v));
    v = fmaxf(v, dpp<0x4E>(v));
    v = fmaxf(v, dpp<0x141>(v));
    v = fmaxf(v, dpp<0x140>(v));
    return v;
}
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp<0xB1>(v);
    v += dpp<0x4E>(v);
    v += dpp<0x141>(v);
    v += dpp<0x140>(v);
    return v;
}

// Lane i receives lane i - N of its row of 16 (0 below the row start).
template <int N>
__device__ __forceinline__ uint32_t row_shr(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x110 + N, 0xF, 0xF, true);
}

// Wave-uniform maximum / minimum of a uint32: DPP within each row of 16
// lanes (quad swaps, then the half-row and row mirrors), then the four rows
// through scalar reads.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, dpp_u32<0xB1>(v));
    v = max(v, dpp_u32<0x4E>(v));
    v = max(v, dpp_u32<0x141>(v));
    v = max(v, dpp_u32<0x140>(v));
    return max(max((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16)),
               max((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48)));
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
    v = min(v, dpp_u32<0xB1>(v));
    v = min(v, dpp_u32<0x4E>(v));
    v = min(v, dpp_u32<0x141>(v));
    v = min(v, dpp_u32<0x140>(v));
    return min(min((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16)),
               min((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48)));
}

// Inclusive scan of uint32 over a wavefront: four DPP row shifts scan each
// row of 16 lanes, then the three lower rows' totals are added in.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) {
    const int lane = threadIdx.x & (kWave - 1);
    v += row_shr<1>(v);
    v += row_shr<2>(v);
    v += row_shr<4>(v);
    v += row_shr<8>(v);
    const uint32_t t0 = __builtin_amdgcn_readlane(v, 15);
    const uint32_t t1 = __builtin_amdgcn_readlane(v, 31);
    const uint32_t t2 = __builtin_amdgcn_readlane(v, 47);
    v += (lane >= 16 ? t0 : 0u) + (lane >= 32 ? t1 : 0u) + (lane >= 48 ? t2 : 0u);
    return v;
}

// Exclusive scan over a workgroup of NT threads (NT a multiple of 64,
// NT / 64 <= 64).  `scratch` holds NT / 64 + 1 words of LDS.  Returns the
// exclusive prefix and writes the total into *total.  Contains barriers:
// every thread of the workgroup must call it.
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* scratch, uint32_t* total) {
    constexpr int NW = NT / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
    uint32_t inc = wave_inclusive_scan(v);
    if (lane == kWave - 1) scratch[w] = inc;
    __syncthreads();
    if (w == 0) {
        uint32_t x = lane < NW ? scratch[lane] : 0u;
        uint32_t xi = wave_inclusive_scan(x);
        if (lane < NW) scratch[lane] = xi - x;
        if (lane == NW - 1) scratch[NW] = xi;
    }
    __syncthreads();
    uint32_t r = inc - v + scratch[w];
    *total = scratch[NW];
    __syncthreads();
    return r;
}

// Maximum / sum over the four 16-lane rows of a wavefront for each lane
// position l % 16 (every lane gets the result).  permlane16_swap(x, x)
// returns (rows 0,0,2,2) and (rows 1,1,3,3) of x; permlane32_swap(y, y)
// returns (rows 0,1,0,1) and (rows 2,3,2,3) of y.  Every lane adds in the
// same order, so the sum is identical across the rows.
__device__ __forceinline__ float rows4_max(float v) {
    const uint32_t u = __float_as_uint(v);
    const auto s = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const float w = fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
    const uint32_t uw = __float_as_uint(w);
    const auto t = __builtin_amdgcn_permlane32_swap(uw, uw, false, false);
    return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}
__device__ __forceinline__ float rows4_sum(float v) {
    const uint32_t u = __float_as_uint(v);
    const auto s = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const float w = __uint_as_float(s[0]) + __uint_as_float(s[1]);
    const uint32_t uw = __float_as_uint(w);
    const auto t = __builtin_amdgcn_permlane32_swap(uw, uw, false, false);
    return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}

// Forces a value into registers at this point and hides where it came
// from, so the compiler cannot re-create it later by reloading memory.
template <typename T>
__device__ __forceinline__ void pin(T& v) {
    asm volatile("" : "+v"(v));
}

// Workgroup barrier for LDS traffic only.  __syncthreads() is a release /
// acquire fence at workgroup scope, which drains every outstanding global
// load of the wavefront (vmcnt(0)), LDS-direct loads included; a kernel
// that keeps such loads in flight across barriers waits for them itself,
// with counts it knows, and synchronises with this: each wavefront's LDS
// reads and writes complete (lgkmcnt(0)), then the barrier.  The empty asm
// statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_sync() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));  // vmcnt 63: no wait; lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// LDS byte offset of a pointer into __shared__ memory (its low 32 bits).
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
    return (uint32_t)(uintptr_t)p;
}

// LDS-direct load (global_load_lds_dwordx4): lane i's 16 bytes at `src`
// land at LDS byte lds + 16 i; `lds` is wave-uniform
// and goes to M0.  It is written as inline assembly so that the
// compiler neither tracks it nor inserts its own waits for it: its
// wait insertion cannot always tell which LDS accesses such a load may
// overlap, and then drains every load in flight before an unrelated LDS
// access.  The caller waits with explicit vmcnt counts (in-order completion)
// before the data is read, and synchronises the workgroup with lds_sync().
__device__ __forceinline__ void lds_dma16(const void* src, uint32_t lds) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds) : "memory");
}
// The same with the non-temporal hint (for data read once).
__device__ __forceinline__ void lds_dma16_nt(const void* src, uint32_t lds) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(src), "{m0}"(lds) : "memory");
}

// A per-token scale is usable when it is a positive finite number: its bit
// pattern lies in [0x00000001, 0x7F7FFFFF] (zero, negatives, infinities and
// NaNs all fall outside).
__device__ __forceinline__ bool scale_ok(float s) {
    return __float_as_uint(s) - 1u < 0x7F7FFFFFu;
}

__device__ __forceinline__ void flag(int32_t* status, int32_t bit) {
    atomicOr(status, bit);
}

}  // namespace dsa
