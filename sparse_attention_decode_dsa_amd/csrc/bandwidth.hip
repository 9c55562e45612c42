// Plain streaming-read and copy kernels (libdsa_bw.so): the measured HBM
// ceilings that the benchmark reports beside the vendor peak.  Each
// workgroup walks one contiguous range; every thread keeps kInFlight 16-byte
// loads outstanding before it uses any of them.  The read comes with and
// without the non-temporal hint: over whole 128-byte lines the hint reads
// faster on this chip.
#include <hip/hip_runtime.h>

#include "dsa_bw.h"

namespace {

constexpr int kThreads = 256;
constexpr int kInFlight = 8;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool kNt>
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                               size_t per_wg, uint32_t* __restrict__ sink) {
    const size_t b0 = (size_t)blockIdx.x * per_wg;
    const size_t b1 = b0 + per_wg < n16 ? b0 + per_wg : n16;
    uint32_t acc = 0;
    for (size_t i = b0 + threadIdx.x; i < b1; i += (size_t)kThreads * kInFlight) {
        u32x4 v[kInFlight];
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) {
            const size_t j = i + (size_t)u * kThreads;
            if constexpr (kNt) v[u] = j < b1 ? __builtin_nontemporal_load(src + j) : u32x4{0u, 0u, 0u, 0u};
            else v[u] = j < b1 ? src[j] : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = acc;
}

__global__ __launch_bounds__(kThreads) void copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                        size_t n16, size_t per_wg) {
    const size_t b0 = (size_t)blockIdx.x * per_wg;
    const size_t b1 = b0 + per_wg < n16 ? b0 + per_wg : n16;
    for (size_t i = b0 + threadIdx.x; i < b1; i += (size_t)kThreads * kInFlight) {
        uint4 v[kInFlight];
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) {
            const size_t j = i + (size_t)u * kThreads;
            if (j < b1) v[u] = src[j];
        }
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) {
            const size_t j = i + (size_t)u * kThreads;
            if (j < b1) dst[j] = v[u];
        }
    }
}

bool bad(const void* p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15) != 0; }

}  // namespace

template <bool kNt>
int stream_read(const void* src, size_t bytes, int32_t workgroups, uint32_t* sink, hipStream_t stream) {
    if (bad(src) || sink == nullptr || bytes == 0 || bytes % 16 != 0 || workgroups < 1) return -1;
    const size_t n16 = bytes / 16;
    const size_t per = (n16 + workgroups - 1) / workgroups;
    stream_read_kernel<kNt><<<workgroups, kThreads, 0, stream>>>(static_cast<const u32x4*>(src), n16, per, sink);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int dsa_bw_stream_read(const void* src, size_t bytes, int32_t workgroups, uint32_t* sink,
                                  hipStream_t stream) {
    return stream_read<false>(src, bytes, workgroups, sink, stream);
}

extern "C" int dsa_bw_stream_read_nt(const void* src, size_t bytes, int32_t workgroups, uint32_t* sink,
                                     hipStream_t stream) {
    return stream_read<true>(src, bytes, workgroups, sink, stream);
}

extern "C" int dsa_bw_copy(const void* src, void* dst, size_t bytes, int32_t workgroups, hipStream_t stream) {
    if (bad(src) || bad(dst) || bytes == 0 || bytes % 16 != 0 || workgroups < 1) return -1;
    const size_t n16 = bytes / 16;
    const size_t per = (n16 + workgroups - 1) / workgroups;
    copy_kernel<<<workgroups, kThreads, 0, stream>>>(static_cast<const uint4*>(src), static_cast<uint4*>(dst), n16,
                                                     per);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}
