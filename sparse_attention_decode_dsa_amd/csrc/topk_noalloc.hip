// dsa_topk_noalloc: dsa_topk for callers that cannot allocate device memory.
//
// dsa_topk takes its candidate workspace from the caller.  This variant uses
// a fixed array that the library holds in device memory instead (one copy per
// GPU, for the life of the process), so a call allocates nothing.  The
// array's device address is looked up once per device, with that device
// current, and kept; kernels only ever see that address (the array's name in
// host code is a host-side stand-in, not a device address).
#include <mutex>

#include "dsa.h"
#include "launch.h"

namespace {

static_assert(DSA_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
__device__ __align__(256) uint8_t scratch[DSA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices];   // device address of `scratch` on each device, once looked up

// Address of the current device's copy of `scratch`; nullptr if it cannot be
// found (no device, or the lookup failed).
void* scratch_on_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
        g_scratch[dev] = p;
    }
    return g_scratch[dev];
}

}  // namespace

extern "C" int dsa_topk_noalloc(const float* scores, int32_t score_stride, const int32_t* row_vis,
                                int32_t n_rows, int32_t top_k, int32_t n_splits, int32_t* topk_idx,
                                int32_t* topk_count, int32_t* status, hipStream_t stream) {
    const int rc = dsa::topk_validate(scores, score_stride, row_vis, n_rows, top_k, n_splits, topk_idx,
                                      topk_count, status);
    if (rc != DSA_OK || n_rows == 0) return rc;
    // The candidates are written before they are read, so the array's
    // leftover contents from an earlier call never matter.
    const size_t need = dsa_topk_workspace_size(n_rows, top_k, n_splits);
    if (need > DSA_NOALLOC_SCRATCH_BYTES) return DSA_ERR_SCRATCH;
    void* ws = nullptr;
    if (need > 0) {
        ws = scratch_on_current_device();
        if (ws == nullptr) return DSA_ERR_LAUNCH;
    }
    return dsa::topk_launch(scores, score_stride, row_vis, n_rows, top_k, n_splits, ws,
                            DSA_NOALLOC_SCRATCH_BYTES, topk_idx, topk_count, status, stream);
}
