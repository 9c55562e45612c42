/*
 * dsa_bw.h -- C ABI of libdsa_bw.so: plain bandwidth kernels that the
 * benchmark runs beside the step, so that its roofline states what this
 * GPU's HBM delivers in the same run next to the vendor peak.  They are
 * measurement tools, not part of the DSA step.
 *
 * Both return 0 when the kernel was enqueued on `stream`, -1 for a NULL
 * pointer or a size that is not a positive multiple of 16 bytes, -5 when the
 * HIP runtime refused the launch.  All pointers are device memory owned by
 * the caller, 16-byte aligned.
 */
#ifndef DSA_BW_H
#define DSA_BW_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Reads `bytes` from `src` once, in 16-byte loads spread over `workgroups`
 * workgroups of 256 threads (each a contiguous range), and writes one
 * uint32 fold of what each thread read to sink[workgroups * 256] (so the
 * loads cannot be removed).
 */
int dsa_bw_stream_read(const void* src, size_t bytes, int32_t workgroups, uint32_t* sink, hipStream_t stream);

/* dsa_bw_stream_read with the non-temporal hint on every load (each load
 * instruction reads whole 128-byte lines). */
int dsa_bw_stream_read_nt(const void* src, size_t bytes, int32_t workgroups, uint32_t* sink, hipStream_t stream);

/* Copies `bytes` from `src` to `dst` in 16-byte loads and stores, the same
 * partition as dsa_bw_stream_read. */
int dsa_bw_copy(const void* src, void* dst, size_t bytes, int32_t workgroups, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_BW_H */
