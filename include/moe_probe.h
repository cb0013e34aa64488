/*
 * moe_probe.h -- device-memory rate probes shipped beside the MoE FFN library
 * (libmoe_native.so).  They are measurement instruments, not steps of the
 * layer: the benchmark times them to state, for this device, the HBM rate a
 * plain streaming read, a streaming write and a copy reach, and sets the
 * layer's kernels against those rates (the published 8 TB/s is a nominal
 * peak no access pattern reaches).
 *
 * Conventions: device pointers owned by the caller, 16-byte aligned, byte
 * counts multiples of 16 (MOE_ERR_MISALIGNED otherwise); a null pointer is
 * MOE_ERR_INVALID_ARG; bytes == 0 is a no-op; each call only enqueues one
 * kernel on `stream` and maps a launch error to MOE_ERR_LAUNCH (status codes
 * of moe_native.h).
 */
#ifndef MOE_PROBE_H
#define MOE_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads all `bytes` of src once (non-temporal 16-byte loads, a contiguous
 * chunk per workgroup); writes at most one word to sink[0] (its value means
 * nothing). */
int moe_probe_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);

/* Writes all `bytes` of dst once with a fixed pattern (16-byte stores). */
int moe_probe_write(void* dst, size_t bytes, hipStream_t stream);

/* dst = src over `bytes` (non-temporal 16-byte loads and stores); the
 * buffers must not overlap. */
int moe_probe_copy(const void* src, void* dst, size_t bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PROBE_H */
