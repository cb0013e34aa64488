/*
 * moe_probe.h -- device-memory rate probes shipped beside the MoE FFN library
 * (libmoe_native.so).  They are measurement instruments, not steps of the
 * layer: the benchmark times them to state, for this device, the HBM rate a
 * plain streaming read, a streaming write and a copy reach, and sets the
 * layer's kernels against those rates (the published 8 TB/s is a nominal
 * peak no access pattern reaches); the access-order probes state what the
 * order of a GEMM tile's weight reads and output writes, and the LDS-DMA
 * ring the GEMMs load through, cost by themselves; the GEMM-loop probe
 * (libmoe_native's gemm_probe.hip) runs the GEMMs' K loop with no gather
 * and no epilogue; the matrix-core and LDS-read probes state the bf16 MFMA
 * rate and the LDS read rate a compute unit reaches with nothing else in
 * the way, and the engine clock it runs them at.
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

/* Access-order probes.  The buffer is a sequence of panels of `rows` rows of
 * `row_bytes` bytes (`bytes` a whole number of panels); one 512-thread
 * workgroup per compute unit walks whole panels, each piece column by piece
 * column: bytes [s, s + piece_bytes) of every row, then the next s -- the
 * order in which a GEMM tile streams a weight panel in K slabs (piece_bytes
 * == row_bytes: front to back).  16-byte accesses, eight in flight per
 * thread.  row_bytes and piece_bytes are multiples of 16 and piece_bytes
 * divides row_bytes (MOE_ERR_MISALIGNED otherwise); rows >= 1, row_bytes
 * and piece_bytes >= 16 and bytes a multiple of rows * row_bytes
 * (MOE_ERR_INVALID_ARG otherwise); one panel below 2^35 bytes
 * (MOE_ERR_UNSUPPORTED).
 *
 * moe_probe_read_pieces reads every byte once (non-temporal loads) and
 * writes at most one word to sink[0] (its value means nothing);
 * moe_probe_write_pieces writes every byte once with a fixed pattern,
 * non-temporal stores when `nontemporal` is nonzero.
 *
 * moe_probe_write_tiles writes the same bytes (same pattern, same argument
 * rules) in the order the weight-gradient GEMM's output tiles reach memory:
 * each piece column of a panel (rows x piece_bytes) is a tile written whole,
 * row after row, by one workgroup, and the pieces of one panel go to
 * neighbouring workgroups of one XCD, so they are written at the same time. */
int moe_probe_read_pieces(const void* src, size_t bytes, int32_t row_bytes, int32_t rows,
                          int32_t piece_bytes, uint32_t* sink, hipStream_t stream);
int moe_probe_write_pieces(void* dst, size_t bytes, int32_t row_bytes, int32_t rows,
                           int32_t piece_bytes, int32_t nontemporal, hipStream_t stream);
int moe_probe_write_tiles(void* dst, size_t bytes, int32_t row_bytes, int32_t rows,
                          int32_t piece_bytes, int32_t nontemporal, hipStream_t stream);

/* The GEMMs' load pipeline without their compute: one 512-thread workgroup
 * per compute unit streams contiguous 1 MiB panels of src in 32 KiB slabs
 * through `stages` (2..5) LDS stages by LDS DMA (non-temporal), with a wait
 * for the current slab and a workgroup barrier per slab.  `bytes` is a
 * multiple of 1 MiB and stages in [2, 5] (MOE_ERR_INVALID_ARG otherwise);
 * writes at most one word to sink[0]. */
int moe_probe_lds_ring(const void* src, size_t bytes, int32_t stages, uint32_t* sink,
                       hipStream_t stream);

/* The grouped FFN GEMMs' K loop alone: E experts' products
 * a[e*Cp .. e*Cp+Cp) (rows of K bf16) times b[e] ([N][K] bf16) over the same
 * 256x256 tiles, 64-deep slabs, LDS-DMA rings (two A and three B stages),
 * persistent XCD-aware tile walk and bf16 MFMA as the layer's kernels, with no
 * gather, no epilogue and no output: each finished tile folds into a word
 * written to sink[0] only in a case that does not occur.  Eight waves of
 * 128x64 outputs each, as the layer's kernels.  Device pointers, a and b
 * 16-byte aligned (MOE_ERR_MISALIGNED); null pointers or negative sizes are
 * MOE_ERR_INVALID_ARG; Cp and N multiples of 256 and K of 64, one expert's a
 * rows and b below 2 GiB (MOE_ERR_UNSUPPORTED); any size 0 is a no-op. */
int moe_probe_gemm_loop(const uint16_t* a, const uint16_t* b, int32_t E, int32_t Cp, int32_t N,
                        int32_t K, uint32_t* sink, hipStream_t stream);

/* The matrix cores alone: `groups` workgroups of 512 threads (one per
 * compute unit: each holds 96 KB of LDS; pass at most the device's compute
 * unit count), every wave issuing `iters` x 4 bf16 32x32x16 MFMAs on four
 * independent accumulators (32768 flops each) and nothing else.  The LDS read
 * path alone: the same workgroups, every wave issuing `iters` x 8 16-byte
 * LDS reads per lane (1 KB per wave and read, eight in flight, no bank
 * conflicts, no ALU work).  Each workgroup g writes clocks[2g] = engine-clock
 * ticks (s_memtime) and clocks[2g + 1] = 100 MHz constant-clock ticks
 * (s_memrealtime) over its loop, bracketed by workgroup barriers, so
 * 1e8 * clocks[2g] / clocks[2g + 1] is the engine clock in Hz.  clocks is a
 * device buffer of 2 * groups words, 8-byte aligned.  A null clocks,
 * groups < 0 or iters < 1 is MOE_ERR_INVALID_ARG; groups == 0 is a no-op. */
int moe_probe_mfma_rate(int32_t groups, int32_t iters, uint64_t* clocks, hipStream_t stream);
int moe_probe_lds_read(int32_t groups, int32_t iters, uint64_t* clocks, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PROBE_H */
