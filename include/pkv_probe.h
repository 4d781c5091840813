/* pkv_probe.h -- measurement kernels, built into libpkvprobe.so on their own.
 *
 * They measure what this GPU reaches in practice, so that each kernel's roofline
 * fraction can be quoted against the measured rate as well as the published one
 * (HBM 8 TB/s, dense bf16 matrix throughput 2.5 PFLOP/s).  They are not part of
 * the paged-attention path and share no code with it.
 *
 * Every call launches on `stream` (NULL: the default stream), returns at once, and
 * give 0 on success, 1 for a bad argument, 2 for a HIP launch error.
 */
#ifndef PKV_PROBE_H
#define PKV_PROBE_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Threads per workgroup of both kernels. */
#define PKV_PROBE_THREADS 256

/* Streaming read: every 16-byte chunk of buf[0 .. bytes) is read exactly once
 * (bytes must be a positive multiple of 16; buf device memory, 16-byte aligned),
 * with coalesced nontemporal 16-byte loads, four in flight per thread over a
 * grid-stride loop.  Each thread writes the XOR of what it read to
 * sink[global thread id], so sink must hold grid * PKV_PROBE_THREADS uint32_t. */
int pkv_probe_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int32_t grid, hipStream_t stream);

/* The same read with another order: workgroup w reads the contiguous span of
 * chunks [w * span, (w + 1) * span), span = ceil(chunks / grid), in order, four
 * loads in flight per thread; each chunk still exactly once.  Same arguments,
 * buffer rules and sink. */
int pkv_probe_stream_read_spans(const void* buf, int64_t bytes, uint32_t* sink, int32_t grid,
                                hipStream_t stream);

/* Matrix-core throughput: each wave runs `iters` rounds of four independent
 * chains of v_mfma_f32_32x32x16_bf16 on register operands (no memory traffic
 * inside the loop): grid * 4 waves * iters * 4 * 32768 flops.  Each thread
 * writes one float (the sum of its accumulators) to sink[global thread id]
 * (grid * PKV_PROBE_THREADS floats). */
int pkv_probe_mfma_bf16(float* sink, int32_t iters, int32_t grid, uint32_t seed, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif
