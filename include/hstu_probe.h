/* Measurement probes (libhstu_probe.so), used by the benchmark to report
 * what this GPU reaches beside the published peaks: the bf16 matrix-core
 * rate of a loop of independent v_mfma_f32_32x32x16_bf16 chains with no
 * memory traffic, the HBM rate of a streaming copy, and the shader clock
 * while the matrix cores are busy. None of them is part of the HSTU layer;
 * they put the layer kernels' rooflines in context.
 *
 * Every call enqueues on `stream` (a hipStream_t, NULL = default stream),
 * allocates nothing and returns a hipError_t value (0 = success; invalid
 * arguments give hipErrorInvalidValue before anything is launched).
 */
#ifndef HSTU_PROBE_H
#define HSTU_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Workgroup size of hstu_probe_mfma_bf16: 256 threads (four waves). */
#define HSTU_PROBE_MFMA_THREADS 256

/* num_groups workgroups of four waves; each wave runs `iters` rounds of four
 * independent 32x32x16 bf16 MFMAs (4 * 32768 FLOP per round). Total work:
 * num_groups * 4 * iters * 131072 FLOP, timed by the caller around the call.
 * sink: device, >= HSTU_PROBE_MFMA_THREADS floats (written only to keep the
 * products live; its contents are meaningless). clocks: device int64
 * [2 * num_groups]: per workgroup, the s_memtime ticks (shader clock) and
 * the s_memrealtime ticks (fixed 100 MHz) across its loop, so that
 * shader GHz = 0.1 * clocks[2g] / clocks[2g + 1]. num_groups >= 1,
 * 1 <= iters <= 2^24. */
int hstu_probe_mfma_bf16(int num_groups, int iters, float *sink, int64_t *clocks, void *stream);

/* dst[0, bytes) = src[0, bytes): 16-byte vector loads and stores, one
 * workgroup per contiguous 16 KB chunk. src and dst device, 16-byte
 * aligned, not overlapping; bytes a multiple of 16, below 2^45. */
int hstu_probe_copy(const void *src, void *dst, size_t bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* HSTU_PROBE_H */
