/*
 * Measured ceilings of the GPU, reported by the benchmark beside the
 * data-sheet peaks it takes its roofline fractions against (HBM 8 TB/s, dense
 * bf16 MFMA 2.5 PFLOP/s).  Built as libqlora_peaks.so next to the library;
 * not part of the linear layer's path.  Every call enqueues one kernel on
 * `stream` (a hipStream_t, NULL for the default stream), allocates nothing
 * and touches only the buffers it is given.  Returns 0, or 1 (a NULL
 * pointer), 2 (a size, alignment or overlap the call refuses; nothing
 * enqueued) or 3 (the launch failed).
 */
#ifndef QLORA_PEAKS_H
#define QLORA_PEAKS_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Read `bytes` (a multiple of 16) of device memory at `buf` (16-byte aligned)
 * once: contiguous = 0 in grid-stride order (consecutive threads on
 * consecutive 16-byte pieces), contiguous = 1 with each of 4096 workgroups on
 * its own contiguous range.  `sink`: one device float, written only in the
 * never-met case that keeps the loads alive.
 */
int qlora_peak_read(const void *buf, size_t bytes, int contiguous, float *sink, void *stream);

/* Copy `bytes` (a multiple of 16) between two disjoint 16-byte aligned device buffers. */
int qlora_peak_copy(const void *src, void *dst, size_t bytes, void *stream);

/*
 * 1024 workgroups of four waves, each wave `iters` iterations of eight
 * independent bf16 MFMA 32x32x16 accumulation chains on register operands;
 * qlora_peak_mfma_flops(iters) is the launch's floating-point operation count.
 */
int qlora_peak_mfma(int iters, float *sink, void *stream);
double qlora_peak_mfma_flops(int iters);

#ifdef __cplusplus
}
#endif

#endif
