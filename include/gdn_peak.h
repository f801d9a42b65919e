/*
 * gdn_peak.h -- measured-peak microbenchmarks for MI355X (gfx950), in their
 * own library (libgdn_peak.so), apart from the gated delta-rule entry points.
 *
 * The roofline fractions the benchmark reports are taken against the
 * published peaks; these loops measure what the chip delivers on the same
 * instructions, as context for those fractions.  They compute nothing of the
 * method.
 *
 * gdn_peak_mfma_loop: every wave of `blocks` workgroups of 256 threads runs
 * `iters` rounds of 8 independent accumulations from register operands, then
 * writes one float per thread to `sink` (device memory of blocks * 256
 * floats, written; it keeps the loop from being removed).
 *   kind 0: v_mfma_f32_16x16x32_bf16 (16384 flops per wave instruction)
 *   kind 1: v_mfma_f32_16x16x4_f32   (2048 flops per wave instruction)
 *   kind 2: v_fma_f32, not packed    (128 flops per wave instruction)
 * Flops per call = blocks * 4 waves * iters * 8 * (flops per instruction).
 * Returns 0 on success, -1 for a bad argument (kind, blocks < 1, iters < 1,
 * NULL sink), -2 if the launch fails.  Asynchronous on `stream` (a
 * hipStream_t; NULL = the default stream).
 */
#ifndef GDN_PEAK_H
#define GDN_PEAK_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

int gdn_peak_mfma_loop(int kind, int iters, int blocks, float *sink, void *stream);

/*
 * gdn_peak_read: `blocks` workgroups of 256 threads read the first
 * floor(bytes / 16) * 16 bytes of `buf` (device memory, 16-byte aligned,
 * not modified) once, in 16-byte words at a grid stride, and write one float
 * per thread to `sink` (blocks * 256 floats, written).  The measured
 * streaming-read rate; the benchmark also uses it to evict the caches without
 * leaving dirty lines behind.  Returns 0, -1 for a bad argument (NULL
 * pointer, misaligned buf, blocks < 1) or -2 if the launch fails.
 */
int gdn_peak_read(const void *buf, size_t bytes, int blocks, float *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif
