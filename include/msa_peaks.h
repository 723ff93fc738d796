/*
 * msa_peaks.h -- attainable-rate probes for the MI355X roofline (measurement
 * only; not part of the attention path).  Built as libmsa_peaks.so next to
 * libmsa.so and used by the benchmark to report each kernel against what the
 * device actually sustains, besides the data-sheet peaks.
 *
 * Both calls allocate their own device memory, run on a private stream, time
 * with HIP events and synchronise before returning.  Return 0 on success or a
 * negative value (HIP error or bad argument).
 */
#ifndef MSA_PEAKS_H_
#define MSA_PEAKS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming read of `bytes` (multiple of 16, > 0) of device memory, 16 bytes
 * per lane per non-temporal load, `iters` timed passes; *gbps = bytes * iters / time. */
int msa_peak_hbm_read(size_t bytes, int iters, double* gbps);

/* Device-to-device copy of `bytes` (multiple of 16, > 0), 16 bytes per lane,
 * non-temporal stores, `iters` timed passes; *gbps counts each byte once read and once written:
 * 2 * bytes * iters / time. */
int msa_peak_hbm_copy(size_t bytes, int iters, double* gbps);

/* Gather of `blocks` 4 KiB blocks at scattered places of a buffer of
 * 2 * blocks * 4 KiB (a seeded permutation, fixed per call), 16 bytes per lane
 * per non-temporal load, one wave per block, `iters` timed passes; *gbps =
 * blocks * 4 KiB * iters / time.  The access pattern of a block-paged KV pool. */
int msa_peak_hbm_gather(int32_t blocks, int iters, double* gbps);

/* v_mfma_f32_32x32x16_bf16 issued back to back on independent accumulators by
 * every wave of a full-device grid, operands in registers, `iters` loop trips;
 * *tflops = dense bf16 FLOPs / time. */
int msa_peak_mfma_bf16(int iters, double* tflops);

#ifdef __cplusplus
}
#endif

#endif /* MSA_PEAKS_H_ */
