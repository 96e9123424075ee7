/* kda_peaks.h -- microbenchmarks of the MI355X peaks that libkda's roofline
 * figures are quoted against (libkda_peaks.so; not part of the KDA operator).
 *
 * The roofline peaks are datasheet figures (dense bf16 matrix products
 * 2.5 PFLOP/s, FP32 matrix products 157.3 TFLOP/s, HBM 8 TB/s).  These probes
 * time what the matrix cores deliver on this machine, so a roofline fraction can
 * be read against both, and time whether a wave's own vector (VALU) work
 * overlaps its dependent matrix-core products.
 *
 * kda_peaks_probe: asynchronous on `stream`; the caller times it (events on
 * the same stream).  Every thread writes one float of `sink` (a value derived
 * from its results, so the work cannot be removed): sink must hold
 * blocks * threads floats of device memory owned by the caller.
 *
 * kind (per wave, per loop iteration):
 *   KDA_PEAK_MFMA_BF16      4 independent v_mfma_f32_32x32x16_bf16 (32,768 FLOP each)
 *   KDA_PEAK_MFMA_FP32      4 independent v_mfma_f32_16x16x4f32    (2,048 FLOP each)
 *   KDA_PEAK_CHAIN_BF16     1 v_mfma_f32_32x32x16_bf16 into the previous iteration's accumulator
 *   KDA_PEAK_CHAIN_BF16_VALU  the same chain plus 8 independent FP32 FMAs (VALU)
 *   KDA_PEAK_VALU           the 8 independent FP32 FMAs alone
 * Returns 0 on success, 1 for an invalid argument (unknown kind, iters < 1,
 * blocks < 1, threads not 64/128/256/512, null sink), 4 for a launch error.
 */
#ifndef KDA_PEAKS_H
#define KDA_PEAKS_H

#include <hip/hip_runtime.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_PEAKS_API __attribute__((visibility("default")))

enum {
  KDA_PEAK_MFMA_BF16 = 0,
  KDA_PEAK_MFMA_FP32 = 1,
  KDA_PEAK_CHAIN_BF16 = 2,
  KDA_PEAK_CHAIN_BF16_VALU = 3,
  KDA_PEAK_VALU = 4
};

KDA_PEAKS_API int kda_peaks_probe(int kind, int iters, int blocks, int threads, float* sink,
                                  hipStream_t stream);

/* Streaming device copy of `bytes` bytes from src to dst (device memory owned
 * by the caller, not overlapping): 16-byte non-temporal loads and stores, a
 * grid-stride loop over `blocks` workgroups of 256 threads.  Measures the HBM
 * bandwidth a plain copy reaches (2 x bytes moved).  Returns 0 on success, 1
 * if a pointer is null or not 16-byte aligned, bytes is not a multiple of 16
 * or blocks < 1, 4 for a launch error. */
KDA_PEAKS_API int kda_peaks_copy(const void* src, void* dst, size_t bytes, int blocks,
                                 hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* KDA_PEAKS_H */
