/*
 * mla_peaks.h - measurement kernels for roofline denominators.
 *
 * Not part of the decode path.  They give the achievable HBM read bandwidth
 * and bf16 MFMA throughput of the device the library runs on, measured the way
 * FlashMLA PR 233 ("Performance") reports its decode kernel against measured
 * read and bf16 peaks rather than data-sheet numbers.
 */
#ifndef MLA_PEAKS_H
#define MLA_PEAKS_H

#include <stddef.h>
#include <stdint.h>

#include "mla_decode.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Read `bytes` (a multiple of 16) of device memory at `buf` with 16-byte
 * vector loads from every CU, `iters` times, on `stream`; *ms_out receives the
 * median time of one pass in milliseconds.  `sink` is a device buffer of at
 * least 1 MiB that receives a reduction so the loads are not elided.
 * Synchronises the stream.  Errors: MLA_ERR_INVALID_ARG, MLA_ERR_HIP.
 */
mla_status mla_peak_stream_read(const void* buf, size_t bytes, void* sink, int32_t iters,
                                float* ms_out, void* stream);

/*
 * Dense bf16 MFMA throughput (v_mfma_f32_16x16x32_bf16 with independent
 * accumulators on every wave of every CU); *tflops_out receives the median of
 * `iters` timed launches in TFLOP/s.  `sink` as above.  Synchronises the stream.
 */
mla_status mla_peak_mfma_bf16(void* sink, int32_t iters, float* tflops_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_PEAKS_H */
