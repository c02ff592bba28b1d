/*
 * sharq_peak.h -- measurement kernels shipped beside the SharQ layer (gfx950).
 *
 * The layer's kernels are reported as fractions of the MI355X's published
 * peaks (dense MXFP4 MFMA, HBM bandwidth).  These two entry points measure
 * what the same chip reaches in practice on the same run, so a benchmark can
 * also report fractions of the measured peaks.  They are not part of the
 * layer and compute nothing the layer uses.
 *
 * Conventions as in sharq.h: device pointers, caller-owned buffers,
 * asynchronous on `stream` (timing is the caller's: events around the call),
 * host-side argument checks before any launch, no allocation.
 */
#ifndef SHARQ_PEAK_H
#define SHARQ_PEAK_H

#include <stddef.h>
#include <stdint.h>

#include "sharq.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Back-to-back block-scaled FP4 MFMAs (v_mfma_scale_f32_16x16x128_f8f6f4,
 * both operands E2M1, E8M0 scales), eight independent accumulators per
 * wave, sixteen waves per compute unit, on operand bytes the caller supplies
 * (the chip is power-limited, so the rate depends on the data: random bytes
 * give the draw of a dense operand, bytes with two zero codes in every four
 * that of a 2:4 backbone).
 *   operands_dev: device, >= 6144 bytes, 16-byte aligned: E2M1 operand bytes,
 *                 bytes 0..4095 the four first operands (1 KiB each, 16 bytes
 *                 per lane), 4096..6143 the two second operands; its first
 *                 64 bytes also give the scale bytes (clamped to E8M0
 *                 120..134);
 *   iters:        loop trips per wave (1 .. 1<<20), eight MFMAs each;
 *   sink_dev:     device float[1], written only if the accumulators happen to
 *                 sum to an impossible sentinel (keeps the work alive);
 *   flops_out:    host; receives the flops the launch executes
 *                 (2*16*16*128 per MFMA).
 * Errors: INVALID_ARG (null, size, alignment, iters), UNSUPPORTED (not
 * gfx950), HIP. */
sharq_status sharq_peak_fp4_mfma(const void* operands_dev, size_t operand_bytes, int32_t iters, float* sink_dev,
                                 double* flops_out, void* stream);

/* Streaming read of `bytes` (a multiple of 16, >= 1 MiB, 16-byte aligned)
 * with 16-byte loads over a grid that fills every compute unit; the loaded
 * words are folded into one value per thread and written to sink_dev[0] only
 * if it equals an impossible sentinel.  bytes_out (host) receives the bytes
 * read.  Use a buffer larger than the 256 MB last-level cache.
 * Errors: INVALID_ARG, UNSUPPORTED (not gfx950), HIP. */
sharq_status sharq_peak_read(const void* buf_dev, size_t bytes, uint32_t* sink_dev, double* bytes_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SHARQ_PEAK_H */
