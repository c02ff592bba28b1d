/*
 * sharq_check.h -- the FP4 (E2M1) conversions, the E4M3 block-scale rounding
 * and the block-scaled FP4 MFMA of the SharQ kernels, exposed so that their
 * rounding and lane layouts can be checked against their definitions on the
 * device.
 *
 * Every E2M1 code the preparation, the weight pack and the NVFP4-style path
 * write comes from the hardware converts behind this entry point, used exactly
 * as those kernels use them; it computes nothing the layer needs.
 * Conventions as in sharq.h (device pointers, caller-owned buffers,
 * asynchronous on `stream`, host-side checks before any launch).
 */
#ifndef SHARQ_CHECK_H
#define SHARQ_CHECK_H

#include <stddef.h>
#include <stdint.h>

#include "sharq.h"

#ifdef __cplusplus
extern "C" {
#endif

/* For scale s (0 <= s < n_scales) with exponent e = exps[s] (-127..125) and
 * the n values x[s][0..n) (binary32, n a multiple of 8), in groups of eight
 * consecutive values packed into one 32-bit word (value 2i in nibble 2i mod 8,
 * the lower value of a pair in the low nibble):
 *   enc[s][i]   = the codes of x / 2^e, converted with the scale 2^e inside
 *                 the convert (the preparation's way: SharQ abstract, backbone
 *                 and residual quantised to FP4 with an MX block scale);
 *   pack[s][i]  = the codes of the binary32 product x * 2^-e converted with
 *                 scale 1 (the weight pack's way, and the NVFP4-style path's);
 *   dec[s][j]   = the value of code j of enc[s] times 2^e (the residual's
 *                 dequantisation);
 *   unpack[s][j] = the value of code j of pack[s] (scale 1).
 * x_dev: float[n_scales][n]; exps_dev: int32[n_scales]; enc_dev, pack_dev:
 * uint32[n_scales][n/8]; dec_dev, unpack_dev: float[n_scales][n].
 * Errors: INVALID_ARG (null, n <= 0 or n % 8, n_scales < 1, n_scales * n >=
 * 2^31, misaligned), UNSUPPORTED (not gfx950), HIP.  Exponents outside
 * -127..125 give unspecified results. */
sharq_status sharq_check_e2m1(const float* x_dev, const int32_t* exps_dev, int64_t n, int32_t n_scales,
                              uint32_t* enc_dev, uint32_t* pack_dev, float* dec_dev, float* unpack_dev, void* stream);

/* The E4M3 block-scale rounding of the NVFP4-style path (NVFP4 per the public
 * description: an E4M3 scale per 16 values), as its kernels round the scales:
 * byte[i] and value[i] = the E4M3 nearest to x[i] (ties to the even mantissa,
 * saturating at 448), dec[i] = byte[i] decoded as their GEMM decodes it.
 * x_dev: float[n], finite and >= 0 (others: unspecified); byte_dev: uint8[n];
 * value_dev, dec_dev: float[n].
 * Errors: INVALID_ARG (null, n outside 1 .. 2^31, misaligned), UNSUPPORTED
 * (not gfx950), HIP. */
sharq_status sharq_check_e4m3(const float* x_dev, int64_t n, uint8_t* byte_dev, float* value_dev, float* dec_dev,
                              void* stream);

/* One block-scaled FP4 MFMA (v_mfma_scale_f32_16x16x128_f8f6f4, E2M1 operands,
 * E8M0 scales) per block, issued exactly as the SharQ GEMM kernels issue it on
 * operands in the tiled layout of sharq.h, so that a test can pin the operand,
 * scale and accumulator lane layouts against the definition (SharQ abstract:
 * both paths are FP4 GEMMs on block-scaled operands):
 *   d[b][m][n] = sum over k < 128 of val(A_b[m][k]) * 2^(sa_b[m][k/32] - 127)
 *                                  * val(B_b[n][k]) * 2^(sb_b[n][k/32] - 127),
 * A_b, B_b: 16 x 128 E2M1 codes, 1 KiB each in the tiled lane order (lane
 * l = row l%16 + 16 * (k/32): 16 bytes, the lower k in the low nibble);
 * sa_b, sb_b: their 64 E8M0 scale bytes in the same lane order.
 * a_dev, b_dev: uint8[n_blocks][1024] (16-byte aligned); sa_dev, sb_dev:
 * uint8[n_blocks][64]; d_dev: float[n_blocks][16][16], m-major.
 * Errors: INVALID_ARG (null, n_blocks outside 1 .. 2^20, misaligned),
 * UNSUPPORTED (not gfx950), HIP. */
sharq_status sharq_check_mfma_fp4(const uint8_t* a_dev, const uint8_t* sa_dev, const uint8_t* b_dev,
                                  const uint8_t* sb_dev, int32_t n_blocks, float* d_dev, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SHARQ_CHECK_H */
