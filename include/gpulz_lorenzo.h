/* gpulz_lorenzo.h -- the Lorenzo-quantizer front end of the chunked LZSS
 * coder, on the device.
 *
 * The GPULZStage page measures the coder on Lorenzo-quantized residuals of a
 * float field (its results paragraph), and says the LorenzoQuant stage in
 * front of it turns float32 values into integer codes (its alignment
 * paragraph).  The pages give no formula; the codes here are the plainest
 * reading, and exactly what the coder's word-size-4 workloads are:
 *
 *   q(z,y,x)   = round-half-even( f(z,y,x) / (2 eb) )   in double precision,
 *   delta      = sum over the cell's lower corners (dz,dy,dx) in {0,1}^3 of
 *                (-1)^(dz+dy+dx) q(z-dz, y-dy, x-dx), cells outside the grid
 *                counting as 0 (the integer Lorenzo predictor's residual),
 *   code       = delta + 32768, clamped to [0, 65535], stored as a u32.
 *
 * Each cell re-quantizes its own lower neighbours from the float field, so
 * every code is a pure function of the input (the codebase notes page
 * describes its fused 2-D tiled Lorenzo predictor the same way).
 */
#ifndef GPULZ_LORENZO_H
#define GPULZ_LORENZO_H

#include "gpulz.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Quantize a float32 field of nx * ny * nz cells (x fastest, then y, then z;
 * a 2-D field has nz = 1, a 1-D one ny = nz = 1) into nx * ny * nz u32 codes.
 *   d_field   device, 4-byte aligned, read only;
 *   eb        the absolute error bound, finite and > 0;
 *   d_codes   device, 4-byte aligned, nx * ny * nz u32 written;
 *   d_clamped device, one u64, overwritten with the number of cells whose
 *             code was clamped into [0, 65535].
 * Codes for non-finite values, or for |f / (2 eb)| >= 2^59, are unspecified.
 * GPULZ_ERR_INVALID_ARG (nothing enqueued): a null pointer, a zero dimension,
 * nx * ny * nz >= 2^32, an unaligned pointer, or eb not finite and > 0.
 * Nothing is allocated; the work is enqueued on `stream`. */
GPULZ_API int gpulz_lorenzo_quant(const float* d_field, uint32_t nx, uint32_t ny, uint32_t nz, double eb,
                                  uint32_t* d_codes, uint64_t* d_clamped, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GPULZ_LORENZO_H */
