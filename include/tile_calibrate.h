/*
 * tile_calibrate.h - a sustained-rate probe of the bf16 matrix cores of AMD Instinct
 * MI355X (gfx950), for reading measured kernel rates against what the chip sustains.
 *
 * The published dense bf16 peak (2.5 PFLOP/s) assumes the 2.4 GHz clock. Under sustained
 * matrix load the clock falls with the switching activity of the operands, so the rate a
 * kernel can reach depends on its data. This probe keeps every SIMD's matrix core busy
 * with v_mfma_f32_32x32x16_bf16 (two waves per SIMD, four independent accumulation
 * chains per wave, operands rotating over eight register pairs) and nothing else, with
 * either all-zero operands or random bf16 operands in [-1, 1). Its rate with random
 * operands is the matrix-core ceiling for random bf16 data.
 */
#ifndef TILE_CALIBRATE_H
#define TILE_CALIBRATE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TILE_CAL_OK       0   /* success: the kernel was enqueued                             */
#define TILE_CAL_EINVAL  -1   /* NULL out or flops, iterations < 1 or > 2^24, random_operands
                                 not 0/1, or out_floats < tile_mfma_calibrate_out_floats()   */
#define TILE_CAL_ELAUNCH -4   /* a failed device query, or hipGetLastError() set after the launch */

/* Elements of `out` one call writes: 256 per workgroup, two workgroups per compute unit of
 * the current device (0 if the device query fails). */
size_t tile_mfma_calibrate_out_floats(void);

/*
 * tile_mfma_calibrate - enqueue the probe on `stream` (a hipStream_t as void*, NULL for the
 * default stream) of the current device.
 *
 *   out              device pointer, fp32, at least tile_mfma_calibrate_out_floats()
 *                    elements; each thread writes the sum of its accumulators (so the
 *                    products cannot be optimised away). Owned by the caller.
 *   out_floats       the size of out, in elements.
 *   iterations       1 .. 2^24; each wave issues 32 * iterations MFMAs.
 *   random_operands  0: all-zero operands; 1: random bf16 operands in [-1, 1).
 *   flops            host pointer; receives the floating-point operations of the call
 *                    (2 * 32 * 32 * 16 per MFMA).
 *
 * Validates on the host before any launch; allocates nothing; returns without
 * synchronising. Time it with events on the same stream.
 */
int tile_mfma_calibrate(float* out, size_t out_floats, int iterations, int random_operands,
                        double* flops, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TILE_CALIBRATE_H */
