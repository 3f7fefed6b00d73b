/* qmx_calib.h -- calibration kernels (libqmx_calib.so).
 *
 * Not part of the quantized path: these measure what one GPU reaches for the
 * operations the path is bounded by, so that measured kernel rates can be set
 * against achievable rather than only published peaks.
 *
 * All pointers are device pointers owned by the caller; nothing is allocated,
 * freed or synchronized; every call is asynchronous on `stream` (a
 * hipStream_t, NULL for the default stream).  Each call returns 0, or -1 for
 * a NULL or misaligned pointer, a size that is not a multiple of 16 bytes, a
 * non-positive grid, or a launch the runtime rejects.
 */
#ifndef QMX_CALIB_H
#define QMX_CALIB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` (a multiple of 16) from the 16-byte aligned `src` once, in
 * 16-byte loads over a grid of `blocks` work-groups of 256 threads.  Writes
 * sink[0] only if the xor of all words read equals `never` (pass a value the
 * data cannot give). */
int qmxc_read(const void* src, size_t bytes, uint32_t* sink, uint32_t never, int blocks, void* stream);

/* Copies `bytes` (a multiple of 16) from `src` to `dst` (both 16-byte
 * aligned, not overlapping) in 16-byte loads and stores. */
int qmxc_copy(const void* src, void* dst, size_t bytes, int blocks, void* stream);

/* `blocks` work-groups of 4 waves, each wave issuing `iters` rounds of
 * independent bf16 matrix-core instructions: shape 16 = eight
 * v_mfma_f32_16x16x32_bf16 per round (16384 flops each), shape 32 = four
 * v_mfma_f32_32x32x16_bf16 (32768 flops each), i.e. 131072 flops per wave and
 * round either way; writes blocks*256 floats to `out`. */
int qmxc_mfma(float* out, int iters, int blocks, int shape, void* stream);

/* Co-issue of the matrix core and the vector ALU: `blocks` work-groups of 4
 * waves, each wave issuing `iters` rounds of four independent
 * v_mfma_f32_32x32x16_bf16, each followed by `fmas` independent float32 FMAs
 * (with_mfma != 0), or the same FMAs alone (with_mfma == 0).  fmas is one of
 * 0, 2, 4, 6, 8, 10, 12, 16 (else -1).  Writes blocks*256 floats to `out`. */
int qmxc_mfma_valu(float* out, int iters, int blocks, int fmas, int with_mfma, void* stream);

/* `blocks` work-groups of one wave that do nothing (the launch floor). */
int qmxc_empty(int blocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QMX_CALIB_H */
