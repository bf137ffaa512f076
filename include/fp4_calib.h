/*
 * fp4_calib.h -- measurement helpers of libfp4.so (not part of the FP4
 * computation): kernels whose only purpose is to measure, on the GPU at
 * hand, the achievable rate of the two resources the library's kernels are
 * priced against, so that roofline fractions can be given against measured
 * as well as published peaks.  Device pointers; work is enqueued on `stream`
 * (a hipStream_t, or NULL for the default stream).  Return 0, -1 on bad
 * arguments, -4 on a launch error.
 */
#ifndef FP4_CALIB_H
#define FP4_CALIB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* `workgroups` workgroups of 256 threads each run `iters` rounds of four
 * independent v_mfma_f32_32x32x16_f16 chains per wave: 4 * iters * 32768 flops
 * per wave, 4 waves per workgroup.  sink: workgroups * 256 floats (written). */
int fp4_calib_mfma_f16(int64_t iters, int32_t workgroups, float* sink, void* stream);

/* Reads `bytes` (a multiple of 16, buf 16-byte aligned) once with 16-byte loads
 * over `workgroups` workgroups of 256 threads.  sink: workgroups * 256 words. */
int fp4_calib_read(const void* buf, size_t bytes, int32_t workgroups, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP4_CALIB_H */
