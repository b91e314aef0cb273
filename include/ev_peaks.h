/*
 * ev_peaks.h — calibration kernels that measure what one MI355X actually sustains, so that
 * rooflines can be stated against the box as well as against the published peaks.
 * Not part of the verification pass.  Pointers are DEVICE memory owned by the caller;
 * calls enqueue on `stream` and return without synchronising; the caller times them.
 */
#ifndef EV_PEAKS_H
#define EV_PEAKS_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "ev.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Dense bf16 matrix-core loop: n_workgroups workgroups of 256 threads (one wavefront per
 * SIMD), each wavefront running `iters` rounds of four independent
 * v_mfma_f32_32x32x16_bf16 products on register operands (32768 flops each), so the work
 * is n_workgroups * 4 * iters * 4 * 32768 flops.  sink[n_workgroups] float receives one
 * value per workgroup so that nothing is optimised away.  EV_ERR_SHAPE unless
 * n_workgroups >= 1 and iters >= 1; EV_ERR_NULL if sink is NULL. */
ev_status ev_peak_mfma_bf16(int32_t n_workgroups, int32_t iters, float *sink, hipStream_t stream);

/* Device-to-device copy of `bytes` bytes in 16-byte pieces with a grid-stride loop
 * (bytes moved = 2 * bytes: one read, one write).  src and dst must be 16-byte aligned and
 * bytes a multiple of 16 (EV_ERR_ARG otherwise); EV_ERR_NULL on a NULL pointer. */
ev_status ev_peak_copy(const void *src, void *dst, size_t bytes, hipStream_t stream);

/* Read of `bytes` bytes in 16-byte pieces by n_workgroups workgroups of 256 threads
 * (grid-stride); sink[n_workgroups] uint32 receives one XOR of the data per workgroup.
 * src 16-byte aligned and bytes a multiple of 16 (EV_ERR_ARG otherwise); EV_ERR_NULL on a
 * NULL pointer; EV_ERR_SHAPE unless n_workgroups >= 1. */
ev_status ev_peak_read(const void *src, size_t bytes, uint32_t *sink, int32_t n_workgroups,
                       hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* EV_PEAKS_H */
