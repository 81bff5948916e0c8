/*
 * dsa3d_peaks.h -- measured-peak microbenchmarks shipped in libdsa3d.so, used by the
 * benchmark to report roofline fractions against what this GPU sustains beside the
 * published peaks.  Not part of the attention computation.  Every call enqueues one
 * kernel on `stream` and returns at once; the caller times it with events on that
 * stream.  All pointers are device pointers owned by the caller.
 */
#ifndef DSA3D_PEAKS_H
#define DSA3D_PEAKS_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* All-CU bf16 matrix-core loop (v_mfma_f32_16x16x32_bf16, eight independent
   accumulators per wave): `blocks` workgroups of 4 waves, `iters` iterations.
   out: blocks * 256 floats (written, to keep the results live).  Returns the flops
   the launch executes, or -1 on a bad argument or launch failure. */
double dsa3d_peak_mfma_bf16(float* out, int blocks, int iters, hipStream_t stream);

/* The same with v_mfma_f32_32x32x16_bf16 (four chains of 16 accumulators per wave). */
double dsa3d_peak_mfma32_bf16(float* out, int blocks, int iters, hipStream_t stream);

/* Streaming read of `bytes` (a multiple of 16, 16-byte aligned) with 16-byte loads by
   `blocks` workgroups of 256 threads; out: blocks * 256 words.  0 or -1. */
int dsa3d_peak_read(const void* src, size_t bytes, uint32_t* out, int blocks, hipStream_t stream);

/* Streaming copy of `bytes` (multiple of 16, 16-byte aligned buffers).  0 or -1. */
int dsa3d_peak_copy(const void* src, void* dst, size_t bytes, int blocks, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA3D_PEAKS_H */
