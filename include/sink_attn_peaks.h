/*
 * sink_attn_peaks.h - microbenchmarks of the GPU itself (libsinkattn_peaks.so),
 * measured beside the nominal MI355X peaks the kernels' rooflines use.  They
 * are not part of the attention path.
 *
 * Every call enqueues one kernel on `stream` (a hipStream_t) and returns 0, 1
 * for an invalid argument (nothing launched) or 4 when the launch failed.
 * Buffers are device memory owned by the caller.  The caller times the call
 * (HIP events) and derives the rate.
 */
#ifndef SINK_ATTN_PEAKS_H
#define SINK_ATTN_PEAKS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming read: reads `bytes` (a multiple of 16) of src once, 16 bytes per
 * lane access, with `grid` workgroups of 256 lanes; out receives one word per
 * workgroup (uint32 [grid]).  Rate = bytes / time. */
int sink_attn_peaks_read(const void* src, size_t bytes, uint32_t* out, int32_t grid, void* stream);

/* Dense bf16 matrix-core rate: `grid` workgroups of 4 wavefronts, each
 * wavefront issuing 4 * iters v_mfma_f32_32x32x16_bf16 in four independent
 * chains (32768 FLOP each); out is float32 [grid * 256].
 * Rate = grid * 4 * 4 * iters * 32768 / time. */
int sink_attn_peaks_mfma(int32_t iters, float* out, int32_t grid, void* stream);

/* v_exp_f32 rate: `grid` workgroups of 256 lanes, each lane evaluating
 * 8 * iters dependent-in-chain exp2 (eight independent chains, one fma
 * each); out is float32 [grid * 256].  Rate = grid * 256 * 8 * iters / time. */
int sink_attn_peaks_exp(int32_t iters, float* out, int32_t grid, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SINK_ATTN_PEAKS_H */
