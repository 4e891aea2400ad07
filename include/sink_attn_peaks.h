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

/* Co-issue of matrix and vector work: `grid` workgroups of 8 wavefronts (two
 * per SIMD, one workgroup per CU), each wavefront running `iters` iterations
 * of 16 v_mfma_f32_32x32x16_bf16 in four chains and/or 32 independent FMAs.
 * mode 0: MFMAs only; 1: FMAs only; 2: both in every wavefront, two FMAs
 * after each MFMA; 3: wavefronts 0-3 the MFMAs, wavefronts 4-7 (sharing
 * their SIMDs) the FMAs.  out is float32 [grid * 512]; cycles receives each
 * wavefront's s_memtime span (int64 [grid * 8]).  Cycles per iteration =
 * cycles / iters. */
int sink_attn_peaks_coissue(int32_t mode, int32_t iters, float* out, long long* cycles, int32_t grid,
                            void* stream);

/* LDS read rate: `grid` workgroups of 8 wavefronts, each lane issuing 16
 * reads per iteration at conflict-free addresses.  mode 0: ds_read_b128
 * (16 bytes per lane); 1: ds_read_b64; 2: ds_read_b64_tr_b16 (8 bytes).
 * out is uint32 [grid * 512]; cycles as for the co-issue probe.  Bytes per
 * clock per CU = 512 * iters * 16 * bytes per lane / slowest wavefront's
 * cycles. */
int sink_attn_peaks_lds(int32_t mode, int32_t iters, uint32_t* out, long long* cycles, int32_t grid,
                        void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SINK_ATTN_PEAKS_H */
