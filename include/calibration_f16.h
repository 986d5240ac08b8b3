/*
 * calibration_f16.h -- C ABI of the MFMA throughput calibration kernel of the
 * MI355X (gfx950) fp16 GEMM library.
 *
 * The tutorial reports its GEMM's Tensor-Core throughput and profiles its
 * kernels (TileLang news article, paragraphs on autotuning and on debugging
 * and profiling); its first kernel, the vector add, doubles here as the HBM
 * calibration (vector_add_f32 in gemm_f16.h).  This is the same idea for the
 * matrix cores: a kernel whose waves do nothing but fp16 MFMAs on registers,
 * so the rate it sustains on all compute units is the practical MFMA ceiling
 * of the part under its board power limit, which the spec figure (which
 * assumes the peak engine clock) is not.
 *
 * mfma_f16_calibration(shape, iters, workgroups, stamps, sink, stream)
 *   shape       16: v_mfma_f32_16x16x32_f16, 32: v_mfma_f32_32x32x16_f16
 *               (GEMM_ERR_UNSUPPORTED otherwise)
 *   iters       loop trips per wave (>= 1); each trip issues 8 independent
 *               MFMAs per wave
 *   workgroups  number of workgroups of 8 waves (two per SIMD), 1 .. 65536
 *   stamps      device pointer, uint64 [workgroups][4], written by wave 0 of
 *               each workgroup: shader-clock counter (s_memtime) before and
 *               after the loop, then the 100 MHz real-time counter
 *               (s_memrealtime) before and after; their ratio gives the
 *               clock the loop ran at
 *   sink        device pointer, float [workgroups * 512]: one sum of the
 *               accumulators per thread, so the loop cannot be elided
 *   stream      hipStream_t (NULL = default); asynchronous like a launch
 * Returns a gemm_status_t: GEMM_ERR_INVALID_DIM for iters or workgroups out
 * of range, GEMM_ERR_NULL_POINTER / GEMM_ERR_MISALIGNED for the buffers
 * (8- and 4-byte alignment), all checked before any HIP call.  The caller
 * owns both buffers.
 *
 * mfma_f16_calibration_flops(shape, iters, workgroups) returns the FLOPs one
 * such launch performs (2*M*N*K per MFMA).
 */
#ifndef CALIBRATION_F16_H
#define CALIBRATION_F16_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int mfma_f16_calibration(int shape, int64_t iters, int64_t workgroups, uint64_t* stamps, float* sink,
                         void* stream);
int64_t mfma_f16_calibration_flops(int shape, int64_t iters, int64_t workgroups);

#ifdef __cplusplus
}
#endif

#endif /* CALIBRATION_F16_H */
