// MFMA throughput calibration for gfx950: the matrix-core counterpart of the
// vector-add HBM calibration.  Every wave runs a register-only loop of
// independent fp16 MFMA chains, with no memory traffic at all, so the rate it
// sustains is what the chip's matrix cores deliver under the board's power
// limit with nothing else drawing power.  It is the practical ceiling that a
// GEMM's MFMA fraction is set against; the published dense fp16 figure
// assumes the peak engine clock.
//
// Declared in include/calibration_f16.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "calibration_f16.h"
#include "gemm_f16.h"

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWaves = 8;    // two waves per SIMD
constexpr int kChains = 8;   // independent accumulators per wave: more than the MFMA's dependency latency

// Operand values: fixed, data-dependent fp16 values in (-1, 1) (a multiplicative hash of the lane and
// register index), so the multipliers toggle as they do on GEMM data rather than on zeros.
__device__ __forceinline__ f16x8 operand(int lane, int salt) {
    f16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t h = (uint32_t)(lane * 8 + e + 1) * 2654435761u ^ (uint32_t)salt * 40503u;
        v[e] = (_Float16)((float)(h >> 8) * (1.0f / 8388608.0f) - 1.0f);
    }
    return v;
}

template <int SHAPE>
__global__ void __launch_bounds__(kWaves * 64) mfma_f16_loop_kernel(int64_t iters, uint64_t* stamps, float* sink) {
    const int lane = threadIdx.x & 63;
    const f16x8 a = operand(lane, 1), b = operand(lane, 2);
    typedef typename std::conditional<SHAPE == 16, f32x4, f32x16>::type acc_t;
    acc_t acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = acc_t{};
    __syncthreads();
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kChains; ++c) {
            if constexpr (SHAPE == 16) {
                acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[c], 0, 0, 0);
            } else {
                acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[c], 0, 0, 0);
            }
        }
    }
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int r = 0; r < (SHAPE == 16 ? 4 : 16); ++r) s += acc[c][r];
    sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
    if (threadIdx.x == 0) {
        uint64_t* o = stamps + 4 * (size_t)blockIdx.x;
        o[0] = t0;
        o[1] = t1;
        o[2] = r0;
        o[3] = r1;
    }
}

}  // namespace

extern "C" {

int mfma_f16_calibration(int shape, int64_t iters, int64_t workgroups, uint64_t* stamps, float* sink, void* stream) {
    if (shape != 16 && shape != 32) return GEMM_ERR_UNSUPPORTED;
    if (iters < 1 || workgroups < 1 || workgroups > 65536) return GEMM_ERR_INVALID_DIM;
    if (!stamps || !sink) return GEMM_ERR_NULL_POINTER;
    if (((uintptr_t)stamps & 7) || ((uintptr_t)sink & 3)) return GEMM_ERR_MISALIGNED;
    const dim3 grid((unsigned)workgroups), block(kWaves * 64);
    if (shape == 16)
        hipLaunchKernelGGL(mfma_f16_loop_kernel<16>, grid, block, 0, (hipStream_t)stream, iters, stamps, sink);
    else
        hipLaunchKernelGGL(mfma_f16_loop_kernel<32>, grid, block, 0, (hipStream_t)stream, iters, stamps, sink);
    return hipGetLastError() == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

int64_t mfma_f16_calibration_flops(int shape, int64_t iters, int64_t workgroups) {
    const int64_t per_mfma = shape == 16 ? 2LL * 16 * 16 * 32 : 2LL * 32 * 32 * 16;
    return per_mfma * kChains * kWaves * iters * workgroups;
}

}  // extern "C"
