// Shared device-side definitions for the gfx950 fp16 GEMM kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gk {

typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define GK_LDS __attribute__((address_space(3)))
#define GK_GLB __attribute__((address_space(1)))

enum Epilogue { EPI_NONE = 0, EPI_BIAS = 1, EPI_BIAS_GELU = 2 };

struct GemmArgs {
    const f16* A;     // [M][K], row stride lda
    const f16* B;     // [K][N], row stride ldb
    const f16* bias;  // [N] or null
    f16* C;           // [M][N], row stride ldc
    int M, N, K;
    int lda, ldb, ldc;  // leading dimensions in elements (>= K, N, N)
    int tiles_m, tiles_n;
    float* partial;     // split-K: fp32 partial sums [k_split][M][N] (workspace), else null
    int k_split;        // split-K: number of K ranges
    int k_chunk;        // split-K: K rows per range (a multiple of the stage depth)
    uint64_t* timeline; // timeline builds only (GK_TIMELINE): per-wave clock stamps, else null
};

// Timeline builds (compiled with -DGK_TIMELINE=1, never the shipped library): the tile kernel records, per
// wave, the shader clock (s_memtime) and the 100 MHz real-time counter (s_memrealtime) at kernel entry, after
// the prologue's barrier, after the K loop and after its C stores have completed.
#ifndef GK_TIMELINE
#define GK_TIMELINE 0
#endif

// GELU in its erf form on an fp32 value:
//   gelu(x) = x * Phi(x),  Phi(x) = 0.5 * erfc(-x / sqrt 2)
//           = 1 - 0.5 erfc(z)  (x >= 0)   or   0.5 erfc(z)  (x < 0),   z = |x| / sqrt 2.
// erfc(z) for z >= 0 uses the Chebyshev-fitted form published in Numerical
// Recipes (Press, Teukolsky, Vetterling, Flannery, 2nd ed., section 6.2,
// "erfcc"):  erfc(z) = t exp(-z^2 + P(t)),  t = 1 / (1 + z/2),  with P a
// degree-9 polynomial.  Its fractional error is below 1.2e-7 for every
// z >= 0.  In fp32 the error stays below 1e-5 relative, far below the fp16
// output's half-ulp of 2.4e-4.
// The evaluation is branch-free: one reciprocal, one exp2 and ~12 FMAs.  The
// constants are folded so that no multiply is spent on them at run time:
//   0.5 erfc(z) = t * 2^(P(t) log2e - 1 - z^2 log2e),  z^2 log2e = |x| * (|x| * log2e / 2),
// with P's coefficients scaled by log2e (each the double product rounded
// once to fp32) and t = 1 / (1 + |x| / (2 sqrt 2)).  Computing erfc(|z|) and
// reflecting avoids the cancellation of 1 + erf(.) for x << 0.
#define GK_L2E 1.44269504088896341
__device__ __forceinline__ float gelu_erf(float x) {
    const float a = __builtin_fabsf(x);
    const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(a, (float)(0.5 * 0.70710678118654752), 1.0f));
    float q = (float)(0.17087277 * GK_L2E);
    q = __builtin_fmaf(q, t, (float)(-0.82215223 * GK_L2E));
    q = __builtin_fmaf(q, t, (float)(1.48851587 * GK_L2E));
    q = __builtin_fmaf(q, t, (float)(-1.13520398 * GK_L2E));
    q = __builtin_fmaf(q, t, (float)(0.27886807 * GK_L2E));
    q = __builtin_fmaf(q, t, (float)(-0.18628806 * GK_L2E));
    q = __builtin_fmaf(q, t, (float)(0.09678418 * GK_L2E));
    q = __builtin_fmaf(q, t, (float)(0.37409196 * GK_L2E));
    q = __builtin_fmaf(q, t, (float)(1.00002368 * GK_L2E));
    q = __builtin_fmaf(q, t, (float)(-1.26551223 * GK_L2E - 1.0));
    const float e2 = __builtin_fmaf(a, a * (float)(-0.5 * GK_L2E), q);  // <= -1: log2 of erfc(z) / (2 t)
    const float half_erfc = t * __builtin_amdgcn_exp2f(e2);
    const float phi = x >= 0.0f ? 1.0f - half_erfc : half_erfc;
    // The product stays an fp32 multiply of its own (the empty asm hides it from instruction selection).
    // Fused into the fp16 conversion it becomes v_fma_mix with a +0 addend, which turns an exact -0
    // product (x = -0, or x below about -14.4 where Phi underflows) into +0.
    float y = x * phi;
    asm("" : "+v"(y));
    return y;
}
#undef GK_L2E

template <int EPI>
__device__ __forceinline__ float apply_epilogue(float s, float b) {
    if constexpr (EPI == EPI_NONE) {
        return s;
    } else if constexpr (EPI == EPI_BIAS) {
        return s + b;
    } else {
        return gelu_erf(s + b);
    }
}

// Workgroup id -> linear tile id.  The dispatcher deals consecutive workgroup
// ids round-robin over the 8 XCDs; this regroups them so that each XCD (each
// with its own L2) receives one contiguous run of tile ids.  A bijection on
// [0, nwg) for any nwg.
__device__ __forceinline__ int xcd_contiguous_id(int wg, int nwg) {
    const int xcd = wg & 7, slot = wg >> 3;
    const int q = nwg >> 3, r = nwg & 7;
    return (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + slot;
}

// Linear tile id -> (tile_m, tile_n), walking GROUP_M tile-rows column by
// column so neighbouring ids share B column panels and A row panels in L2.
template <int GROUP_M>
__device__ __forceinline__ void grouped_tile(int lid, int tiles_m, int tiles_n, int& tm, int& tn) {
    const int per_group = GROUP_M * tiles_n;
    const int group = lid / per_group;
    const int first_m = group * GROUP_M;
    const int rows = min(tiles_m - first_m, GROUP_M);
    const int in_g = lid - group * per_group;
    tm = first_m + in_g % rows;
    tn = in_g / rows;
}

__device__ __forceinline__ f16x4 lds_read_tr16_b64(const GK_LDS char* p) {
    s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((GK_LDS s16x4*)p);
    return __builtin_bit_cast(f16x4, v);
}

// ---- asynchronous HBM/L2 -> LDS copies (LDS-DMA) ----
// Issued through inline assembly on purpose: when the compiler sees an
// LDS-DMA builtin it must assume any later LDS read may alias the copy and
// places "s_waitcnt vmcnt(0)" before it, which serialises the prefetch of
// stage s+1 behind the compute of stage s.  Here the kernels order the copies
// themselves (wait_vmcnt<> + barrier before a stage is read).  The LDS
// destination of lane l is m0 + size*l; the destination is an "{m0}" operand,
// so the compiler itself writes m0 before each copy (often computing the
// address straight into it) and knows what m0 holds afterwards.  The s_nop
// covers the one wait state that gfx9 parts need between an SALU write of m0
// and an LDS-DMA that reads it.
__device__ __forceinline__ uint32_t lds_addr(const GK_LDS void* p) { return (uint32_t)(uintptr_t)p; }

// 16 bytes per lane from sbase + voff (global, 64-bit scalar base + 32-bit lane offset).
__device__ __forceinline__ void dma_global_16(const void* sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds)
                 : "memory");
}
// Through a buffer resource: each dword that is not wholly below num_records
// reads as 0.  16 bytes per lane.
__device__ __forceinline__ void dma_buffer_16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t lds) {
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(r), "{m0}"(lds)
                 : "memory");
}
// 16 bytes per lane, marked non-temporal: for data streamed exactly once (the
// skinny path's B), so it does not displace reused lines in the caches.
__device__ __forceinline__ void dma_buffer_16_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t lds) {
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds" ::"v"(voff), "s"(r), "{m0}"(lds)
                 : "memory");
}
// 4 bytes per lane.
__device__ __forceinline__ void dma_buffer_4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t lds) {
    asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(r), "{m0}"(lds)
                 : "memory");
}

__device__ __forceinline__ void wait_vmcnt0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Wait until at most CNT vector-memory operations of this wave are outstanding.
template <int CNT>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(CNT >= 0 && CNT <= 63, "vmcnt field");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(CNT) : "memory");
}

}  // namespace gk
