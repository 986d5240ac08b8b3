// Row-wise softmax of an fp16 matrix on gfx950: the tutorial's register-resident
// reduction kernel (news article on TileLang kernel design, paragraph on the
// fused epilogue, last sentences: a row softmax from fragment-level max and sum
// reductions that keeps the normalisation in registers; blog post on TileLang,
// "three-piece set" section, item 2: one kernel per row-wise normalisation,
// nothing intermediate in HBM).
//
//   m = max_j x_j,  e_j = exp(x_j - m),  s = sum_j e_j,  y_j = e_j / s
//
// The work is HBM-bound (2 bytes read and 2 written per element), so the design
// is about moving each byte once:
//  * softmax_reg_kernel<TPR, VPT>: TPR threads own one row, 256 / TPR rows per
//    workgroup of 256 threads.  TPR is the smallest power of two from 16 to 256
//    that leaves at most 8 chunks per thread, so short rows do not idle lanes.
//    Each thread holds VPT 16-byte chunks of the row in registers (chunk c of
//    the row goes to thread c % TPR, so a wave's loads cover consecutive runs).
//    The row is read once, reduced twice (max, then sum: butterfly shuffles
//    inside groups of lanes, one LDS exchange when a row spans several waves)
//    and written once.  Rows up to 256 * 8 * 8 = 16384 columns.  Matrices of
//    128 MiB and more are read with non-temporal loads (streamed once, larger
//    than what the Infinity Cache keeps).
//  * softmax_online_kernel: rows longer than the register path holds.  One pass
//    keeps a running (max, sum) per thread, rescaling the sum when the max
//    grows; the pairs are merged across the row; a second pass re-reads the row
//    and writes exp(x - m) / s.  Three row transfers instead of two.
// exp is exp2 of (x - m) * log2(e): x - m is formed first, in fp32, so the
// shift never loses the small differences that matter (an FMA of x * log2 e
// against m * log2 e would lose them for |m| in the thousands).  1/s is an IEEE
// fp32 division, once per row.  Chunks that straddle the end of a row are
// loaded and stored element by element; columns past the end read as -inf.
// IEEE semantics match the plain definition: -inf entries give 0, a row of all
// -inf gives NaN (m = -inf, x - m = NaN), and a +inf or NaN entry makes the
// whole row NaN (v_max_f32 ignores a NaN operand, but its exp is NaN and so is s).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "common.h"
#include "gemm_f16.h"
#include "softmax_f16.h"

using namespace gk;

namespace {

constexpr float kLog2e = 1.44269504088896341f;
constexpr int kThreads = 256;

typedef f16x8 f16x8_u __attribute__((aligned(2)));

// Reduce over the TPR threads of a row.  TPR <= 64: butterfly shuffles inside
// aligned groups of TPR lanes.  TPR = 128 or 256: the row's waves exchange
// their wave results through `red` (one float per wave of the workgroup),
// between two barriers that every wave of the workgroup reaches.
template <int TPR, bool MAX>
__device__ __forceinline__ float row_reduce(float v, float* red) {
#pragma unroll
    for (int off = (TPR < 64 ? TPR : 64) / 2; off >= 1; off >>= 1) {
        const float o = __shfl_xor(v, off, 64);
        v = MAX ? fmaxf(v, o) : v + o;
    }
    if constexpr (TPR <= 64) {
        return v;
    } else {
        constexpr int WPR = TPR / 64;  // waves per row
        const int wave = threadIdx.x >> 6, first = wave - wave % WPR;
        if ((threadIdx.x & 63) == 0) red[wave] = v;
        __syncthreads();
        float r = red[first];
#pragma unroll
        for (int w = 1; w < WPR; ++w) r = MAX ? fmaxf(r, red[first + w]) : r + red[first + w];
        __syncthreads();  // red is reused by the next reduction
        return r;
    }
}

// Chunk of 8 values starting at column `col` of row `x` (length cols); columns
// past the end read as -inf.  NT: non-temporal load, for matrices streamed
// through once that are too large to stay in the caches.
template <bool NT = false>
__device__ __forceinline__ void load8(const f16* x, int64_t col, int64_t cols, float* v) {
    if (col + 8 <= cols) {
        const f16x8 h = NT ? __builtin_nontemporal_load((const f16x8_u*)(x + col)) : *(const f16x8_u*)(x + col);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (float)h[e];
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = col + e < cols ? (float)x[col + e] : -INFINITY;
    }
}
__device__ __forceinline__ void store8(f16* y, int64_t col, int64_t cols, const float* v) {
    if (col + 8 <= cols) {
        f16x8 h;
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = (f16)v[e];
        *(f16x8_u*)(y + col) = h;
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (col + e < cols) y[col + e] = (f16)v[e];
    }
}

template <int TPR, int VPT, bool NT>
__global__ void __launch_bounds__(kThreads) softmax_reg_kernel(const f16* X, f16* Y, int64_t rows,
                                                                int64_t cols) {
    constexpr int RPW = kThreads / TPR;  // rows per workgroup
    __shared__ float red[kThreads / 64];
    const int t = threadIdx.x % TPR;
    const int64_t row = (int64_t)blockIdx.x * RPW + threadIdx.x / TPR;
    // Threads past the last row recompute the last row and store nothing, so
    // every wave reaches the barriers of the reductions.
    const bool active = row < rows;
    const f16* x = X + (active ? row : rows - 1) * cols;
    f16* y = Y + row * cols;

    float v[VPT][8];
#pragma unroll
    for (int i = 0; i < VPT; ++i) load8<NT>(x, ((int64_t)i * TPR + t) * 8, cols, v[i]);
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < VPT; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) m = fmaxf(m, v[i][e]);
    m = row_reduce<TPR, true>(m, red);
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < VPT; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            v[i][e] = __builtin_amdgcn_exp2f((v[i][e] - m) * kLog2e);
            s += v[i][e];
        }
    s = row_reduce<TPR, false>(s, red);
    if (!active) return;
    const float inv = 1.0f / s;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[i][e] *= inv;
        store8(y, ((int64_t)i * TPR + t) * 8, cols, v[i]);
    }
}

// Running (max, sum) pair: sum of exp(x - max) over the values seen so far.
// A pair whose max is -inf has seen only -inf values and contributes nothing.
__device__ __forceinline__ void merge(float& m, float& s, float m2, float s2) {
    const float M = fmaxf(m, m2);
    const float a = m == -INFINITY ? 0.0f : s * __builtin_amdgcn_exp2f((m - M) * kLog2e);
    const float b = m2 == -INFINITY ? 0.0f : s2 * __builtin_amdgcn_exp2f((m2 - M) * kLog2e);
    m = M;
    s = a + b;
}

__global__ void __launch_bounds__(kThreads) softmax_online_kernel(const f16* X, f16* Y, int64_t cols) {
    __shared__ float red_m[4], red_s[4];
    const int64_t row = blockIdx.x;
    const f16* x = X + row * cols;
    f16* y = Y + row * cols;
    float m = -INFINITY, s = 0.0f;
    for (int64_t col = (int64_t)threadIdx.x * 8; col < cols; col += (int64_t)kThreads * 8) {
        float v[8];
        load8(x, col, cols, v);
        float mc = v[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) mc = fmaxf(mc, v[e]);
        if (mc == -INFINITY) continue;  // contributes nothing (all -inf or past the end)
        float sc = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) sc += __builtin_amdgcn_exp2f((v[e] - mc) * kLog2e);
        merge(m, s, mc, sc);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float m2 = __shfl_xor(m, off, 64), s2 = __shfl_xor(s, off, 64);
        merge(m, s, m2, s2);
    }
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        red_m[wave] = m;
        red_s[wave] = s;
    }
    __syncthreads();
    m = red_m[0];
    s = red_s[0];
#pragma unroll
    for (int w = 1; w < 4; ++w) merge(m, s, red_m[w], red_s[w]);
    // all -inf: m = -inf and s = 0, so x - m = NaN below, as the definition gives
    const float inv = 1.0f / s;
    for (int64_t col = (int64_t)threadIdx.x * 8; col < cols; col += (int64_t)kThreads * 8) {
        float v[8];
        load8(x, col, cols, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = __builtin_amdgcn_exp2f((v[e] - m) * kLog2e) * inv;
        store8(y, col, cols, v);
    }
}

template <int TPR, int VPT, bool NT>
hipError_t launch_reg(const f16* X, f16* Y, int64_t rows, int64_t cols, hipStream_t s) {
    constexpr int RPW = kThreads / TPR;
    const int64_t blocks = (rows + RPW - 1) / RPW;
    hipLaunchKernelGGL((softmax_reg_kernel<TPR, VPT, NT>), dim3((unsigned)blocks), dim3(kThreads), 0, s, X, Y, rows,
                       cols);
    return hipGetLastError();
}

template <int TPR, bool NT>
hipError_t launch_reg_vpt(int vpt, const f16* X, f16* Y, int64_t rows, int64_t cols, hipStream_t s) {
    switch (vpt) {
        case 1: return launch_reg<TPR, 1, NT>(X, Y, rows, cols, s);
        case 2: return launch_reg<TPR, 2, NT>(X, Y, rows, cols, s);
        case 3: return launch_reg<TPR, 3, NT>(X, Y, rows, cols, s);
        case 4: return launch_reg<TPR, 4, NT>(X, Y, rows, cols, s);
        case 5: return launch_reg<TPR, 5, NT>(X, Y, rows, cols, s);
        case 6: return launch_reg<TPR, 6, NT>(X, Y, rows, cols, s);
        case 7: return launch_reg<TPR, 7, NT>(X, Y, rows, cols, s);
        default: return launch_reg<TPR, 8, NT>(X, Y, rows, cols, s);
    }
}

template <bool NT>
hipError_t launch_reg_tpr(int tpr, int vpt, const f16* X, f16* Y, int64_t rows, int64_t cols, hipStream_t s) {
    switch (tpr) {
        case 16: return launch_reg_vpt<16, NT>(vpt, X, Y, rows, cols, s);
        case 32: return launch_reg_vpt<32, NT>(vpt, X, Y, rows, cols, s);
        case 64: return launch_reg_vpt<64, NT>(vpt, X, Y, rows, cols, s);
        case 128: return launch_reg_vpt<128, NT>(vpt, X, Y, rows, cols, s);
        default: return launch_reg_vpt<256, NT>(vpt, X, Y, rows, cols, s);
    }
}

// Matrices of at least this many bytes are read with non-temporal loads: they
// are streamed once and are too large for the 256 MB Infinity Cache to keep
// alongside other data.  Smaller ones keep the cached loads, which profit when
// X was just written by the producing kernel.
constexpr int64_t kStreamBytes = (int64_t)128 << 20;

// Threads per row for the register path: the fewest (16 .. 256, powers of
// two) that hold the row's 8-column chunks with at most 8 per thread.
int threads_per_row(int64_t cols) {
    const int64_t chunks = (cols + 7) / 8;
    int tpr = 16;
    while (tpr < kThreads && (int64_t)tpr * 8 < chunks) tpr *= 2;
    return tpr;
}

}  // namespace

extern "C" {

int softmax_rows_f16_path(int64_t rows, int64_t cols) {
    if (rows <= 0 || cols <= 0) return SOFTMAX_PATH_NONE;
    if (cols > (int64_t)SOFTMAX_REG_MAX_COLS) return SOFTMAX_PATH_ONLINE;
    return threads_per_row(cols) <= 64 ? SOFTMAX_PATH_WAVE : SOFTMAX_PATH_WORKGROUP;
}

int softmax_rows_f16(int64_t rows, int64_t cols, const void* X, void* Y, void* stream) {
    if (rows < 0 || cols < 0 || rows > INT32_MAX || cols > INT32_MAX) return GEMM_ERR_INVALID_DIM;
    if (rows == 0 || cols == 0) return GEMM_OK;
    if (!X || !Y) return GEMM_ERR_NULL_POINTER;
    if (((uintptr_t)X | (uintptr_t)Y) % 2 != 0) return GEMM_ERR_MISALIGNED;
    const f16* x = (const f16*)X;
    f16* y = (f16*)Y;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    if (softmax_rows_f16_path(rows, cols) == SOFTMAX_PATH_ONLINE) {
        hipLaunchKernelGGL(softmax_online_kernel, dim3((unsigned)rows), dim3(kThreads), 0, s, x, y, cols);
        e = hipGetLastError();
    } else {
        const int tpr = threads_per_row(cols);
        const int vpt = (int)(((cols + 7) / 8 + tpr - 1) / tpr);
        e = rows * cols * 2 >= kStreamBytes ? launch_reg_tpr<true>(tpr, vpt, x, y, rows, cols, s)
                                            : launch_reg_tpr<false>(tpr, vpt, x, y, rows, cols, s);
    }
    return e == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

}  // extern "C"
