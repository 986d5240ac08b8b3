/*
 * gemm_f16.h -- C ABI of the MI355X (gfx950) half-precision GEMM library.
 *
 * The operation is the tiled half-precision matrix multiply of the TileLang
 * GEMM tutorial (blog post "Designing High-Performance GPU Kernels with
 * TileLang", section "Step 4": fp16 tiles of A [block_M x block_K] and
 * B [block_K x block_N], i.e. B held K x N, multiplied into a float32
 * accumulator fragment), extended as in the tutorial's fused-epilogue
 * chapter (TileLang news article, paragraph on fusing the bias add and the
 * GELU activation into the register-resident accumulator before the output
 * tensor is written):
 *
 *     C[i][j] = fp16( epi( sum_k A[i][k] * B[k][j] ) ),   0 <= i < M, 0 <= j < N
 *     epi(s)  = s                                  GEMM_EPI_NONE
 *             = s + bias[j]                        GEMM_EPI_BIAS
 *             = gelu(s + bias[j])                  GEMM_EPI_BIAS_GELU
 *     gelu(x) = 0.5 * x * (1 + erf(x / sqrt(2)))   (exact erf form)
 *
 * The sum is accumulated in fp32 (products of fp16 values are exact in
 * fp32); bias add and GELU run in fp32 on the accumulator; C is rounded to
 * fp16 once, round-to-nearest-even, and written once.
 *
 * Layout: every matrix is dense row-major with no padding:
 *   A: fp16 [M][K] (leading dimension K), B: fp16 [K][N] (leading dimension N),
 *   C: fp16 [M][N] (leading dimension N), bias: fp16 [N].
 * fp16 means IEEE binary16, passed as raw 16-bit storage.
 *
 * Pointers: A, B, bias and C are DEVICE pointers (memory the caller allocated
 * on the current HIP device).  Any 2-byte-aligned pointer is accepted;
 * 16-byte alignment of A, B and C together with K % 8 == 0 and N % 8 == 0
 * enables the fastest paths.  Other shapes with K % 8 == 0 load through
 * range-checked buffer copies, and the rest through registers with
 * element-wise edges.  Misalignment is never an error.
 *
 * Reads: the library reads only A, B and bias, with one exception.  With odd N
 * it may read the 2 bytes that follow B's last element, and then only when they
 * lie in the same 4 KiB page as that element, so the read cannot fault.  Those
 * bytes reach only output columns past N, which are never written.
 *
 * Ownership: the caller owns every buffer.  The library never allocates,
 * frees or retains caller memory.  C must not overlap A, B or bias.
 *
 * Streams: `stream` is a hipStream_t (NULL = the default stream).  Calls are
 * asynchronous, like a kernel launch: C is complete once the stream has been
 * synchronised.  No call synchronises the device.
 *
 * Errors: arguments are validated before any HIP call; on a validation error
 * nothing is launched and C is left untouched.  Status codes are listed below;
 * gemm_f16_status_string() names them.  GEMM_ERR_LAUNCH carries no detail
 * beyond the fact that hipGetLastError() reported a failure after the launch.
 *
 * Degenerate sizes: M == 0 or N == 0 is a successful no-op (pointers may be
 * NULL).  K == 0 writes C = epi(0), i.e. zeros, bias, or gelu(bias).
 *
 * Thread safety: the library holds no mutable state; calls from several host
 * threads on different streams are safe.
 */
#ifndef GEMM_F16_H
#define GEMM_F16_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GEMM_EPI_NONE = 0,
    GEMM_EPI_BIAS = 1,
    GEMM_EPI_BIAS_GELU = 2
} gemm_epilogue_t;

typedef enum {
    GEMM_OK = 0,
    GEMM_ERR_INVALID_DIM = 1,   /* M, N or K negative, or above 2^31 - 1     */
    GEMM_ERR_NULL_POINTER = 2,  /* A/B/C NULL with M*N > 0 (A/B only if K > 0),
                                   or bias NULL with a bias epilogue          */
    GEMM_ERR_BAD_EPILOGUE = 3,  /* epilogue not one of gemm_epilogue_t        */
    GEMM_ERR_LAUNCH = 4,        /* the HIP runtime reported a launch failure  */
    GEMM_ERR_NO_CONFIG = 5,     /* config index out of range                  */
    GEMM_ERR_UNSUPPORTED = 6,   /* the forced config cannot run this call
                                   (alignment / divisibility it requires)     */
    GEMM_ERR_MISALIGNED = 7     /* a pointer is not 2-byte aligned            */
} gemm_status_t;

/*
 * C = epi(A.B) as described above, on `stream`.  The library picks the kernel
 * configuration from the call's shape class (skinny M, tiled aligned, tiled
 * general).  Returns a gemm_status_t.
 */
int gemm_f16(int64_t M, int64_t N, int64_t K,
             const void* A, const void* B, const void* bias, void* C,
             int epilogue, void* stream);

/*
 * The same product on row-major matrices with leading dimensions (row strides,
 * in elements): A[i][k] at A + i*lda + k, B[k][j] at B + k*ldb + j, C[i][j] at
 * C + i*ldc + j, so A, B and C may be sub-matrices of larger row-major arrays
 * (e.g. a column slice).  Requires lda >= K and ldb >= N when K > 0, and
 * ldc >= N; otherwise GEMM_ERR_INVALID_DIM (also for strides above 2^31 - 1).
 * Elements between the end of a row and the next row start are never written;
 * the padding of A and B may be read, but only inside the arrays' extent
 * (plus, with odd N, the 2 bytes after B's last element, under the rule given
 * for gemm_f16).  The fast paths additionally want lda, ldb and ldc to be
 * multiples of 8.  gemm_f16() is gemm_f16_ex() with lda = K, ldb = ldc = N.
 */
int gemm_f16_ex(int64_t M, int64_t N, int64_t K,
                const void* A, int64_t lda, const void* B, int64_t ldb,
                const void* bias, void* C, int64_t ldc,
                int epilogue, void* stream);

/*
 * C = epi(A . Bt^T) with B given transposed: Bt is fp16 [N][K] row-major with
 * row stride ldb >= K (the layout of a linear layer's weight, out-features x
 * in-features), so C[i][j] = epi(sum_k A[i][k] * Bt[j][k]).  Everything else
 * (lda, ldc, epilogue, errors, streams) is as in gemm_f16_ex; ldb < K with
 * K > 0 is GEMM_ERR_INVALID_DIM.  No bytes past Bt's last element are read.
 */
int gemm_f16_bt(int64_t M, int64_t N, int64_t K,
                const void* A, int64_t lda, const void* Bt, int64_t ldb,
                const void* bias, void* C, int64_t ldc,
                int epilogue, void* stream);

/* Static, NUL-terminated name of a status code ("GEMM_OK", ...).  The two
 * names are the same function. */
const char* gemm_f16_status_string(int status);
const char* gemm_status_string(int status);

/*
 * Latency of the product, the way the tutorial's timing utility measures a
 * kernel: the median over repeated launches, each bracketed by events on the
 * stream (TileLang blog post "Designing High-Performance GPU Kernels with
 * TileLang", section "Step 2").
 *
 * Runs gemm_f16's product (same arguments and layout) once untimed, then
 * `iters` times back to back on `stream`, with an event recorded before the
 * first launch and after each one; *median_ms receives the median of the
 * `iters` per-launch times in milliseconds (the mean of the middle two for an
 * even count).  idx = -1 launches the configuration gemm_f16 would pick; idx
 * >= 0 forces configuration idx (GEMM_ERR_NO_CONFIG if out of range,
 * GEMM_ERR_UNSUPPORTED if it cannot run the call).  C is written iters + 1
 * times with the same result.
 *
 * Unlike every other entry point this call is synchronous: it returns after
 * the last launch has finished.  All arguments are validated before any HIP
 * call: besides gemm_f16's checks, median_ms NULL is GEMM_ERR_NULL_POINTER and
 * iters outside [1, GEMM_TIME_MAX_ITERS] is GEMM_ERR_INVALID_DIM.  M == 0 or
 * N == 0 launches nothing and reports 0.  A failure of an event call is
 * GEMM_ERR_LAUNCH.  The events are created and destroyed inside the call.
 */
#define GEMM_TIME_MAX_ITERS 100000
int gemm_f16_time(int idx, int64_t M, int64_t N, int64_t K,
                  const void* A, const void* B, const void* bias, void* C,
                  int epilogue, void* stream, int iters, float* median_ms);

/*
 * Kernel configurations compiled into the library (the offline sweep space;
 * the tutorial's autotuner picks among tile sizes, K-block, pipeline depth
 * and thread count under a shared-memory budget, TileLang news article,
 * paragraph on autotuning).
 */
int gemm_f16_num_configs(void);

/* JSON description of config `idx` written into buf (NUL-terminated, truncated
 * to buflen).  Returns the full length, or -GEMM_ERR_NO_CONFIG.  Keys: idx,
 * name, kind ("tile" | "skinny"), bm, bn, bk, waves_m, waves_n, loader,
 * group_m, stages, bslot, dstride, cslot, waves_per_simd, mfma (32 or 16),
 * spread (schedule flags of the tile kernel: 1 LDS reads spread over the
 * k-step, 2 A fragments refilled in place, 4 MFMAs on accumulators pinned to
 * AGPRs, 8 copies issued right after the stage barrier, 16 the next k-step's
 * B reads front-loaded, 32 C staged through LDS and written with
 * row-contiguous 16-byte stores, 64 those stores non-temporal, 128 A given a
 * third LDS buffer so its copies run a stage ahead of B's, 256 the ping-pong
 * schedule, whose two wave groups alternate between MFMAs and loads over a
 * ring of four 32-deep k-slices; of the skinny
 * kernel: 1 A copied with 16-byte LDS-DMA), b_transposed, k_rotate (skinny:
 * K order rotated per workgroup), lds_bytes, threads. */
int gemm_f16_config_info(int idx, char* buf, int buflen);

/* Index of the configuration gemm_f16() would launch for these arguments
 * (no launch; -1 for a no-op call); negative gemm_status_t on bad arguments. */
int gemm_f16_select_config(int64_t M, int64_t N, int64_t K,
                           const void* A, const void* B, const void* bias, void* C,
                           int epilogue);

/* Same as gemm_f16 but with a forced configuration (used by the sweep and the
 * tests).  GEMM_ERR_UNSUPPORTED if that config cannot handle the call. */
int gemm_f16_with_config(int idx, int64_t M, int64_t N, int64_t K,
                         const void* A, const void* B, const void* bias, void* C,
                         int epilogue, void* stream);

/* The strided forms of the two calls above (leading dimensions as in gemm_f16_ex). */
int gemm_f16_select_config_ex(int64_t M, int64_t N, int64_t K,
                              const void* A, int64_t lda, const void* B, int64_t ldb,
                              const void* bias, void* C, int64_t ldc, int epilogue);
int gemm_f16_with_config_ex(int idx, int64_t M, int64_t N, int64_t K,
                            const void* A, int64_t lda, const void* B, int64_t ldb,
                            const void* bias, void* C, int64_t ldc,
                            int epilogue, void* stream);

/* The same two calls for a transposed B (as in gemm_f16_bt). */
int gemm_f16_bt_select_config(int64_t M, int64_t N, int64_t K,
                              const void* A, int64_t lda, const void* Bt, int64_t ldb,
                              const void* bias, void* C, int64_t ldc, int epilogue);
int gemm_f16_bt_with_config(int idx, int64_t M, int64_t N, int64_t K,
                            const void* A, int64_t lda, const void* Bt, int64_t ldb,
                            const void* bias, void* C, int64_t ldc,
                            int epilogue, void* stream);

/*
 * Element-wise fp32 vector add C[i] = A[i] + B[i], 0 <= i < n (the tutorial's
 * first kernel: TileLang blog post, section "Step 3"; news article, paragraph
 * on the vector-add kernel).  Device pointers, asynchronous on `stream`.  It is
 * HBM-bound and doubles as the bandwidth calibration kernel.  Returns a
 * gemm_status_t (GEMM_ERR_INVALID_DIM for n < 0).
 */
int vector_add_f32(int64_t n, const float* A, const float* B, float* C, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_F16_H */
