/*
 * softmax_f16.h -- C ABI of the row-wise softmax in the MI355X (gfx950) library
 * libgemm_f16.so (status codes: gemm_status_t in gemm_f16.h).
 *
 * The operation is the tutorial's register-resident row reduction (TileLang
 * news article, paragraph on the fused epilogue, closing sentences: a row-wise
 * softmax built from fragment-level max and sum reductions that keeps the
 * normalisation in registers; TileLang blog post, "three-piece set" section,
 * item 2: the row-wise normalisation as one kernel with no intermediate in
 * HBM).  The pages give no formula; the standard max-shifted one is used:
 *
 *     m_i = max_j X[i][j]
 *     Y[i][j] = fp16( exp(X[i][j] - m_i) / sum_k exp(X[i][k] - m_i) )
 *
 * computed in fp32 and rounded to fp16 (round-to-nearest-even) once.  IEEE
 * cases: -inf entries give 0; a row of all -inf gives NaN; a row holding +inf
 * or NaN gives NaN everywhere.
 *
 * Layout: X and Y are dense row-major fp16 [rows][cols] (leading dimension
 * cols), DEVICE pointers, any 2-byte alignment.  Y may be X itself (in place);
 * any other overlap is undefined.
 *
 * Ownership and streams: the caller owns both buffers; the call allocates
 * nothing, is asynchronous on `stream` (a hipStream_t, NULL = default stream)
 * and does not synchronise.
 *
 * Errors: GEMM_ERR_INVALID_DIM (rows or cols negative or above 2^31 - 1),
 * GEMM_ERR_NULL_POINTER (X or Y NULL with rows * cols > 0),
 * GEMM_ERR_MISALIGNED (odd address), GEMM_ERR_LAUNCH.  Nothing is launched on
 * a validation error.  rows == 0 or cols == 0 is a successful no-op.
 */
#ifndef SOFTMAX_F16_H
#define SOFTMAX_F16_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Rows up to this many columns are held in registers (one HBM read); longer
 * rows take the two-pass online path (two reads). */
#define SOFTMAX_REG_MAX_COLS 16384

typedef enum {
    SOFTMAX_PATH_NONE = 0,       /* empty call                                   */
    SOFTMAX_PATH_WAVE = 1,       /* cols <= 4096: row in registers of 16..64 threads (one wave or less) */
    SOFTMAX_PATH_WORKGROUP = 2,  /* cols <= SOFTMAX_REG_MAX_COLS: row in registers of 128 or 256 threads */
    SOFTMAX_PATH_ONLINE = 3      /* longer rows: running (max, sum), then a second pass */
} softmax_path_t;

/* Y = softmax over each row of X, on `stream`.  Returns a gemm_status_t. */
int softmax_rows_f16(int64_t rows, int64_t cols, const void* X, void* Y, void* stream);

/* The softmax_path_t softmax_rows_f16 takes for this shape (no launch). */
int softmax_rows_f16_path(int64_t rows, int64_t cols);

#ifdef __cplusplus
}
#endif

#endif /* SOFTMAX_F16_H */
