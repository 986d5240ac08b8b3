/*
 * Plain fp64 CPU oracle for the half-precision GEMM with an optional fused
 * bias / bias+GELU epilogue.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the independent checker of the GPU
 * library: only the test-suite, the smoke entry point and the benchmark's CPU
 * baseline may build, load or call it.  It shares no code, header, table or
 * helper with the GPU path.
 *
 * What it computes (the plain definition, written out):
 *   S[i][j] = sum_{k=0}^{K-1} A[i][k] * B[k][j]        fp64, increasing k
 *   X[i][j] = S[i][j] + bias[j]                        (bias epilogues)
 *   Y[i][j] = X  or  0.5 * X * (1 + erf(X / sqrt 2))   (GELU, exact erf form)
 *   C[i][j] = fp16_round_nearest_even(Y[i][j])         one rounding, at the end
 *
 * Sources, from the TileLang GEMM tutorial pages:
 *  - the tiled GEMM takes fp16 A[M,K] and B[K,N] (B held K x N, i.e. row-major
 *    [K,N]) and accumulates in a float32 fragment: blog post "Designing
 *    High-Performance GPU Kernels with TileLang", section "Step 4"; the news
 *    article on TileLang kernel design, paragraph on the tiled GEMM.  The
 *    oracle accumulates in fp64, which contains the fp32 result to within
 *    the fp32 rounding the GPU adds.
 *  - bias add and GELU are applied to the accumulator before the one write of
 *    the output: news article, paragraph on the fused epilogue.  GELU is read
 *    as the exact erf form, applied after the bias add, with bias indexed by
 *    output column and broadcast over rows.
 *  - the output is half precision; rounding is IEEE round-to-nearest-even,
 *    with overflow to infinity (the pages are silent; IEEE default).
 *
 * The fp16 codec is written from the IEEE 754 binary16 definition: 1 sign
 * bit, 5 exponent bits with bias 15, 10 fraction bits; exponent field 0 is
 * zero/subnormal (fraction * 2^-24); 31 is infinity (fraction 0) or NaN.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC gemm_oracle.c -o liboracle.so -lm
 * (no -ffast-math: the arithmetic must stay IEEE fp64.)
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_EPI_NONE = 0, ORACLE_EPI_BIAS = 1, ORACLE_EPI_BIAS_GELU = 2 };

/* ---- binary16 -> double, exact ---------------------------------------- */
double oracle_f16_decode(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24);                 /* zero or subnormal */
    } else if (e == 31) {
        v = (f == 0) ? INFINITY : NAN;
    } else {
        v = ldexp((double)(1024 + f), e - 25);     /* (1 + f/1024) * 2^(e-15) */
    }
    return sign ? -v : v;
}

/* ---- double -> binary16, round to nearest, ties to even ---------------- */
uint16_t oracle_f16_encode(double x) {
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x)) return (uint16_t)(sign | 0x7e00);
    double a = fabs(x);
    if (isinf(a)) return (uint16_t)(sign | 0x7c00);
    if (a == 0.0) return sign;
    /* a = m * 2^e with m in [0.5, 1)  =>  floor(log2 a) = e - 1 */
    int e;
    (void)frexp(a, &e);
    int E = e - 1;
    if (E < -14) E = -14;                          /* subnormal range: fixed quantum */
    /* quantum of the binary16 grid at this exponent: 2^(E-10) */
    double n = ldexp(a, 10 - E);                   /* exact: scaling by a power of two */
    double fl = floor(n);
    double rem = n - fl;                           /* exact */
    double q;
    if (rem > 0.5) q = fl + 1.0;
    else if (rem < 0.5) q = fl;
    else q = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;   /* tie: to even */
    /* value = q * 2^(E-10); q in [0, 2048] */
    uint32_t bits;
    if (q < 1024.0) {
        /* only reachable at E == -14: subnormal (or zero) */
        bits = (uint32_t)q;
    } else {
        /* normal; q == 2048 carries into the next binade through the add */
        bits = ((uint32_t)(E + 15) << 10) + ((uint32_t)q - 1024u);
    }
    if (bits >= 0x7c00u) return (uint16_t)(sign | 0x7c00);   /* overflow -> inf */
    return (uint16_t)(sign | bits);
}

/* ---- GELU, exact erf form, fp64 ---------------------------------------- */
double oracle_gelu(double x) {
    return 0.5 * x * (1.0 + erf(x / sqrt(2.0)));
}

static double apply_epilogue(double s, int epilogue, const uint16_t* bias, int64_t j) {
    if (epilogue == ORACLE_EPI_NONE) return s;
    double x = s + oracle_f16_decode(bias[j]);
    if (epilogue == ORACLE_EPI_BIAS) return x;
    return oracle_gelu(x);
}

/*
 * Full product.  A: M*K fp16 bits, row-major; B: K*N, row-major; bias: N
 * (ignored for epilogue 0); C: M*N fp16 bits, row-major.  Y (optional, may be
 * NULL): M*N doubles, the value before the final rounding.
 * Row i is computed as: S[:] = 0; for k in 0..K-1: S[:] += A[i][k] * B[k][:].
 * Every S[i][j] therefore sums its K products in increasing k, exactly the
 * order of the plain dot product (so the result does not depend on threads).
 * Returns 0, or -1 on a bad argument / allocation failure.
 */
int oracle_gemm_f16(int64_t M, int64_t N, int64_t K,
                    const uint16_t* A, const uint16_t* B, const uint16_t* bias,
                    uint16_t* C, double* Y, int epilogue, int nthreads) {
    if (M < 0 || N < 0 || K < 0) return -1;
    if (epilogue < 0 || epilogue > 2) return -1;
    if (M == 0 || N == 0) return 0;
    if (epilogue != ORACLE_EPI_NONE && !bias) return -1;
    /* decode B once: K*N doubles */
    double* Bd = (double*)malloc((size_t)(K > 0 ? K : 1) * (size_t)N * sizeof(double));
    if (!Bd) return -1;
    for (int64_t t = 0; t < K * N; ++t) Bd[t] = oracle_f16_decode(B[t]);
    int failed = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
#endif
    {
        double* S = (double*)malloc((size_t)N * sizeof(double));
        if (!S) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            failed = 1;
        } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 4)
#endif
            for (int64_t i = 0; i < M; ++i) {
                for (int64_t j = 0; j < N; ++j) S[j] = 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    double a = oracle_f16_decode(A[i * K + k]);
                    const double* brow = Bd + k * N;
                    for (int64_t j = 0; j < N; ++j) S[j] += a * brow[j];
                }
                for (int64_t j = 0; j < N; ++j) {
                    double y = apply_epilogue(S[j], epilogue, bias, j);
                    if (Y) Y[i * N + j] = y;
                    C[i * N + j] = oracle_f16_encode(y);
                }
            }
            free(S);
        }
    }
    free(Bd);
    return failed ? -1 : 0;
}

/*
 * Selected outputs only: for t in 0..npts-1, C_out[t] = C[rows[t]][cols[t]]
 * computed as the plain dot product over increasing k (same order as above,
 * so the value equals the full product's bit for bit).  Used to check huge
 * shapes at sampled positions.
 */
int oracle_gemm_f16_points(int64_t M, int64_t N, int64_t K,
                           const uint16_t* A, const uint16_t* B, const uint16_t* bias,
                           int epilogue, int64_t npts, const int64_t* rows, const int64_t* cols,
                           uint16_t* C_out, double* Y_out, int nthreads) {
    if (M < 0 || N < 0 || K < 0 || npts < 0) return -1;
    if (epilogue < 0 || epilogue > 2) return -1;
    if (epilogue != ORACLE_EPI_NONE && !bias) return -1;
    for (int64_t t = 0; t < npts; ++t)
        if (rows[t] < 0 || rows[t] >= M || cols[t] < 0 || cols[t] >= N) return -1;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 16)
#endif
    for (int64_t t = 0; t < npts; ++t) {
        int64_t i = rows[t], j = cols[t];
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k)
            s += oracle_f16_decode(A[i * K + k]) * oracle_f16_decode(B[k * N + j]);
        double y = apply_epilogue(s, epilogue, bias, j);
        if (Y_out) Y_out[t] = y;
        C_out[t] = oracle_f16_encode(y);
    }
    return 0;
}

/* Vectorised codec / GELU helpers for the pin tests. */
void oracle_f16_decode_n(const uint16_t* h, double* out, int64_t n) {
    for (int64_t t = 0; t < n; ++t) out[t] = oracle_f16_decode(h[t]);
}
void oracle_f16_encode_n(const double* x, uint16_t* out, int64_t n) {
    for (int64_t t = 0; t < n; ++t) out[t] = oracle_f16_encode(x[t]);
}
void oracle_gelu_n(const double* x, double* out, int64_t n) {
    for (int64_t t = 0; t < n; ++t) out[t] = oracle_gelu(x[t]);
}

/*
 * fp32 vector add, the tutorial's first kernel: C[i] = A[i] + B[i] on float32
 * vectors (blog post "Designing High-Performance GPU Kernels with TileLang",
 * section "Step 3", whose example kernel adds two float32 vectors element by
 * element; news article on TileLang kernel design, paragraph on the vector-add
 * kernel).  The pages fix the precision: float32 in and out, so each result
 * is the IEEE binary32 sum, rounded to nearest-even.  It is formed here as the
 * fp64 sum of the two values, rounded once to binary32.  Rounding an exact sum
 * first to binary64 and then to binary32 gives the correctly rounded binary32
 * sum, because 53 >= 2*24 + 2 (S. A. Figueroa, "When is double rounding
 * innocuous?", ACM SIGNUM Newsletter 30(3), 1995).  NaN inputs give NaN.
 * Returns 0, or -1 on a bad argument.
 */
int oracle_vector_add_f32(int64_t n, const float* A, const float* B, float* C) {
    if (n < 0 || (n > 0 && (!A || !B || !C))) return -1;
    for (int64_t i = 0; i < n; ++i) {
        const double s = (double)A[i] + (double)B[i];
        C[i] = (float)s;
    }
    return 0;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Row-wise softmax of an fp16 matrix, the tutorial's register-resident
 * reduction kernel: per row, a max reduction, then a sum reduction of the
 * shifted exponentials, then the normalisation (news article on TileLang
 * kernel design, paragraph on the fused epilogue, whose last sentences
 * describe the row softmax built from fragment-level max and sum
 * reductions; blog post on TileLang, the "three-piece set" section, item 2:
 * one kernel per row-wise normalisation, with no intermediate in HBM).  The
 * pages give no formula; this is the standard definition, shifted by the
 * row maximum as such kernels do:
 *   m    = max_j x[i][j]                 (NaN entries never win the comparison)
 *   e_j  = exp(x[i][j] - m)              fp64, libm exp
 *   s    = sum_j e_j                     fp64, increasing j
 *   y_j  = e_j / s                       fp64
 *   Y[i][j] = fp16_round_nearest_even(y_j)
 * In IEEE arithmetic this gives: -inf entries -> 0; a row of all -inf
 * (m = -inf, x - m = NaN) -> NaN everywhere; a +inf or NaN entry makes s NaN,
 * so the whole row is NaN.  Yd (optional) receives the fp64 y before rounding.
 * Returns 0, or -1 on a bad argument.
 */
int oracle_softmax_rows_f16(int64_t rows, int64_t cols, const uint16_t* X, uint16_t* Y, double* Yd,
                            int nthreads) {
    if (rows < 0 || cols < 0) return -1;
    if (rows == 0 || cols == 0) return 0;
    if (!X || !Y) return -1;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 8)
#endif
    for (int64_t i = 0; i < rows; ++i) {
        const uint16_t* x = X + i * cols;
        double m = -INFINITY;
        for (int64_t j = 0; j < cols; ++j) {
            double v = oracle_f16_decode(x[j]);
            if (v > m) m = v;
        }
        double s = 0.0;
        for (int64_t j = 0; j < cols; ++j) s += exp(oracle_f16_decode(x[j]) - m);
        for (int64_t j = 0; j < cols; ++j) {
            double y = exp(oracle_f16_decode(x[j]) - m) / s;
            if (Yd) Yd[i * cols + j] = y;
            Y[i * cols + j] = oracle_f16_encode(y);
        }
    }
    return 0;
}

/*
 * Attention forward, the tutorial's FlashAttention workload (news article on
 * TileLang kernel design, paragraph on FlashAttention: query, key and value
 * tiles, an online softmax with running maxima, normalising sums and rescale
 * factors, causal and non-causal variants, checked against PyTorch's scaled
 * dot-product attention; blog post on TileLang, "three-piece set" section,
 * item 3).  The tiled online form only reorganises this plain definition, so
 * the oracle is the definition itself, in fp64:
 *   for each batch b, head h and query row i:
 *     s_j = scale * sum_d Q[i][d] K[j][d]     over the allowed keys j
 *           (j < Nkv; causal: also j <= i, the top-left-aligned mask of
 *            PyTorch's is_causal)
 *     m   = max_j s_j,  p_j = exp(s_j - m),  l = sum_j p_j
 *     O[i][d] = fp16_round_nearest_even( sum_j p_j V[j][d] / l )
 * Q is [B][H][Nq][D], K and V are [B][H][Nkv][D], O is [B][H][Nq][D], all
 * row-major fp16.  Sums run in increasing d and j.  Nkv must be >= 1, so
 * every query row has at least key 0.
 * Od (optional) receives the fp64 values before rounding.
 * Returns 0, or -1 on a bad argument or an allocation failure.
 */
/* One query row: output row r = (b*H + h)*Nq + i of O (and of Od when given). */
static void attention_row(int64_t H, int64_t Nq, int64_t Nkv, int64_t D, const uint16_t* Q, const uint16_t* K,
                          const uint16_t* V, int64_t r, int causal, double scale, double* s, double* acc,
                          uint16_t* O_row, double* Od_row) {
    const int64_t bh = r / Nq, i = r % Nq;
    (void)H;
    const uint16_t* q = Q + r * D;
    const uint16_t* k = K + bh * Nkv * D;
    const uint16_t* v = V + bh * Nkv * D;
    const int64_t nj = causal ? (i + 1 < Nkv ? i + 1 : Nkv) : Nkv;
    double m = -INFINITY;
    for (int64_t j = 0; j < nj; ++j) {
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d) dot += oracle_f16_decode(q[d]) * oracle_f16_decode(k[j * D + d]);
        s[j] = scale * dot;
        if (s[j] > m) m = s[j];
    }
    double l = 0.0;
    for (int64_t d = 0; d < D; ++d) acc[d] = 0.0;
    for (int64_t j = 0; j < nj; ++j) {
        const double pj = exp(s[j] - m);
        l += pj;
        for (int64_t d = 0; d < D; ++d) acc[d] += pj * oracle_f16_decode(v[j * D + d]);
    }
    for (int64_t d = 0; d < D; ++d) {
        const double y = acc[d] / l;
        if (Od_row) Od_row[d] = y;
        O_row[d] = oracle_f16_encode(y);
    }
}

/*
 * rows == NULL: every output row r = (b*H + h)*Nq + i, into O[r*D ..].
 * rows != NULL: only the nrows rows listed (each in [0, B*H*Nq)), into
 * O[t*D ..] for the t-th listed row; for checking large shapes at samples.
 */
static int attention_impl(int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t D, const uint16_t* Q,
                          const uint16_t* K, const uint16_t* V, uint16_t* O, double* Od, int causal, double scale,
                          int64_t nrows, const int64_t* rows, int nthreads) {
    if (B < 0 || H < 0 || Nq < 0 || Nkv < 1 || D < 1 || nrows < 0) return -1;
    if (B == 0 || H == 0 || Nq == 0) return 0;
    const int64_t total = rows ? nrows : B * H * Nq;
    if (rows)
        for (int64_t t = 0; t < nrows; ++t)
            if (rows[t] < 0 || rows[t] >= B * H * Nq) return -1;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
#endif
    {
        double* s = (double*)malloc((size_t)Nkv * sizeof(double));
        double* acc = (double*)malloc((size_t)D * sizeof(double));
        if (!s || !acc) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            failed = 1;
        } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 4)
#endif
            for (int64_t t = 0; t < total; ++t) {
                const int64_t r = rows ? rows[t] : t;
                attention_row(H, Nq, Nkv, D, Q, K, V, r, causal, scale, s, acc, O + t * D, Od ? Od + t * D : NULL);
            }
        }
        free(s);
        free(acc);
    }
    return failed ? -1 : 0;
}

int oracle_attention_f16(int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t D, const uint16_t* Q,
                         const uint16_t* K, const uint16_t* V, uint16_t* O, double* Od, int causal, double scale,
                         int nthreads) {
    return attention_impl(B, H, Nq, Nkv, D, Q, K, V, O, Od, causal, scale, 0, NULL, nthreads);
}

int oracle_attention_f16_rows(int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t D, const uint16_t* Q,
                              const uint16_t* K, const uint16_t* V, int causal, double scale, int64_t nrows,
                              const int64_t* rows, uint16_t* O_rows, double* Od_rows, int nthreads) {
    return attention_impl(B, H, Nq, Nkv, D, Q, K, V, O_rows, Od_rows, causal, scale, nrows, rows, nthreads);
}
