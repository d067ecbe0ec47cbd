/*
 * oracle.c -- the reference GEMM that the pipelined GPU kernels are checked
 * against.  TEST INFRASTRUCTURE ONLY: only the tests, the package's smoke
 * entry and the benchmark's CPU-baseline leg may load this library.  The
 * product path never calls it and shares no code, header or table with it.
 *
 * What it computes (the plain definition, written out):
 *
 *     C[i*ldc + j] = alpha * sum_{k=0}^{K-1} A[i*lda + k] * B[k*ldb + j]
 *                    + beta * C0[i*ldc + j]
 *
 * for 0 <= i < M, 0 <= j < N, with A, B, C row-major.  This is the epilogue
 * and indexing of the double-buffered SGEMM kernel on the page "Double
 * Buffering: Software Pipelining the K-Loop" (section "The Kernel": A indexed
 * by row*K + k, B by k*N + col, and the alpha/beta read-modify-write of C),
 * with general leading dimensions in place of the page's tight K, N, N.
 * Software pipelining reorders only the loads and leaves the arithmetic as it
 * is (page "GPU-Kernel pipelinen", step 5 on correctness; same point in the
 * first page's section "What The Overlap Cost"), so the plain triple loop is
 * the exact target up to floating-point summation order.
 *
 * Readings where the pages are silent:
 *   - beta == 0: C0 is not read at all (BLAS convention), so NaN/Inf in C0
 *     do not reach C.
 *   - K == 0: the sum is empty and C = beta*C0 (C0 unread if beta == 0).
 *   - Float inputs (fp32, fp16, bf16) are decoded exactly to double, the sum
 *     runs in double in increasing k, and the result is returned in double.
 *   - int8 inputs: the sum and the epilogue run in exact 64-bit integers;
 *     alpha and beta are integers; the stored int32 value is the exact result
 *     reduced modulo 2^32 (two's complement), which is what int32 arithmetic
 *     produces.  The function returns how many outputs did not fit in int32
 *     (and, separately via *acc_overflow, how many raw sums did not) so tests
 *     can assert that a workload never wraps.
 *
 * Loop order: rows i in parallel (OpenMP), then k, then j with one
 * accumulator per output of the row (double for floats, int64 for int8).  For
 * each output the sum is therefore formed in increasing k, independent of the
 * thread count.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC (no -march, no
 * fast-math: the arithmetic is exactly what is written).
 */
#include <stdint.h>
#include <string.h>
#include <math.h>
#include <stdlib.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- element decoders (written from the IEEE-754 / bfloat16 formats) ---- */

/* bfloat16 is the top 16 bits of an IEEE-754 binary32. */
static double dec_bf16(uint16_t h) {
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* IEEE-754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 mantissa bits. */
static double dec_f16(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)m, -24);             /* zero or subnormal: m * 2^-24 */
    } else if (e == 31) {
        v = (m == 0) ? INFINITY : NAN;
    } else {
        v = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
    }
    return sign ? -v : v;
}

static double dec_f32(float f) { return (double)f; }

enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2 };

static double load_elem(const void* p, int64_t idx, int kind) {
    switch (kind) {
    case OR_F32: return dec_f32(((const float*)p)[idx]);
    case OR_F16: return dec_f16(((const uint16_t*)p)[idx]);
    default: return dec_bf16(((const uint16_t*)p)[idx]);
    }
}

/* Decoders exported so tests can pin them against independent libraries. */
double oracle_decode_f16(uint16_t h) { return dec_f16(h); }
double oracle_decode_bf16(uint16_t h) { return dec_bf16(h); }

/*
 * Float GEMM.  kind: 0 = fp32 inputs, 1 = fp16, 2 = bf16.  C0 is fp32 (the
 * output type of every float configuration) and is read only when
 * beta != 0.  Out is M x ldo doubles.  Returns 0, or -1 on a bad argument.
 */
int oracle_gemm_float(int kind, int64_t M, int64_t N, int64_t K, double alpha,
                      const void* A, int64_t lda, const void* B, int64_t ldb,
                      double beta, const float* C0, int64_t ldc,
                      double* out, int64_t ldo, double* row_scratch) {
    if (M < 0 || N < 0 || K < 0) return -1;
    if (kind < 0 || kind > 2) return -1;
    if (M == 0 || N == 0) return 0;
    if (lda < K || ldb < N || ldo < N || (beta != 0.0 && ldc < N)) return -1;
    (void)row_scratch;
    int64_t i;
#pragma omp parallel for schedule(dynamic, 1)
    for (i = 0; i < M; ++i) {
        double* acc = out + i * ldo;   /* the row of Out doubles as the accumulator */
        for (int64_t j = 0; j < N; ++j) acc[j] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double a = load_elem(A, i * lda + k, kind);
            for (int64_t j = 0; j < N; ++j)
                acc[j] += a * load_elem(B, k * ldb + j, kind);
        }
        for (int64_t j = 0; j < N; ++j) {
            double v = alpha * acc[j];
            if (beta != 0.0) v += beta * (double)C0[i * ldc + j];
            acc[j] = v;
        }
    }
    return 0;
}

/*
 * int8 GEMM with int32 output.  alpha and beta are integers.  Exact int64
 * arithmetic; Out[i*ldc+j] = (int32) (result mod 2^32).  Returns the number
 * of outputs whose exact value lies outside int32 (0 for every shipped
 * workload), or -1 on a bad argument.  *acc_overflow (if non-null) receives
 * the number of raw sums outside int32.
 */
int64_t oracle_gemm_i8(int64_t M, int64_t N, int64_t K, int64_t alpha,
                       const int8_t* A, int64_t lda, const int8_t* B, int64_t ldb,
                       int64_t beta, const int32_t* C0, int64_t ldc,
                       int32_t* out, int64_t ldo, int64_t* acc_overflow) {
    if (M < 0 || N < 0 || K < 0) return -1;
    if (acc_overflow) *acc_overflow = 0;
    if (M == 0 || N == 0) return 0;
    if (lda < K || ldb < N || ldo < N || (beta != 0 && ldc < N)) return -1;
    int64_t n_out_over = 0, n_acc_over = 0;
    int64_t i;
    int bad_alloc = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : n_out_over, n_acc_over, bad_alloc)
    for (i = 0; i < M; ++i) {
        /* exact integer sums: the summation order does not matter */
        int64_t* s = (int64_t*)calloc((size_t)N, sizeof(int64_t));
        if (!s) { bad_alloc++; continue; }
        for (int64_t k = 0; k < K; ++k) {
            const int64_t a = (int64_t)A[i * lda + k];
            for (int64_t j = 0; j < N; ++j)
                s[j] += a * (int64_t)B[k * ldb + j];
        }
        for (int64_t j = 0; j < N; ++j) {
            if (s[j] < INT32_MIN || s[j] > INT32_MAX) n_acc_over++;
            /* alpha*s and beta*C0 fit in int64: |alpha|, |beta| <= 2^31 (int32 values),
             * |s| <= K * 2^14 and |C0| <= 2^31, so for K <= 2^16 the sum stays below 2^63. */
            int64_t v = alpha * s[j];
            if (beta != 0) v += beta * (int64_t)C0[i * ldc + j];
            if (v < INT32_MIN || v > INT32_MAX) n_out_over++;
            out[i * ldo + j] = (int32_t)(uint32_t)(uint64_t)v;
        }
        free(s);
    }
    if (bad_alloc) return -1;
    if (acc_overflow) *acc_overflow = n_acc_over;
    return n_out_over;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
