/* Drives the oracle's C code under the address and undefined-behaviour
 * sanitizers: every entry point on small shapes, tight and padded leading
 * dimensions, beta zero and nonzero, K = 0, M or N = 0, int8 sums that
 * overflow int32, and bad arguments.  Every buffer is allocated at its exact
 * size, so a read or write one element outside it is reported.  This checks
 * memory safety; the oracle's values are pinned elsewhere.  Prints "OK <n>". */
#include "../oracle/oracle.c"

#include <stdio.h>

static void* exact(size_t bytes) { return malloc(bytes ? bytes : 1); }

int main(void) {
    const int64_t sizes[] = {0, 1, 2, 3, 7, 16, 33};
    int calls = 0;
    for (int kind = 0; kind <= 2; ++kind) {
        const size_t es = kind == 0 ? 4 : 2;
        for (int a = 0; a < 7; ++a)
            for (int b = 0; b < 7; ++b)
                for (int c = 0; c < 7; ++c)
                    for (int pad = 0; pad <= 3; pad += 3) {
                        const int64_t M = sizes[a], N = sizes[b], K = sizes[c];
                        const int64_t lda = K + pad, ldb = N + pad, ldc = N + pad, ldo = N;
                        unsigned char* A = exact((size_t)(M ? (M - 1) * lda + K : 0) * es);
                        unsigned char* B = exact((size_t)(K ? (K - 1) * ldb + N : 0) * es);
                        float* C0 = exact((size_t)(M ? (M - 1) * ldc + N : 0) * sizeof(float));
                        double* out = exact((size_t)(M * ldo) * sizeof(double));
                        for (size_t i = 0; i < (size_t)(M ? (M - 1) * lda + K : 0) * es; ++i) A[i] = (unsigned char)(i * 7 + 1);
                        for (size_t i = 0; i < (size_t)(K ? (K - 1) * ldb + N : 0) * es; ++i) B[i] = (unsigned char)(i * 5 + 3);
                        for (size_t i = 0; i < (size_t)(M ? (M - 1) * ldc + N : 0); ++i) C0[i] = (float)i;
                        for (int beta_nz = 0; beta_nz <= 1; ++beta_nz) {
                            const int r = oracle_gemm_float(kind, M, N, K, 1.5, A, lda, B, ldb, beta_nz ? -0.5 : 0.0,
                                                            C0, ldc, out, ldo, NULL);
                            ++calls;
                            if (r != 0) { printf("FAIL float kind %d %lld %lld %lld\n", kind, (long long)M, (long long)N, (long long)K); return 1; }
                        }
                        free(A); free(B); free(C0); free(out);
                    }
    }
    for (int a = 0; a < 7; ++a)
        for (int b = 0; b < 7; ++b)
            for (int c = 0; c < 7; ++c) {
                const int64_t M = sizes[a], N = sizes[b], K = sizes[c] * 40;
                const int64_t lda = K + 1, ldb = N + 2, ldc = N + 3, ldo = N;
                int8_t* A = exact((size_t)(M ? (M - 1) * lda + K : 0));
                int8_t* B = exact((size_t)(K ? (K - 1) * ldb + N : 0));
                int32_t* C0 = exact((size_t)(M ? (M - 1) * ldc + N : 0) * sizeof(int32_t));
                int32_t* out = exact((size_t)(M * ldo) * sizeof(int32_t));
                for (int64_t i = 0; i < (M ? (M - 1) * lda + K : 0); ++i) A[i] = -128;
                for (int64_t i = 0; i < (K ? (K - 1) * ldb + N : 0); ++i) B[i] = -128;
                for (int64_t i = 0; i < (M ? (M - 1) * ldc + N : 0); ++i) C0[i] = INT32_MAX;
                int64_t acc_over = -1;
                const int64_t r = oracle_gemm_i8(M, N, K, 3, A, lda, B, ldb, -2, C0, ldc, out, ldo, &acc_over);
                ++calls;
                if (r < 0) { printf("FAIL i8 %lld %lld %lld\n", (long long)M, (long long)N, (long long)K); return 1; }
                free(A); free(B); free(C0); free(out);
            }
    /* bad arguments are refused without touching memory */
    calls += 4;
    if (oracle_gemm_float(3, 1, 1, 1, 1.0, NULL, 1, NULL, 1, 0.0, NULL, 1, NULL, 1, NULL) != -1) return 1;
    if (oracle_gemm_float(0, 2, 2, 2, 1.0, NULL, 1, NULL, 2, 0.0, NULL, 2, NULL, 2, NULL) != -1) return 1;
    if (oracle_gemm_i8(-1, 1, 1, 1, NULL, 1, NULL, 1, 0, NULL, 1, NULL, 1, NULL) != -1) return 1;
    if (oracle_gemm_i8(2, 2, 2, 1, NULL, 2, NULL, 1, 0, NULL, 2, NULL, 2, NULL) != -1) return 1;
    for (unsigned h = 0; h < 65536; h += 7) { (void)oracle_decode_f16((uint16_t)h); (void)oracle_decode_bf16((uint16_t)h); ++calls; }
    printf("OK %d\n", calls);
    return 0;
}
