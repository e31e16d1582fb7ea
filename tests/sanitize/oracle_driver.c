/* The C oracle on exactly sized heap buffers (so a read one element past an
 * operand trips AddressSanitizer), for every transpose pair, padded leading
 * dimensions and the degenerate sizes, under AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_sanitizers.py). Also checks that the
 * entries functions agree bitwise with the full results. Exits non-zero on a
 * failed expectation. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_gemm(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda, const float *B, int64_t ldb,
                double *C, int64_t ldc, double *S, int64_t lds);
int oracle_gemm_entries(int64_t n, const int64_t *rows, const int64_t *cols, int64_t K, const float *A,
                        int64_t lda, const float *B, int64_t ldb, double *out, double *sabs);
int oracle_gemm_ex(int transA, int transB, int64_t M, int64_t N, int64_t K, double alpha, const float *A,
                   int64_t lda, const float *B, int64_t ldb, double beta, const float *C_in, int64_t ldc_in,
                   double *Out, int64_t ldo, double *Sout, int64_t lds);
int oracle_gemm_ex_entries(int transA, int transB, int64_t n, const int64_t *rows, const int64_t *cols, int64_t K,
                           double alpha, const float *A, int64_t lda, const float *B, int64_t ldb, double beta,
                           const float *C_in, int64_t ldc_in, double *Out, double *Sout);

static int failures = 0;
static uint64_t state = 12345;

static float draw(void)
{
    state = state * 6364136223846793005ULL + 1442695040888963407ULL;
    return (float)((int)(state >> 40) % 17 - 8);
}

/* rows x cols matrix with leading dimension ld, in a buffer of exactly the
 * elements that matrix spans (NULL when it spans none). */
static float *matrix(int64_t rows, int64_t cols, int64_t ld)
{
    if (rows == 0 || cols == 0) return NULL;
    const int64_t n = (rows - 1) * ld + cols;
    float *p = (float *)malloc((size_t)n * sizeof(float));
    for (int64_t i = 0; i < n; ++i) p[i] = draw();
    return p;
}

static void one(int64_t M, int64_t N, int64_t K, int ta, int tb, int64_t pad)
{
    const int64_t ar = ta ? K : M, ac = ta ? M : K, br = tb ? N : K, bc = tb ? K : N;
    const int64_t lda = (ac > 0 ? ac : 1) + pad, ldb = (bc > 0 ? bc : 1) + pad, ldc = (N > 0 ? N : 1) + pad;
    float *A = matrix(ar, ac, lda), *B = matrix(br, bc, ldb), *C0 = matrix(M, N, ldc);
    double *Out = (double *)malloc((size_t)(M * N > 0 ? M * N : 1) * sizeof(double));
    double *S = (double *)malloc((size_t)(M * N > 0 ? M * N : 1) * sizeof(double));
    if (oracle_gemm_ex(ta, tb, M, N, K, 0.5, A, lda, B, ldb, -2.0, C0, ldc, Out, N, S, N) != 0) {
        fprintf(stderr, "FAILED: oracle_gemm_ex %lld %lld %lld\n", (long long)M, (long long)N, (long long)K);
        ++failures;
    }
    if (M > 0 && N > 0) {
        const int64_t n = M * N;
        int64_t *rows = (int64_t *)malloc((size_t)n * sizeof(int64_t));
        int64_t *cols = (int64_t *)malloc((size_t)n * sizeof(int64_t));
        for (int64_t e = 0; e < n; ++e) {
            rows[e] = e / N;
            cols[e] = e % N;
        }
        double *E = (double *)malloc((size_t)n * sizeof(double));
        double *ES = (double *)malloc((size_t)n * sizeof(double));
        oracle_gemm_ex_entries(ta, tb, n, rows, cols, K, 0.5, A, lda, B, ldb, -2.0, C0, ldc, E, ES);
        if (memcmp(E, Out, (size_t)n * sizeof(double)) != 0 || memcmp(ES, S, (size_t)n * sizeof(double)) != 0) {
            fprintf(stderr, "FAILED: ex entries differ %lld %lld %lld\n", (long long)M, (long long)N, (long long)K);
            ++failures;
        }
        if (!ta && !tb) {
            double *P = (double *)malloc((size_t)n * sizeof(double));
            double *PS = (double *)malloc((size_t)n * sizeof(double));
            oracle_gemm(M, N, K, A, lda, B, ldb, P, N, PS, N);
            oracle_gemm_entries(n, rows, cols, K, A, lda, B, ldb, E, ES);
            if (memcmp(E, P, (size_t)n * sizeof(double)) != 0 || memcmp(ES, PS, (size_t)n * sizeof(double)) != 0) {
                fprintf(stderr, "FAILED: entries differ %lld %lld %lld\n", (long long)M, (long long)N, (long long)K);
                ++failures;
            }
            free(P);
            free(PS);
        }
        free(rows);
        free(cols);
        free(E);
        free(ES);
    }
    free(A);
    free(B);
    free(C0);
    free(Out);
    free(S);
}

int main(void)
{
    const int64_t sizes[] = {0, 1, 2, 5, 17, 33};
    for (int a = 0; a < 6; ++a)
        for (int b = 0; b < 6; ++b)
            for (int c = 0; c < 6; ++c)
                for (int t = 0; t < 4; ++t)
                    one(sizes[a], sizes[b], sizes[c], t & 1, t >> 1, (a + b + c + t) % 3);
    if (oracle_gemm(-1, 1, 1, NULL, 1, NULL, 1, NULL, 1, NULL, 1) != -1) {
        fprintf(stderr, "FAILED: negative size accepted\n");
        ++failures;
    }
    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    printf("oracle ok\n");
    return 0;
}
