/*
 * CPU oracle for the FP32 matrix product C = A * B and its general form
 * C = alpha * op(A) * op(B) + beta * C.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the library calls this; only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg load it. It
 * shares no source with the GPU path.
 *
 * Definition followed ("Shared Memory Tiling for Matrix Multiplication",
 * opening definition; "Matrix Multiplication -- Naive to Tiled", section 02):
 *     C[i][j] = sum over k = 0 .. K-1 of A[i][k] * B[k][j]
 * with A of M x K, B of K x N, C of M x N, all stored row-major; a leading
 * dimension gives the distance in elements between consecutive rows.
 *
 * Precision: every product and partial sum is formed in double, and each
 * C[i][j] is summed in ascending k, exactly as the textbook triple loop does
 * it. The loops are written i, k, j: that only changes which element is
 * worked on next, never the order of the terms of any one element, so the
 * result is bit-for-bit the i, j, k loop's. The rows are shared among OpenMP
 * threads; each element is still summed by one thread in ascending k.
 *
 * Alongside C the oracle can return S[i][j] = sum_k |A[i][k]| * |B[k][j]|,
 * which scales the elementwise error bound of a float32 result.
 *
 * oracle_gemm_ex adds the scalars and transpose flags of the BLAS-style call
 * (C = alpha * op(A) * op(B) + beta * C) with the same per-element order.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off (no -ffast-math: the sums must not
 * be reassociated).
 */
#include <stdint.h>
#include <stddef.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double absd(double x) { return x < 0.0 ? -x : x; }

/* Full product. C (and S, when not NULL) receive M x N doubles with leading
 * dimension ldc (lds). Returns 0, or -1 on a negative size. */
int oracle_gemm(int64_t M, int64_t N, int64_t K,
                const float *A, int64_t lda,
                const float *B, int64_t ldb,
                double *C, int64_t ldc,
                double *S, int64_t lds)
{
    if (M < 0 || N < 0 || K < 0) return -1;
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < M; ++i) {
        double *c = C + i * ldc;
        double *s = S ? S + i * lds : NULL;
        for (int64_t j = 0; j < N; ++j) c[j] = 0.0;
        if (s)
            for (int64_t j = 0; j < N; ++j) s[j] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = (double)A[i * lda + k];
            const float *b = B + k * ldb;
            for (int64_t j = 0; j < N; ++j) c[j] += a * (double)b[j];
            if (s) {
                const double aa = absd(a);
                for (int64_t j = 0; j < N; ++j) s[j] += aa * absd((double)b[j]);
            }
        }
    }
    return 0;
}

/* Selected elements only: out[e] = C[rows[e]][cols[e]] (and sabs[e] = S[..]
 * when sabs is not NULL), each summed in ascending k like oracle_gemm. For
 * checking a few outputs of a product too large to form on the CPU. */
int oracle_gemm_entries(int64_t n, const int64_t *rows, const int64_t *cols,
                        int64_t K,
                        const float *A, int64_t lda,
                        const float *B, int64_t ldb,
                        double *out, double *sabs)
{
    if (n < 0 || K < 0) return -1;
    int64_t e;
#pragma omp parallel for schedule(static)
    for (e = 0; e < n; ++e) {
        const int64_t i = rows[e], j = cols[e];
        double acc = 0.0, accabs = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = (double)A[i * lda + k];
            const double b = (double)B[k * ldb + j];
            acc += a * b;
            accabs += absd(a) * absd(b);
        }
        out[e] = acc;
        if (sabs) sabs[e] = accabs;
    }
    return 0;
}

/* The general form C = alpha * op(A) * op(B) + beta * C of the vendor call
 * on "Matrix Multiplication -- Naive to Tiled", section 07 (where alpha = 1,
 * beta = 0), with op(X) = X or its transpose:
 *   op(A) is M x K: transA == 0 reads A[i][k] = A[i*lda + k] (A stored M x K),
 *                   transA != 0 reads A[k][i] = A[k*lda + i] (A stored K x M);
 *   op(B) is K x N: transB == 0 reads B[k*ldb + j] (B stored K x N),
 *                   transB != 0 reads B[j*ldb + k] (B stored N x K).
 * C_in (M x N float, leading dimension ldc_in) is read only when beta != 0;
 * A and B only when alpha != 0. The result of element (i, j) is
 * alpha * sum_k op(A)[i][k] op(B)[k][j] + beta * C_in[i][j], and its error
 * scale is |alpha| * sum_k |op(A)[i][k]| |op(B)[k][j]| + |beta * C_in[i][j]|.
 * Each sum runs in ascending k, in double. */
static void ex_element(int transA, int transB, int64_t i, int64_t j, int64_t K, double alpha, const float *A,
                       int64_t lda, const float *B, int64_t ldb, double beta, const float *C_in, int64_t ldc_in,
                       double *out, double *scale)
{
    double acc = 0.0, accabs = 0.0;
    if (alpha != 0.0) {
        for (int64_t k = 0; k < K; ++k) {
            const double a = (double)(transA ? A[k * lda + i] : A[i * lda + k]);
            const double b = (double)(transB ? B[j * ldb + k] : B[k * ldb + j]);
            acc += a * b;
            accabs += absd(a) * absd(b);
        }
    }
    const double c = beta != 0.0 ? beta * (double)C_in[i * ldc_in + j] : 0.0;
    *out = alpha * acc + c;
    *scale = absd(alpha) * accabs + absd(c);
}

/* The whole M x N result into Out (double, leading dimension ldo) and, when
 * Sout is not NULL, the error scales into Sout (leading dimension lds). */
int oracle_gemm_ex(int transA, int transB, int64_t M, int64_t N, int64_t K, double alpha,
                   const float *A, int64_t lda, const float *B, int64_t ldb, double beta,
                   const float *C_in, int64_t ldc_in, double *Out, int64_t ldo, double *Sout, int64_t lds)
{
    if (M < 0 || N < 0 || K < 0) return -1;
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < M; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            double s;
            ex_element(transA, transB, i, j, K, alpha, A, lda, B, ldb, beta, C_in, ldc_in, &Out[i * ldo + j], &s);
            if (Sout) Sout[i * lds + j] = s;
        }
    }
    return 0;
}

/* Selected elements: Out[e] (and Sout[e] when not NULL) for element
 * (rows[e], cols[e]) of oracle_gemm_ex's result, formed the same way. */
int oracle_gemm_ex_entries(int transA, int transB, int64_t n, const int64_t *rows, const int64_t *cols, int64_t K,
                           double alpha, const float *A, int64_t lda, const float *B, int64_t ldb, double beta,
                           const float *C_in, int64_t ldc_in, double *Out, double *Sout)
{
    if (n < 0 || K < 0) return -1;
    int64_t e;
#pragma omp parallel for schedule(static)
    for (e = 0; e < n; ++e) {
        double s;
        ex_element(transA, transB, rows[e], cols[e], K, alpha, A, lda, B, ldb, beta, C_in, ldc_in, &Out[e], &s);
        if (Sout) Sout[e] = s;
    }
    return 0;
}

/* Number of OpenMP threads a parallel region of the oracle will use. */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
