/*
 * CPU oracle for single-precision GEMM:  C = alpha * A * B + beta * C_in.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * reference that the GPU library is checked against.  Only the test suite,
 * the package smoke check and the benchmark's CPU-baseline leg may load it.
 * It shares no code, header or build step with the HIP library, and the HIP
 * library never calls it.
 *
 * What it computes (the plain definition, evaluated in fp64):
 *   - Problem statement: C = A . B with A of shape [M,K], B of shape [K,N],
 *     C of shape [M,N], all row-major FP32; each output is a length-K dot
 *     product ("Matmul I: tiling and shared memory", section 1).
 *   - Epilogue form alpha*acc + beta*C ("2D Register Tiling: The Outer
 *     Product", The Kernel; "The Final Kernel", Skipping The Read Of C).
 *   - beta == 0 means C_in is not read at all, so NaN or Inf in C_in never
 *     reaches the result ("The Final Kernel", Skipping The Read Of C).
 *   - Elements outside [0,M)x[0,K) and [0,K)x[0,N) contribute nothing; only
 *     in-range outputs exist ("Matmul I", section 6, notes 1-2).
 *
 * Arithmetic: every product (double)a * (double)b of two floats is exact in
 * fp64 (24 + 24 significand bits < 53).  The products are summed in fp64 with
 * k ascending, then alpha*S + beta*C_in is formed in fp64 and returned in
 * fp64.  Rows are independent, so the OpenMP split over rows leaves every
 * bit of the result unchanged for any thread count.
 *
 * Layout: row-major with leading dimensions, A[i*lda + k], B[k*ldb + j],
 * C_in[i*ldc + j], out[i*ldo + j].  Columns beyond the logical extent
 * (k >= K in A, j >= N in B and C_in) are never read.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC (no -ffast-math,
 * no BLAS).
 */
#include <stdlib.h>
#include <omp.h>

#define ORACLE_VERSION 1

int oracle_version(void) { return ORACLE_VERSION; }

/* Threads the next call may use; n <= 0 leaves the OpenMP default. */
void oracle_set_threads(int n) {
    if (n > 0) omp_set_num_threads(n);
}

int oracle_max_threads(void) { return omp_get_max_threads(); }

/*
 * Full product.  out must hold M rows of ldo >= N doubles.
 * Returns 0 on success, -1 on a bad dimension, -2 on allocation failure.
 */
int oracle_sgemm_f64(int M, int N, int K, float alpha,
                     const float *A, long lda,
                     const float *B, long ldb,
                     float beta, const float *C_in, long ldc,
                     double *out, long ldo)
{
    if (M < 0 || N < 0 || K < 0) return -1;
    if (M == 0 || N == 0) return 0;
    if (ldo < N) return -1;
    if (K > 0 && (lda < K || ldb < N)) return -1;
    if (beta != 0.0f && ldc < N) return -1;

    const double a_s = (double)alpha;
    const double b_s = (double)beta;
    int failed = 0;

    #pragma omp parallel
    {
        double *S = (double *)malloc((size_t)N * sizeof(double));
        if (S == NULL) {
            #pragma omp atomic write
            failed = 1;
        }
        #pragma omp for schedule(static)
        for (long i = 0; i < M; ++i) {
            if (S == NULL) continue;
            for (long j = 0; j < N; ++j) S[j] = 0.0;
            /* S[j] = sum over k = 0..K-1, ascending, of A[i][k] * B[k][j] */
            for (long k = 0; k < K; ++k) {
                const double a = (double)A[i * lda + k];
                const float *Bk = B + k * ldb;
                for (long j = 0; j < N; ++j) S[j] += a * (double)Bk[j];
            }
            double *o = out + i * ldo;
            if (beta == 0.0f) {
                for (long j = 0; j < N; ++j) o[j] = a_s * S[j];
            } else {
                const float *c = C_in + i * ldc;
                for (long j = 0; j < N; ++j) o[j] = a_s * S[j] + b_s * (double)c[j];
            }
        }
        free(S);
    }
    return failed ? -2 : 0;
}

/*
 * Selected outputs only: out[s] = C[I[s]][J[s]] for s in [0, n).
 * Each entry is the same k-ascending fp64 dot product as the full product,
 * so a sampled entry is bitwise equal to the matching full-product entry.
 * Returns 0 on success, -1 on a bad dimension or an index out of range.
 */
int oracle_sgemm_sampled(int M, int N, int K, float alpha,
                         const float *A, long lda,
                         const float *B, long ldb,
                         float beta, const float *C_in, long ldc,
                         long n, const long *I, const long *J, double *out)
{
    if (M < 0 || N < 0 || K < 0 || n < 0) return -1;
    if (K > 0 && (lda < K || ldb < N)) return -1;
    if (beta != 0.0f && ldc < N) return -1;
    for (long s = 0; s < n; ++s)
        if (I[s] < 0 || I[s] >= M || J[s] < 0 || J[s] >= N) return -1;

    const double a_s = (double)alpha;
    const double b_s = (double)beta;

    #pragma omp parallel for schedule(static)
    for (long s = 0; s < n; ++s) {
        const long i = I[s], j = J[s];
        double S = 0.0;
        for (long k = 0; k < K; ++k) S += (double)A[i * lda + k] * (double)B[k * ldb + j];
        double v = a_s * S;
        if (beta != 0.0f) v = v + b_s * (double)C_in[i * ldc + j];
        out[s] = v;
    }
    return 0;
}
