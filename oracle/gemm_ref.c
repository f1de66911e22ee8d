/*
 * gemm_ref.c -- CPU oracle for the FP32 matrix product C = op(A) . op(B).
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke
 * check and the CPU-baseline leg of the benchmark may load this library.  It
 * shares no source, header, table or build step with the HIP library, and the
 * HIP library never calls it.
 *
 * What it computes.  The pages define the product by its naive loop: one
 * output element per (row, column), a running sum over k of A[row][k] times
 * B[k][col] ("3 . La memoire partagee", section 3.1, the naive kernel; the
 * same definition, rectangular M x K times K x N and row-major, appears in the
 * cuda-oxide book's tiled_sgemm listing).  The tiled kernels on those pages
 * reach the same product and only change where operands are read from, so
 * the plain definition is the oracle for every kernel.  Written out:
 *
 *     C[i][j] = sum_{k=0}^{K-1} opA(i, k) * opB(k, j)      0 <= i < M, 0 <= j < N
 *
 *     opA(i, k) = A[i*lda + k]  (transA == 0, A stored M x K)
 *               = A[k*lda + i]  (transA == 1, A stored K x M)
 *     opB(k, j) = B[k*ldb + j]  (transB == 0, B stored K x N)
 *               = B[j*ldb + k]  (transB == 1, B stored N x K)
 *
 * Products and sums are taken in double precision.  The product of two
 * float32 values is exact in double (24 + 24 significand bits < 53), so the
 * only rounding is in the running double sum, k in increasing order.  The
 * result is returned in double and is never rounded to float.
 *
 * The loops are the definition and nothing more: rows are split across
 * OpenMP threads, each (i, j) is a straight k loop.  No blocking, no
 * reordering of the sum.
 *
 * Counting.  When `stats` is not NULL the oracle also counts, per output
 * element, the multiply-adds it performs and the operand elements it reads
 * (one from A and one from B per multiply-add), which is how section 3.1 of
 * the course page counts the naive kernel's operations and bytes.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

static double op_a(const float *A, int64_t lda, int transA, int64_t i, int64_t k)
{
    return transA ? (double)A[k * lda + i] : (double)A[i * lda + k];
}

static double op_b(const float *B, int64_t ldb, int transB, int64_t k, int64_t j)
{
    return transB ? (double)B[j * ldb + k] : (double)B[k * ldb + j];
}

static double dot(int64_t K, const float *A, int64_t lda, int transA,
                  const float *B, int64_t ldb, int transB, int64_t i, int64_t j)
{
    double s = 0.0;
    for (int64_t k = 0; k < K; ++k)
        s += op_a(A, lda, transA, i, k) * op_b(B, ldb, transB, k, j);
    return s;
}

/* Checks only what keeps the loops in bounds of the described storage. */
static int args_ok(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                   int transA, int transB)
{
    if (M < 0 || N < 0 || K < 0) return 0;
    if ((transA != 0 && transA != 1) || (transB != 0 && transB != 1)) return 0;
    if (lda < (transA ? M : K)) return 0;
    if (ldb < (transB ? K : N)) return 0;
    return 1;
}

/*
 * Full product.  C is an M x N double array with leading dimension ldc.
 * stats (nullable): stats[0] += multiply-adds, stats[1] += operand reads.
 * Returns 0, or -1 on arguments that do not describe valid storage.
 */
int gemm_ref_f64(int64_t M, int64_t N, int64_t K,
                 const float *A, int64_t lda, const float *B, int64_t ldb,
                 double *C, int64_t ldc, int transA, int transB, int64_t *stats)
{
    if (!args_ok(M, N, K, lda, ldb, transA, transB) || ldc < N) return -1;
    int64_t macs = 0, reads = 0;
#pragma omp parallel for schedule(static) reduction(+ : macs, reads)
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            C[i * ldc + j] = dot(K, A, lda, transA, B, ldb, transB, i, j);
            macs += K;
            reads += 2 * K;
        }
    }
    if (stats) {
        stats[0] += macs;
        stats[1] += reads;
    }
    return 0;
}

/*
 * Selected entries: out[t] = C[rows[t]][cols[t]] for t < count.  Lets the
 * tests check full-size products one element at a time.
 * Returns 0, -1 on bad storage arguments, -2 on an index outside M x N.
 */
int gemm_ref_f64_entries(int64_t M, int64_t N, int64_t K,
                         const float *A, int64_t lda, const float *B, int64_t ldb,
                         int transA, int transB, int64_t count,
                         const int64_t *rows, const int64_t *cols, double *out)
{
    if (!args_ok(M, N, K, lda, ldb, transA, transB) || count < 0) return -1;
    for (int64_t t = 0; t < count; ++t)
        if (rows[t] < 0 || rows[t] >= M || cols[t] < 0 || cols[t] >= N) return -2;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t t = 0; t < count; ++t)
        out[t] = dot(K, A, lda, transA, B, ldb, transB, rows[t], cols[t]);
    return 0;
}

/*
 * Fused-epilogue reference, in place on a double result:
 *     C[i][j] = act(C[i][j] + bias[j])      (bias may be NULL: no bias)
 * act 0: identity.  act 1: GELU, x * Phi(x) with Phi the standard normal
 * distribution function, Phi(x) = (1 + erf(x / sqrt 2)) / 2.  Both in double.
 * Returns 0, or -1 for an unknown act.
 */
int gemm_ref_epilogue(int64_t M, int64_t N, double *C, int64_t ldc,
                      const float *bias, int act)
{
    if (act != 0 && act != 1) return -1;
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            double x = C[i * ldc + j] + (bias ? (double)bias[j] : 0.0);
            if (act == 1) x = x * 0.5 * (1.0 + erf(x / sqrt(2.0)));
            C[i * ldc + j] = x;
        }
    }
    return 0;
}

/*
 * Mixed precision (the Smallem page, "Rendre le GPU rapide", section "Les
 * Tensor Cores").  A bf16 is the upper 16 bits of a float32: same sign and
 * exponent, 7 stored significand bits.  The page rounds to the nearest bf16
 * by adding half a step to the 32-bit pattern before dropping its low 16
 * bits; the half step is 0x7FFF plus the lowest bit that is kept, so an
 * exact tie goes to the neighbour whose last kept bit is 0 (ties to even).
 * The carry out of the significand moves the exponent up, and the largest
 * values round to infinity, as the bit pattern arithmetic gives by itself.
 * NaN is returned unchanged (the page does not treat it).  The result is
 * returned as the float32 it stands for (low 16 bits zero).
 */
static float round_bf16(float x)
{
    if (isnan(x)) return x;
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    u &= 0xFFFF0000u;
    memcpy(&x, &u, sizeof x);
    return x;
}

/* out[t] = round_bf16(in[t]) for t < n. */
void gemm_ref_round_bf16(int64_t n, const float *in, float *out)
{
    for (int64_t t = 0; t < n; ++t) out[t] = round_bf16(in[t]);
}

/* One element of the mixed-precision product: each operand element rounded
 * to bf16, the exact product of the two rounded values summed in double,
 * k in increasing order.  (A product of two bf16 values has at most 16
 * significant bits, so it is exact in double.) */
static double dot_bf16(int64_t K, const float *A, int64_t lda, int transA,
                       const float *B, int64_t ldb, int transB, int64_t i, int64_t j)
{
    double s = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        const float a = round_bf16((float)op_a(A, lda, transA, i, k));
        const float b = round_bf16((float)op_b(B, ldb, transB, k, j));
        s += (double)a * (double)b;
    }
    return s;
}

/*
 * Mixed-precision product: C[i][j] = sum_k bf16(opA(i,k)) * bf16(opB(k,j)),
 * in double, storage as gemm_ref_f64.  Returns 0, or -1 on bad arguments.
 */
int gemm_ref_f64_bf16(int64_t M, int64_t N, int64_t K,
                      const float *A, int64_t lda, const float *B, int64_t ldb,
                      double *C, int64_t ldc, int transA, int transB)
{
    if (!args_ok(M, N, K, lda, ldb, transA, transB) || ldc < N) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j)
            C[i * ldc + j] = dot_bf16(K, A, lda, transA, B, ldb, transB, i, j);
    return 0;
}

/* Selected entries of the mixed-precision product, as gemm_ref_f64_entries. */
int gemm_ref_f64_bf16_entries(int64_t M, int64_t N, int64_t K,
                              const float *A, int64_t lda, const float *B, int64_t ldb,
                              int transA, int transB, int64_t count,
                              const int64_t *rows, const int64_t *cols, double *out)
{
    if (!args_ok(M, N, K, lda, ldb, transA, transB) || count < 0) return -1;
    for (int64_t t = 0; t < count; ++t)
        if (rows[t] < 0 || rows[t] >= M || cols[t] < 0 || cols[t] >= N) return -2;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t t = 0; t < count; ++t)
        out[t] = dot_bf16(K, A, lda, transA, B, ldb, transB, rows[t], cols[t]);
    return 0;
}

/* Threads the OpenMP runtime will use for the loops above. */
int gemm_ref_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
