/* rows_f32.h -- row reductions of the library libgemm_f32.so: the causal
 * softmax of attention scores and its gradient, and the row normalisation
 * and its gradient, in FP32 on the GPU.
 *
 * These are the operations the Smallem page ("Rendre le GPU rapide") gives
 * their own kernels next to its matrix products (section "Les kernels
 * fusionnés") and then reduces with a whole warp per row (section "Un warp
 * par ligne"); here a whole 64-lane wave reduces each row.
 *
 * Common contract:
 *  - Matrices are row-major float32 device arrays with a leading dimension
 *    (ld >= the row length, >= 1); row r starts at ptr + r*ld.  Elements of
 *    the padding (columns >= the row length) are never read or written.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL is the
 *    default stream).  The library allocates, copies and synchronises
 *    nothing; the caller owns all memory.
 *  - An output may be one of the inputs (same pointer and leading
 *    dimension: in place); any other overlap is undefined.
 *  - Returns 0 on success; -i if argument i (1-based) is invalid, checked on
 *    the host before any HIP call; a positive hipError_t from the launch.
 *    rows == 0 or a row length of 0 writes nothing and returns 0.
 *  - Arithmetic is FP32; row sums and maxima are taken across the wave in a
 *    fixed tree order, so results are deterministic.
 */
#ifndef ROWS_F32_H
#define ROWS_F32_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Softmax of scaled scores along each row of x[rows x width]:
 *     y[r][c] = exp(scale*x[r][c] - m_r - log s_r)   for kept columns,
 *     y[r][c] = 0                                      otherwise,
 * m_r the maximum of scale*x over row r's kept columns and s_r the sum over
 * them of exp(scale*x - m_r) (computed as exp(scale*x - m_r) / s_r, the same
 * value, with one exponential per element).  causal = 1: rows come in groups of `queries`
 * consecutive query rows (one group per sequence and head) whose queries are
 * the last `queries` of `width` positions, so row r's query is at position
 * width - queries + r % queries and the kept columns are those at or before
 * it (the page's causal softmax, which computes the mask from the row
 * instead of reading one); x is never read beyond it.  causal = 0: every
 * column is kept and `queries` is ignored.
 * Errors: -1 rows, -2 width (negative or >= 2^31), -3 queries not in
 * [1, width] when causal, -4 causal not 0/1, -6 x NULL, -7 ldx, -8 y NULL,
 * -9 ldy. */
int rows_softmax_f32(int64_t rows, int64_t width, int64_t queries, int causal, float scale,
                     const float *x, int64_t ldx, float *y, int64_t ldy, void *stream);

/* Gradient of the softmax with respect to the unscaled scores x, from its
 * output y and the incoming gradient dy:
 *     dx[r][c] = scale * y[r][c] * (dy[r][c] - sum_c' dy[r][c'] * y[r][c']).
 * Columns a causal forward pass masked hold y = 0 and get dx = 0 (for finite
 * dy).  Errors: -1 rows, -2 width, -4 y NULL, -5 ldy, -6 dy NULL, -7 lddy,
 * -8 dx NULL, -9 lddx. */
int rows_softmax_backward_f32(int64_t rows, int64_t width, float scale,
                              const float *y, int64_t ldy, const float *dy, int64_t lddy,
                              float *dx, int64_t lddx, void *stream);

/* Row normalisation of x[rows x n]:
 *     y[r][c] = (x[r][c] - mu_r) / sqrt(var_r + eps),
 * mu_r the mean of row r and var_r the mean of its squared deviations from
 * mu_r; no scale or shift parameters.  Errors: -1 rows, -2 n, -3 eps
 * negative, infinite or NaN, -4 x NULL, -5 ldx, -6 y NULL, -7 ldy. */
int rows_normalize_f32(int64_t rows, int64_t n, float eps, const float *x, int64_t ldx,
                       float *y, int64_t ldy, void *stream);

/* Gradient of a loss through y = normalize(x), from x and dy = dL/dy:
 *     dx = (dy - mean(dy) - xhat * mean(dy * xhat)) / sigma   per row,
 * sigma = sqrt(var + eps) and xhat = (x - mu) / sigma recomputed from x.
 * Errors: -1 rows, -2 n, -3 eps, -4 x NULL, -5 ldx, -6 dy NULL, -7 lddy,
 * -8 dx NULL, -9 lddx. */
int rows_normalize_backward_f32(int64_t rows, int64_t n, float eps,
                                const float *x, int64_t ldx, const float *dy, int64_t lddy,
                                float *dx, int64_t lddx, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* ROWS_F32_H */
