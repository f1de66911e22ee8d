/*
 * gemm_f32.h -- FP32 dense matrix multiply for AMD Instinct MI355X (gfx950).
 *
 *     C[M x N] = op(A)[M x K] . op(B)[K x N]          (FP32 in, FP32 out)
 *
 * The operation is the matrix product the course page "3 . La memoire
 * partagee" builds up to in sections 3.1-3.4 (naive kernel, tiled kernel,
 * register tiles), taken rectangular and row-major as in the cuda-oxide
 * book's tiled_sgemm (page "shared memory and synchronisation"), with
 * leading dimensions and optional transposes added so that the backward
 * products of a training step need no transpose copies (the Smallem page,
 * "Rendre le GPU rapide", section on the comparison with PyTorch, names
 * transpose copies as a cost).
 *
 * Storage (all row-major, element (r, c) of a stored matrix at ptr[r*ld + c]):
 *   transA == 0: A is stored M x K, element opA(i,k) = A[i*lda + k], lda >= max(1,K)
 *   transA == 1: A is stored K x M, element opA(i,k) = A[k*lda + i], lda >= max(1,M)
 *   transB == 0: B is stored K x N, element opB(k,j) = B[k*ldb + j], ldb >= max(1,N)
 *   transB == 1: B is stored N x K, element opB(k,j) = B[j*ldb + k], ldb >= max(1,K)
 *   C is stored M x N, C[i*ldc + j], ldc >= max(1,N).  C is overwritten
 *   (there is no alpha/beta); elements of the padding (columns N..ldc-1) are
 *   never written, and elements of A/B outside the used region are never
 *   folded into the result (their values, NaN included, do not matter).
 *
 * Pointers and ownership: A, B and C are DEVICE pointers owned by the caller.
 * The library allocates, frees and copies nothing, keeps no state between
 * calls (gemm_f32_splitk_noalloc's per-GPU scratch array aside) and never
 * synchronises: each call enqueues its kernels on `stream`
 * (a hipStream_t passed as void*; NULL means the default stream) and
 * returns; C is complete when the stream reaches that point.  C must not
 * overlap A or B.  Concurrent calls on different streams are safe.
 *
 * Arithmetic: products and sums in FP32 (IEEE round-to-nearest-even,
 * fused multiply-add allowed).  The summation order over k is not the
 * plain sequential one: partial sums over short runs of k are formed first
 * and then added together, which bounds the rounding error growth for long
 * K.  Any order is a correct evaluation of the product; results agree with
 * an exact product to within 1e-6*K + 1e-5*|C| elementwise for inputs of
 * magnitude <= 1.
 *
 * Return value (all entry points):
 *     0   success (also for the quick returns below)
 *    -i   the i-th argument (1-based, in the order of the prototype) is
 *         invalid: M/N/K < 0 (-1/-2/-3); A NULL while M*K > 0 (-4); lda too
 *         small (-5); B NULL while K*N > 0 (-6); ldb too small (-7); C NULL
 *         while M*N > 0 (-8); ldc too small (-9); transA/transB not 0 or 1
 *         (-10/-11); algo unknown, or GEMM_F32_ALGO_MFMA_WIDE for a
 *         problem outside its domain (-13, gemm_f32_ex only); a dimension
 *         or leading dimension >= 2^31 is reported as invalid for that
 *         argument.  Validation is done on the host before any HIP call,
 *         so these codes are returned even on a machine without a GPU.
 *    >0   a hipError_t reported by the kernel launch (hipGetLastError()
 *         is checked after every launch).
 * Quick returns: M == 0 or N == 0 enqueues nothing; K == 0 writes C = 0
 * (the empty sum) over the M x N region.
 */
#ifndef GEMM_F32_H
#define GEMM_F32_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Kernel families selectable through gemm_f32_ex. */
enum gemm_f32_algo {
    GEMM_F32_ALGO_AUTO = 0,  /* the fastest path for the shape: currently MFMA */
    GEMM_F32_ALGO_MFMA = 1,  /* LDS-staged tiles, FP32 matrix-core MFMA micro-tiles;
                                the tile size is chosen from the problem size */
    GEMM_F32_ALGO_FMA = 2,   /* LDS-staged tiles, register-blocked vector FMA */
    GEMM_F32_ALGO_TILED = 3, /* T x T LDS tiles, one output per thread (section 3.3) */
    GEMM_F32_ALGO_NAIVE = 4, /* one lane per output, operands from global memory (3.1) */
    GEMM_F32_ALGO_MFMA_TILE128 = 5, /* MFMA with the 128 x 128 tile forced */
    GEMM_F32_ALGO_MFMA_TILE64 = 6,  /* MFMA with the 64 x 64 (split-k-group) tile forced */
    GEMM_F32_ALGO_MFMA_TILE256 = 7, /* MFMA with the 256 x 128 tile forced */
    GEMM_F32_ALGO_MFMA_WIDE = 8     /* MFMA with the 256 x 256 tile and one running
                                       FP32 sum per output (relative error about
                                       2^-24 * sqrt(K / 12) on zero-mean data, so
                                       K <= 1024 keeps it below 1e-6).  Only for
                                       M and N multiples of 256, K a multiple of 32
                                       and at most 1024, A and B 16-byte aligned with
                                       lda and ldb multiples of 4 (either transpose);
                                       any other non-empty problem returns -13.
                                       AUTO takes it for such problems with at least
                                       256 tiles. */
};

/* Kernel configurations of the automatic choice, as reported by
 * gemm_f32_plan. */
enum gemm_f32_plan_code {
    GEMM_F32_PLAN_NOTHING = 0,   /* M or N is 0: nothing is written */
    GEMM_F32_PLAN_ZERO_FILL = 1, /* K is 0: C is set to 0 */
    GEMM_F32_PLAN_MFMA_256X256 = 2, /* 256 x 256 tile, one running sum per output */
    GEMM_F32_PLAN_MFMA_256X128 = 3, /* 256 x 128 tile */
    GEMM_F32_PLAN_MFMA_128X128 = 4, /* 128 x 128 tile, two workgroups per CU */
    GEMM_F32_PLAN_MFMA_128X128_ONE_ROUND = 5, /* 128 x 128, at most one tile per CU */
    GEMM_F32_PLAN_MFMA_128X128_KK = 6, /* 128 x 128, both operands k-contiguous */
    GEMM_F32_PLAN_MFMA_128X64 = 7,  /* outputs at most 64 columns wide */
    GEMM_F32_PLAN_MFMA_64X64 = 8,   /* small grids: two k-slices of waves */
    GEMM_F32_PLAN_MFMA_64X64_PAIR = 9 /* 64 x 64, larger grids: 64-k stages, two workgroups per CU */
};

/* C = op(A) . op(B) on the fastest path (GEMM_F32_ALGO_AUTO). */
int gemm_f32(int64_t M, int64_t N, int64_t K,
             const float *A, int64_t lda,
             const float *B, int64_t ldb,
             float *C, int64_t ldc,
             int transA, int transB, void *stream);

/* The naive baseline of section 3.1 of the course page: one lane per
 * element of C, each lane reading its row of op(A) and column of op(B)
 * straight from global memory.  Same contract as gemm_f32. */
int gemm_f32_naive(int64_t M, int64_t N, int64_t K,
                   const float *A, int64_t lda,
                   const float *B, int64_t ldb,
                   float *C, int64_t ldc,
                   int transA, int transB, void *stream);

/* gemm_f32 with an explicit kernel family (enum gemm_f32_algo). */
int gemm_f32_ex(int64_t M, int64_t N, int64_t K,
                const float *A, int64_t lda,
                const float *B, int64_t ldb,
                float *C, int64_t ldc,
                int transA, int transB, void *stream, int algo);

/* Strided-batched product: for b = 0 .. batch-1,
 *     C + b*strideC  =  op(A + b*strideA) . op(B + b*strideB)
 * with every product as in gemm_f32 (same storage, ld and transpose rules).
 * This is the attention-score product of the Smallem page ("Rendre le GPU
 * rapide", section on the generation cache: queries [B,H,N,D] times
 * transposed keys [B,H,D,T], one product per batch and head).  Strides are
 * in floats; strideA or strideB 0 shares one operand across the batch;
 * products must not overlap in C (strideC >= (M-1)*ldc + N when batch > 1).
 * Return codes as for gemm_f32, with -i numbering THIS prototype's
 * arguments: -6/-9/-12 a negative or overlapping stride, -13 batch < 0 or
 * >= 2^31.  batch == 0 returns 0 and writes nothing.  Runs on the MFMA path. */
int gemm_f32_strided_batched(int64_t M, int64_t N, int64_t K,
                             const float *A, int64_t lda, int64_t strideA,
                             const float *B, int64_t ldb, int64_t strideB,
                             float *C, int64_t ldc, int64_t strideC, int64_t batch,
                             int transA, int transB, void *stream);

/* Epilogues of gemm_f32_bias_act. */
enum gemm_f32_act {
    GEMM_F32_ACT_NONE = 0,
    GEMM_F32_ACT_GELU = 1  /* x * Phi(x) = x/2 * (1 + erf(x / sqrt 2)) */
};

/* Fused linear layer: C = act(op(A) . op(B) + bias), the bias added to every
 * row (bias[j] for column j; bias may be NULL for none), the activation
 * applied elementwise in FP32 before C is written.  The Smallem page
 * ("Rendre le GPU rapide", sections on fused kernels and on the comparison
 * with PyTorch) gives GELU its own kernel and names the unfused bias add as
 * a cost; here both ride in the product's store.  bias, if not NULL, is a
 * device array of N floats.  Storage, ownership and the other codes as for
 * gemm_f32; -13: act not a gemm_f32_act value.  K == 0 writes act(bias).
 * Runs on the MFMA path. */
int gemm_f32_bias_act(int64_t M, int64_t N, int64_t K,
                      const float *A, int64_t lda,
                      const float *B, int64_t ldb,
                      float *C, int64_t ldc,
                      int transA, int transB,
                      const float *bias, int act, void *stream);

/* Mixed precision: C = op(A) . op(B) with each operand element rounded to
 * bf16 (8 significant bits, the exponent range of FP32; round to nearest,
 * ties to even) before it is multiplied, the products added in FP32 and C
 * written in FP32.  A, B and C are FP32 arrays as for gemm_f32; the rounding
 * happens on the way into the kernel, and neither operand is modified.
 * This is the Smallem page's mixed precision ("Rendre le GPU rapide",
 * section "Les Tensor Cores"): only the operands of the multiplication are
 * rounded to 16 bits; sums and tensors stay FP32.  Results agree with the
 * exact product of the rounded operands to within 1e-6*K + 1e-5*|C|
 * elementwise for operands of magnitude <= 1, and equal it exactly when
 * every rounded operand is an integer and every partial sum of the integer
 * products has magnitude below 2^24 (for instance integers in [-8, 8] with
 * K <= 2^18).  Storage, ownership, quick returns and status codes as for
 * gemm_f32.  Runs on the bf16 matrix cores (v_mfma_f32_32x32x16_bf16). */
int gemm_f32_bf16(int64_t M, int64_t N, int64_t K,
                  const float *A, int64_t lda,
                  const float *B, int64_t ldb,
                  float *C, int64_t ldc,
                  int transA, int transB, void *stream);

/* Mixed precision in two steps, rounding each operand once: pack it with
 * gemm_f32_pack_bf16, then multiply packed operands with
 * gemm_f32_bf16_packed.  Same arithmetic as gemm_f32_bf16 (the Smallem
 * page, "Rendre le GPU rapide", section "Les Tensor Cores": operands rounded
 * to bf16, sums and C in FP32); the same page's comparison with PyTorch
 * notes that keeping the 16-bit copies, as PyTorch does, saves converting on
 * every read.  A packed operand is a row-major array of bf16 bit patterns
 * (uint16_t: the upper half of the FP32 encoding) with k along its rows. */

/* dst[r*ldd + c] = bf16(op(src)[r][c]) for r < rows, c < cols, rounded to
 * nearest with ties to even; columns c >= cols of dst are not written.
 * op(src) = src, stored rows x cols (lds >= max(1, cols)), when trans == 0;
 * src^T, with src stored cols x rows (lds >= max(1, rows)), when trans == 1.
 * To pack A of gemm_f32 for gemm_f32_bf16_packed: rows = M, cols = K,
 * trans = transA.  To pack B (K x N): rows = N, cols = K, trans = !transB.
 * src (FP32) and dst are device arrays the caller owns; they must not
 * overlap.  ldd >= max(1, cols); an ldd that is a multiple of 8 with a
 * 16-byte aligned dst lets the product copy whole 16-byte vectors.
 * Returns 0, or -1 rows / -2 cols negative or >= 2^31, -3 src NULL with
 * rows*cols > 0, -4 lds too small or >= 2^31, -5 trans not 0 or 1, -6 dst
 * NULL with rows*cols > 0, -7 ldd < max(1, cols) or >= 2^31 (checked on the
 * host before any HIP call), or a positive hipError_t from the launch.
 * rows == 0 or cols == 0 writes nothing.  Asynchronous on `stream`. */
int gemm_f32_pack_bf16(int64_t rows, int64_t cols, const float *src, int64_t lds, int trans,
                       uint16_t *dst, int64_t ldd, void *stream);

/* C = A . B^T with A (M x K, lda >= max(1, K)) and B (N x K, ldb >= max(1,
 * K)) packed bf16 operands, the products summed in FP32 and C (M x N, ldc >=
 * max(1, N)) written in FP32, overwritten.  C[i][j] = sum over k of
 * A[i][k] * B[j][k].  Results agree with the exact sum of the products to
 * within 1e-6*K + 1e-5*|C| elementwise for operands of magnitude <= 1, and
 * equal it exactly under the conditions given for gemm_f32_bf16.  Device
 * arrays the caller owns; C must not overlap A or B.  Codes -1 .. -9 as for
 * gemm_f32's first nine arguments (the stored rows of A and B hold K
 * elements); M == 0 or N == 0 writes nothing; K == 0 writes zeros.  Interior
 * tiles copy whole 16-byte vectors straight into LDS when A and B are
 * 16-byte aligned and lda, ldb are multiples of 8; otherwise every tile is
 * staged through registers (same results, slower).  Runs on the bf16 matrix
 * cores (v_mfma_f32_32x32x16_bf16). */
int gemm_f32_bf16_packed(int64_t M, int64_t N, int64_t K,
                         const uint16_t *A, int64_t lda,
                         const uint16_t *B, int64_t ldb,
                         float *C, int64_t ldc, void *stream);

/* Split-k product: C = op(A) . op(B) as in gemm_f32, computed as `splits`
 * partial products over consecutive runs of k followed by their sum.  The
 * Smallem page ("Rendre le GPU rapide", section "Ce qui n'a pas marche")
 * computes the weight gradient as one product per sequence plus a sum,
 * which ran faster than a single product over all tokens; this is that
 * decomposition along k for any product.
 *
 * The runs are len = ceil(K / splits) rounded up to a multiple of 32, so
 * s_used = ceil(K / len) <= splits partial products are formed (the last
 * one shorter).  Partial s (packed M x N, leading dimension N) is written to
 * workspace + s*M*N; C is then their sum in increasing s, so the result does
 * not depend on scheduling.  workspace is a device array the caller owns,
 * of at least gemm_f32_splitk_workspace_size(M, N, K, splits) bytes; its
 * contents on return are unspecified and it must not overlap A, B or C.  It
 * may be NULL when that size is 0 (s_used == 1, K == 0, M == 0 or N == 0),
 * which runs as gemm_f32.  Storage, ownership, quick returns and the codes
 * of arguments 1-12 as for gemm_f32 (argument 12 is splits here; the stream
 * is argument 15); -12: splits < 1 or >= 2^31, or s_used*M*N*4 bytes beyond
 * 2^62; -13: workspace NULL where one is needed; -14: workspace_bytes
 * smaller than needed.  Runs on the MFMA path. */
int gemm_f32_splitk(int64_t M, int64_t N, int64_t K,
                    const float *A, int64_t lda,
                    const float *B, int64_t ldb,
                    float *C, int64_t ldc,
                    int transA, int transB, int64_t splits,
                    float *workspace, int64_t workspace_bytes, void *stream);

/* The largest partial products, in bytes (s_used*M*N*4), that
 * gemm_f32_splitk_noalloc holds: 64 MiB of device memory per GPU. */
#define GEMM_F32_SPLITK_SCRATCH_BYTES (64LL << 20)

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc:
 * gemm_f32_splitk without a workspace argument.  The partial products go to
 * a scratch array of GEMM_F32_SPLITK_SCRATCH_BYTES that the library keeps in
 * each GPU's memory (reserved when the library's code is first loaded on
 * that GPU and held until the process ends); the call itself allocates and
 * frees nothing.  Same arithmetic, results and codes as gemm_f32_splitk with
 * the same splits (bit for bit), arguments 1-12 numbered as there and the
 * stream as argument 13; -12 also when s_used*M*N*4 exceeds
 * GEMM_F32_SPLITK_SCRATCH_BYTES (fewer splits fit; splits = 1 always does).
 * Every call on one GPU shares that GPU's scratch array: calls that overlap
 * in time on the same GPU (on different streams, or from different host
 * threads without stream ordering) race and give wrong results; calls
 * ordered on one stream are safe.  Nothing needs clearing between calls
 * (each partial is written whole before it is summed).  The stream's GPU
 * must be the one that owns C; its scratch address is looked up on its
 * first call (a positive hipError_t if that fails). */
int gemm_f32_splitk_noalloc(int64_t M, int64_t N, int64_t K,
                            const float *A, int64_t lda,
                            const float *B, int64_t ldb,
                            float *C, int64_t ldc,
                            int transA, int transB, int64_t splits, void *stream);

/* Bytes of workspace gemm_f32_splitk needs for these sizes: s_used*M*N*4,
 * or 0 when it runs as a single product.  Negative (-1, -2, -3, -12) for an
 * invalid M, N, K or splits, numbered as in gemm_f32_splitk. */
int64_t gemm_f32_splitk_workspace_size(int64_t M, int64_t N, int64_t K, int64_t splits);

/* A static, human-readable description of a return value (never NULL).
 * Messages for -1 .. -11 name gemm_f32's arguments; -12 .. -14 list what the
 * position means for each entry point that uses it. */
const char *gemm_f32_strerror(int status);

/* The kernel configuration that gemm_f32 would run for these arguments
 * (and gemm_f32_strided_batched, or gemm_f32_bias_act, for the same
 * shapes), decided on the host exactly as a call decides it: a
 * gemm_f32_plan_code.  Nothing is launched and the pointers are never
 * dereferenced, but their alignment counts (the 256 x 256 tile needs
 * 16-byte aligned operands and strides).  batch = 1 for a single product.
 * Returns -i for an invalid argument, numbered in this prototype's order:
 * -1/-2/-3 a dimension, -5/-7/-8 a leading dimension, -9/-10 a transpose
 * flag, -11/-12 a negative stride, -13 batch < 1 or >= 2^31. */
int gemm_f32_plan(int64_t M, int64_t N, int64_t K,
                  const float *A, int64_t lda,
                  const float *B, int64_t ldb, int64_t ldc,
                  int transA, int transB,
                  int64_t strideA, int64_t strideB, int64_t batch);

/* Library interface version: major * 10000 + minor * 100 + patch. */
int gemm_f32_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_F32_H */
