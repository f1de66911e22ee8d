// gemm_internal.hpp -- declarations shared by the host API and the kernel
// translation units of the FP32 GEMM library.  Not installed; the public
// interface is include/gemm_f32.h.
#pragma once

#include <hip/hip_runtime.h>

#include "gemm_f32.h"

#include <cstdint>

namespace gemmf32 {

// A validated problem.  Dimensions fit in 31 bits (the API rejects larger);
// leading dimensions are kept 64-bit so row offsets never overflow.
struct Problem {
    int M, N, K;
    const float *A;
    int64_t lda;
    const float *B;
    int64_t ldb;
    float *C;
    int64_t ldc;
    int transA, transB;
    // Strided batch: product b reads A + b*stride_a, B + b*stride_b and
    // writes C + b*stride_c, for b < batch (a single product: batch 1).
    int64_t stride_a = 0, stride_b = 0, stride_c = 0;
    int64_t batch = 1;
    // Fused epilogue: C = act(product + bias[j]); bias may be null.
    const float *bias = nullptr;
    int act = 0;  // 0: none, 1: GELU (erf form)
    // Split k (MFMA path): when k_total > 0, product b is the partial product
    // over k in [b*K, min(k_total, (b+1)*K)); the strides move A and B along
    // k.  0: every product spans K.
    int k_total = 0;
};

// Each launcher enqueues its kernel(s) on `stream` and returns
// hipGetLastError() after the launch.  All assume M, N, K >= 1.
hipError_t launch_naive(const Problem &p, hipStream_t stream);
hipError_t launch_tiled(const Problem &p, hipStream_t stream);
hipError_t launch_fma(const Problem &p, hipStream_t stream);
// tile: 0 chooses by problem size (the 256 x 256 kernel when it is preferred);
// 256 (256 x 128), 128 or 64 forces that tile.
hipError_t launch_mfma(const Problem &p, hipStream_t stream, int tile);
// The configuration launch_mfma runs for p and tile: a gemm_f32_plan_code
// (one of the GEMM_F32_PLAN_MFMA_* values).  Host only; launches nothing.
int plan_mfma(const Problem &p, int tile);
// The 256 x 256 MFMA kernel with one running sum per output
// (gemm_mfma_wide.hip).  fits: the problem is in its domain (any
// transposes, M and N multiples of 256, K a multiple of 32 and at most
// 1024, 16-byte aligned operands and strides, no split k).  preferred: it
// fits and has at least one tile per CU; launch_mfma with tile 0 then takes
// it.  The launcher assumes fits.
bool mfma_wide_fits(const Problem &p);
bool mfma_wide_preferred(const Problem &p);
hipError_t launch_mfma_wide(const Problem &p, hipStream_t stream);
// tile: 0 chooses by problem size; 256 (256 x 256) or 128 forces that tile.
// Operands rounded to bf16 (nearest, ties to even), bf16 matrix-core
// products, FP32 sums and output.  Ignores batch, bias and act.
hipError_t launch_bf16(const Problem &p, hipStream_t stream, int tile = 0);
// A product of two packed bf16 operands (bit patterns): A is M x K and B is
// N x K, both with k along their rows; C = A . B^T in FP32.
struct PackedProblem {
    int M, N, K;
    const uint16_t *A;
    int64_t lda;
    const uint16_t *B;
    int64_t ldb;
    float *C;
    int64_t ldc;
};
// tile: 0 chooses by problem size; a tile area (65536 for 256 x 256, 32768
// for 256 x 128, 16384 for 128 x 128) forces that tile (the first two fall
// back to 128 x 128 beyond K = 16384).  Assumes M, N, K >= 1.
hipError_t launch_bf16_packed(const PackedProblem &p, hipStream_t stream, int tile = 0);
// dst[r * ldd + c] = bf16 bits of op(src)[r][c] (nearest, ties to even) for
// r < rows, c < cols; op(src) = src (stored rows x cols) or, with trans,
// src^T (stored cols x rows).  Assumes rows, cols >= 1.
hipError_t launch_pack_bf16(int rows, int cols, const float *src, int64_t lds, int trans, uint16_t *dst,
                            int64_t ldd, hipStream_t stream);
// C[i][j] = sum over s < splits, in increasing s, of ws[s*M*N + i*N + j]:
// the fixed-order sum of split-k partial products (packed M x N each).
hipError_t launch_splitk_reduce(const float *ws, int splits, int M, int N, float *C, int64_t ldc,
                                hipStream_t stream);
// C := act(0 + bias[j]) over M x N (the empty sum, K == 0), for every
// product of the batch.  Assumes M, N >= 1.
hipError_t launch_zero_fill(const Problem &p, hipStream_t stream);

// GELU in its exact form x * Phi(x) = x/2 * (1 + erf(x / sqrt 2)), Phi the
// standard normal distribution function.
__device__ __forceinline__ float gelu(float x)
{
    return 0.5f * x * (1.0f + erff(x * 0.70710678118654752440f));
}

// Number of 32-bit words per 16-byte vector.
constexpr int kVec = 4;

__host__ __device__ constexpr int ceil_div(int a, int b) { return (a + b - 1) / b; }

// True if every float4 this operand's vector loads touch is 16-byte aligned:
// the base pointer is 16-byte aligned and the leading dimension is a
// multiple of four floats.
inline bool vec4_ok(const float *ptr, int64_t ld)
{
    return (reinterpret_cast<uintptr_t>(ptr) % 16 == 0) && (ld % kVec == 0);
}

}  // namespace gemmf32
