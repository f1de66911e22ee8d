// gemm_simple.hip -- the two reference-shaped kernels of the library and
// the K == 0 fill:
//
//  * naive: one lane per element of C, operands straight from global memory
//    (course page "3 . La memoire partagee", section 3.1).
//  * tiled: T x T tiles of A and B staged through LDS, one output per thread,
//    load / barrier / compute / barrier / next (same page, sections 3.2-3.3),
//    with zero-filled edge tiles so any M, N, K works.
//
// Both accumulate in FP32.  The k loop sums short runs of k into a fresh
// partial and adds each partial into the running total: with plain
// sequential accumulation the rounding error of an FP32 dot product grows
// like sqrt(K) and exceeds a 1e-6 relative Frobenius error near K = 3300 for
// uniform inputs; summing runs of 32 first keeps it near 2e-7 at K = 4096.
#include "gemm_internal.hpp"

namespace gemmf32 {
namespace {

constexpr int kChunk = 32;  // k values summed into one partial before it is folded in

template <int TRANS>
__device__ __forceinline__ float load_a(const float *__restrict__ A, int64_t lda, int i, int k)
{
    return TRANS ? A[int64_t(k) * lda + i] : A[int64_t(i) * lda + k];
}

template <int TRANS>
__device__ __forceinline__ float load_b(const float *__restrict__ B, int64_t ldb, int k, int j)
{
    return TRANS ? B[int64_t(j) * ldb + k] : B[int64_t(k) * ldb + j];
}

// ---------------------------------------------------------------- naive ----
// Block = 64 x 4 lanes: each wave is one row segment of 64 consecutive
// columns, so a wave's loads of B (transB == 0) are one contiguous 256-byte
// run and its element of A is the same address for all lanes (wave-uniform;
// readfirstlane lets the compiler fetch it with a scalar load).  Rows are
// walked with a grid stride so any M fits in the 65535-block y limit.
constexpr int kNaiveX = 64, kNaiveY = 4;

template <int TA, int TB>
__global__ __launch_bounds__(kNaiveX *kNaiveY) void naive_kernel(
    int M, int N, int K, const float *__restrict__ A, int64_t lda,
    const float *__restrict__ B, int64_t ldb, float *__restrict__ C, int64_t ldc)
{
    const int j = blockIdx.x * kNaiveX + threadIdx.x;
    const int row0 = __builtin_amdgcn_readfirstlane(blockIdx.y * kNaiveY + threadIdx.y);
    const int row_step = gridDim.y * kNaiveY;
    if (j >= N) return;  // no barrier in this kernel: idle lanes may leave
    for (int i = row0; i < M; i += row_step) {
        float acc = 0.0f;
        for (int k0 = 0; k0 < K; k0 += kChunk) {
            const int kend = min(K, k0 + kChunk);
            float part = 0.0f;
            for (int k = k0; k < kend; ++k)
                part = __builtin_fmaf(load_a<TA>(A, lda, i, k), load_b<TB>(B, ldb, k, j), part);
            acc += part;
        }
        C[int64_t(i) * ldc + j] = acc;
    }
}

// ---------------------------------------------------------------- tiled ----
// T x T threads per block, one output each.  The LDS rows are padded to
// T + 1 floats: with a transposed operand the cooperative load writes a tile
// column per wave, and without padding those writes all land in one bank
// (section 3.6 of the course page).  Tiles walk a 1-D grid with a stride so
// any number of tiles fits the launch limits; every thread of a block walks
// the same tiles, so the barriers are never inside divergent code.
template <int T, int TA, int TB>
__global__ __launch_bounds__(T *T) void tiled_kernel(
    int M, int N, int K, const float *__restrict__ A, int64_t lda,
    const float *__restrict__ B, int64_t ldb, float *__restrict__ C, int64_t ldc)
{
    __shared__ float As[T][T + 1];  // As[r][c] = opA(i0 + r, k0 + c)
    __shared__ float Bs[T][T + 1];  // Bs[r][c] = opB(k0 + r, j0 + c)
    const int tx = threadIdx.x, ty = threadIdx.y;
    const int tiles_n = ceil_div(N, T);
    const int tiles = ceil_div(M, T) * tiles_n;
    for (int tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
        const int i0 = (tile / tiles_n) * T, j0 = (tile % tiles_n) * T;
        float acc = 0.0f;
        for (int k0 = 0; k0 < K; k0 += T) {
            // 1. cooperative, coalesced load: consecutive tx read consecutive
            //    addresses; elements outside the matrices are zero.
            if (!TA) {
                const int i = i0 + ty, k = k0 + tx;
                As[ty][tx] = (i < M && k < K) ? load_a<0>(A, lda, i, k) : 0.0f;
            } else {
                const int k = k0 + ty, i = i0 + tx;
                As[tx][ty] = (i < M && k < K) ? load_a<1>(A, lda, i, k) : 0.0f;
            }
            if (!TB) {
                const int k = k0 + ty, j = j0 + tx;
                Bs[ty][tx] = (k < K && j < N) ? load_b<0>(B, ldb, k, j) : 0.0f;
            } else {
                const int j = j0 + ty, k = k0 + tx;
                Bs[tx][ty] = (k < K && j < N) ? load_b<1>(B, ldb, k, j) : 0.0f;
            }
            __syncthreads();  // 2. the tile is complete before anyone reads it
            float part = 0.0f;  // 3. T-term partial from LDS (one chunk)
#pragma unroll
            for (int k = 0; k < T; ++k) part = __builtin_fmaf(As[ty][k], Bs[k][tx], part);
            acc += part;
            __syncthreads();  // 4. everyone has read it before it is overwritten
        }
        const int i = i0 + ty, j = j0 + tx;
        if (i < M && j < N) C[int64_t(i) * ldc + j] = acc;
    }
}

// ------------------------------------------------------------ zero fill ----
// C := act(0 + bias[j]) over M x N of product batch_base + blockIdx.y
// (without bias and activation: zero).
__global__ __launch_bounds__(256) void zero_fill_kernel(int M, int N, float *__restrict__ C,
                                                        int64_t ldc, int64_t stride_c,
                                                        int64_t batch_base,
                                                        const float *__restrict__ bias, int act)
{
    C += (batch_base + blockIdx.y) * stride_c;
    const int64_t total = int64_t(M) * N;
    for (int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x; e < total;
         e += int64_t(gridDim.x) * 256) {
        const int64_t j = e % N;
        float x = bias != nullptr ? bias[j] : 0.0f;
        if (act == 1) x = gelu(x);
        C[(e / N) * ldc + j] = x;
    }
}

constexpr int kMaxGridX = 1 << 20;  // block cap for grid-stride kernels
constexpr int kMaxGridY = 65535;   // grid y cap (batched fill)

template <int TA, int TB>
void naive_dispatch(const Problem &p, hipStream_t s)
{
    const dim3 block(kNaiveX, kNaiveY);
    const dim3 grid(ceil_div(p.N, kNaiveX), min(ceil_div(p.M, kNaiveY), 65535));
    naive_kernel<TA, TB><<<grid, block, 0, s>>>(p.M, p.N, p.K, p.A, p.lda, p.B, p.ldb, p.C, p.ldc);
}

template <int T, int TA, int TB>
void tiled_dispatch(const Problem &p, hipStream_t s)
{
    const int64_t tiles = int64_t(ceil_div(p.M, T)) * ceil_div(p.N, T);
    const dim3 grid(unsigned(tiles < kMaxGridX ? tiles : kMaxGridX));
    tiled_kernel<T, TA, TB><<<grid, dim3(T, T), 0, s>>>(p.M, p.N, p.K, p.A, p.lda, p.B, p.ldb,
                                                         p.C, p.ldc);
}

}  // namespace

hipError_t launch_naive(const Problem &p, hipStream_t s)
{
    if (p.transA) {
        if (p.transB) naive_dispatch<1, 1>(p, s); else naive_dispatch<1, 0>(p, s);
    } else {
        if (p.transB) naive_dispatch<0, 1>(p, s); else naive_dispatch<0, 0>(p, s);
    }
    return hipGetLastError();
}

hipError_t launch_tiled(const Problem &p, hipStream_t s)
{
    constexpr int T = 32;  // the course page's tile; 1024 threads = 16 waves
    if (p.transA) {
        if (p.transB) tiled_dispatch<T, 1, 1>(p, s); else tiled_dispatch<T, 1, 0>(p, s);
    } else {
        if (p.transB) tiled_dispatch<T, 0, 1>(p, s); else tiled_dispatch<T, 0, 0>(p, s);
    }
    return hipGetLastError();
}

hipError_t launch_zero_fill(const Problem &p, hipStream_t s)
{
    const int64_t blocks = (int64_t(p.M) * p.N + 255) / 256;
    const unsigned gx = unsigned(blocks < kMaxGridX ? blocks : kMaxGridX);
    for (int64_t b0 = 0; b0 < p.batch; b0 += kMaxGridY) {
        const int64_t nb = p.batch - b0 < kMaxGridY ? p.batch - b0 : kMaxGridY;
        zero_fill_kernel<<<dim3(gx, unsigned(nb)), dim3(256), 0, s>>>(p.M, p.N, p.C, p.ldc,
                                                                       p.stride_c, b0, p.bias,
                                                                       p.act);
    }
    return hipGetLastError();
}

}  // namespace gemmf32
