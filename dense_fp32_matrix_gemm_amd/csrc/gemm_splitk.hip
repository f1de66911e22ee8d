// gemm_splitk.hip -- the reduction step of a split-k product: C is the sum,
// in a fixed order, of the partial products of consecutive runs of k.
//
// The Smallem page ("Rendre le GPU rapide", section "Ce qui n'a pas
// marche") computes the weight gradient as one product per sequence
// followed by a sum, which ran faster than one product over all tokens; a
// split over k is that decomposition: product s covers its own run of k,
// and the partial M x N results are added.  Here the partials are written
// packed (leading dimension N) into a caller-provided workspace by the MFMA
// kernel, and this kernel adds them in increasing s into C, so the result
// does not depend on scheduling.
//
// The work is element-wise and bound by memory traffic ((splits + 1) * 4
// bytes per output): each lane handles four consecutive columns of one row,
// read as 16-byte vectors when the row allows it, and consecutive lanes
// take consecutive column groups so every wave reads whole row segments.
#include "tile_common.hpp"

namespace gemmf32 {
namespace {

constexpr int kReduceThreads = 256;

template <bool VEC>
__global__ __launch_bounds__(kReduceThreads) void splitk_reduce_kernel(
    const float *__restrict__ ws, int splits, int M, int N, float *__restrict__ C, int64_t ldc)
{
    const int groups = (N + 3) / 4;  // four-column groups per row
    const int64_t total = int64_t(M) * groups;
    const int64_t slice = int64_t(M) * N;
    for (int64_t g = int64_t(blockIdx.x) * kReduceThreads + threadIdx.x; g < total;
         g += int64_t(gridDim.x) * kReduceThreads) {
        const int i = int(g / groups);
        const int j = 4 * int(g % groups);
        const float *src = ws + int64_t(i) * N + j;
        float *dst = C + int64_t(i) * ldc + j;
        if (VEC && j + 3 < N) {
            v4f acc = *reinterpret_cast<const v4f *>(src);
            for (int s = 1; s < splits; ++s) {
                const v4f x = *reinterpret_cast<const v4f *>(src + s * slice);
                acc[0] += x[0];
                acc[1] += x[1];
                acc[2] += x[2];
                acc[3] += x[3];
            }
            *reinterpret_cast<v4f *>(dst) = acc;
        } else {
            const int w = N - j < 4 ? N - j : 4;
            for (int e = 0; e < w; ++e) {
                float acc = src[e];
                for (int s = 1; s < splits; ++s) acc += src[s * slice + e];
                dst[e] = acc;
            }
        }
    }
}

}  // namespace

hipError_t launch_splitk_reduce(const float *ws, int splits, int M, int N, float *C, int64_t ldc,
                                hipStream_t stream)
{
    const int64_t groups = int64_t(M) * ((N + 3) / 4);
    // Enough workgroups to fill the chip several times over; the loop
    // strides over whatever remains.
    const int64_t want = (groups + kReduceThreads - 1) / kReduceThreads;
    const unsigned grid = unsigned(want < 8192 ? want : 8192);
    const bool vec = N % 4 == 0 && vec4_ok(ws, N) && vec4_ok(C, ldc);
    if (vec)
        splitk_reduce_kernel<true><<<grid, kReduceThreads, 0, stream>>>(ws, splits, M, N, C, ldc);
    else
        splitk_reduce_kernel<false><<<grid, kReduceThreads, 0, stream>>>(ws, splits, M, N, C, ldc);
    return hipGetLastError();
}

}  // namespace gemmf32
