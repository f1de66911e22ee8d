// rows.hip -- row reductions for the operations around the GEMM in a
// transformer step: the causal softmax of attention scores and its
// gradient, and the row normalisation and its gradient.  Contract:
// include/rows_f32.h.
//
// The Smallem page ("Rendre le GPU rapide") gives these their own kernels
// (section "Les kernels fusionnés": the causal softmax decides the mask from
// the row's query position instead of reading a mask) and then reduces each
// row with a whole warp instead of one thread (section "Un warp par ligne"):
// lane l reads elements l, l + 32, ..., so every load instruction reads
// neighbouring elements, and the partial results are combined by exchanging
// registers across the warp (xor distances 16, 8, ..., 1).  On gfx950 the
// unit is a 64-lane wave, so the exchange has six steps (32 .. 1), and each
// lane reads 16-byte vectors where the row allows it: a wave instruction
// then reads 1 KB of contiguous row.
//
//  * One wave per row, four independent waves per workgroup (no barriers,
//    no LDS).  Waves stride over the rows of the launch.
//  * Rows of up to 4096 elements are held in registers (VPL 16-byte vectors
//    per lane), so each input element is read from memory once and each
//    output written once: the algorithmic minimum, making these kernels
//    HBM-bound.  Longer rows are streamed in passes.
//  * Arithmetic is FP32 with FP32 row sums (per-lane sums, then the DPP
//    combination order of wave_reduce); expf is the library's.
//  * In place is allowed (output pointer and leading dimension equal to an
//    input's): a wave reads every element of a row it needs before it
//    writes that element, so the pointers carry no no-alias qualifier.
#include "gemm_internal.hpp"
#include "rows_f32.h"

#include <climits>
#include <cmath>
#include <type_traits>

namespace {

constexpr int kWave = 64;
constexpr int kWavesPerGroup = 4;
constexpr int kThreads = kWave * kWavesPerGroup;

typedef float v4f __attribute__((ext_vector_type(4)));

// Lane exchange through DPP (data-parallel primitives: a VALU operand read
// from another lane of the same row of 16 lanes, or broadcast from the
// previous row).  Lanes of rows outside ROW_MASK receive `old`.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp(float x, float old)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                                                  __builtin_bit_cast(int, x), CTRL,
                                                                  ROW_MASK, 0xf, false));
}

// The page reduces a row across the warp with xor exchanges (distances
// 16 .. 1).  On gfx9 a cross-lane exchange through __shfl_xor is an LDS
// permute, six dependent ones per reduction; here the combination runs on
// DPP instead: xor 1 and xor 2 inside each quad, then the mirrors of 8 and
// of 16 lanes (after which every lane of a 16-lane row holds the row's
// total), then lane 15 of rows 0 and 2 is added into rows 1 and 3, and
// lane 31 into rows 2 and 3.  Lane 63 ends with the wave's total, read back
// as a wave-uniform value (+1-2 % on the softmax kernels and the
// normalisation gradient).
template <class Op>
__device__ __forceinline__ float wave_reduce(float v, Op op, float identity)
{
    v = op(v, dpp<0xB1>(v, identity));        // quad_perm [1, 0, 3, 2]
    v = op(v, dpp<0x4E>(v, identity));        // quad_perm [2, 3, 0, 1]
    v = op(v, dpp<0x141>(v, identity));       // row_half_mirror
    v = op(v, dpp<0x140>(v, identity));       // row_mirror
    v = op(v, dpp<0x142, 0xa>(v, identity));  // row_bcast:15 into rows 1, 3
    v = op(v, dpp<0x143, 0xc>(v, identity));  // row_bcast:31 into rows 2, 3
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), kWave - 1));
}

__device__ __forceinline__ float wave_sum(float v)
{
    return wave_reduce(v, [](float a, float b) { return a + b; }, 0.0f);
}

__device__ __forceinline__ float wave_max(float v)
{
    return wave_reduce(v, [](float a, float b) { return fmaxf(a, b); }, -INFINITY);
}

// Element slot e (0 <= e < 4*VPL) of a lane: with 16-byte vectors, vector
// e/4 of the lane covers columns 4*(lane + 64*(e/4)) .. +3; otherwise slot e
// is column lane + 64*e.  Either way the slots of all lanes cover columns
// 0 .. 256*VPL - 1 exactly once.
template <bool VEC>
__device__ __forceinline__ int col_of(int lane, int e)
{
    return VEC ? 4 * (lane + kWave * (e / 4)) + (e % 4) : lane + kWave * e;
}

// Load the row's elements into v (columns >= width get `fill`).
template <int VPL, bool VEC>
__device__ __forceinline__ void load_row(const float *row, int width, int lane, float (&v)[4 * VPL],
                                         float fill)
{
#pragma unroll
    for (int q = 0; q < VPL; ++q) {
        if (VEC) {
            const int c = 4 * (lane + kWave * q);
            if (c < width) {  // width % 4 == 0 on this path: the vector is inside the row
                const v4f x = *reinterpret_cast<const v4f *>(row + c);
                v[4 * q] = x[0];
                v[4 * q + 1] = x[1];
                v[4 * q + 2] = x[2];
                v[4 * q + 3] = x[3];
            } else {
                v[4 * q] = v[4 * q + 1] = v[4 * q + 2] = v[4 * q + 3] = fill;
            }
        } else {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int c = col_of<false>(lane, 4 * q + u);
                v[4 * q + u] = c < width ? row[c] : fill;
            }
        }
    }
}

// NT: streaming (non-temporal) stores, for outputs nothing here reads back
// (the normalisation: 8192 x 1024, 7.5 vs 6.1 TB/s; its gradient +1.6 %; the
// softmax was 1 % slower with them).
template <int VPL, bool VEC, bool NT = false>
__device__ __forceinline__ void store_row(float *row, int width, int lane, const float (&v)[4 * VPL])
{
#pragma unroll
    for (int q = 0; q < VPL; ++q) {
        if (VEC) {
            const int c = 4 * (lane + kWave * q);
            const v4f x = v4f{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
            if (c < width) {
                if (NT)
                    __builtin_nontemporal_store(x, reinterpret_cast<v4f *>(row + c));
                else
                    *reinterpret_cast<v4f *>(row + c) = x;
            }
        } else {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int c = col_of<false>(lane, 4 * q + u);
                if (c < width) {
                    if (NT)
                        __builtin_nontemporal_store(v[4 * q + u], row + c);
                    else
                        row[c] = v[4 * q + u];
                }
            }
        }
    }
}

struct Rows {
    int rows, width;
};

__device__ __forceinline__ int wave_id() { return int(blockIdx.x) * kWavesPerGroup + int(threadIdx.x) / kWave; }
__device__ __forceinline__ int wave_count() { return int(gridDim.x) * kWavesPerGroup; }
__device__ __forceinline__ int lane_id() { return int(threadIdx.x) % kWave; }

// ------------------------------------------------------------- softmax ---
// y = exp(scale*x - m) / s over the kept columns (c <= the row's query
// position when causal), 0 elsewhere; masked inputs are never used.  The
// page writes exp(scale*x - m - log s), the same value; dividing by s needs
// one exponential per element instead of two, and the exponentials, not the
// memory traffic, bounded the two-exponential form (5.8 vs 6.9 TB/s on the
// attention-score workload).
template <int VPL, bool VEC>
__global__ __launch_bounds__(kThreads) void softmax_kernel(Rows sh, int queries, int causal, float scale,
                                                           const float *x, int64_t ldx,
                                                           float *y, int64_t ldy)
{
    const int lane = lane_id();
    for (int r = wave_id(); r < sh.rows; r += wave_count()) {
        const int keep = causal ? sh.width - queries + r % queries + 1 : sh.width;
        float v[4 * VPL];
        load_row<VPL, VEC>(x + int64_t(r) * ldx, sh.width, lane, v, 0.0f);
        float m = -INFINITY;
#pragma unroll
        for (int e = 0; e < 4 * VPL; ++e) {
            const bool kept = col_of<VEC>(lane, e) < keep;
            v[e] = kept ? scale * v[e] : -INFINITY;
            m = fmaxf(m, v[e]);
        }
        m = wave_max(m);
        float s = 0.0f;
#pragma unroll
        for (int e = 0; e < 4 * VPL; ++e) {
            v[e] = col_of<VEC>(lane, e) < keep ? expf(v[e] - m) : 0.0f;
            s += v[e];
        }
        const float inv = 1.0f / wave_sum(s);
#pragma unroll
        for (int e = 0; e < 4 * VPL; ++e) v[e] *= inv;
        store_row<VPL, VEC>(y + int64_t(r) * ldy, sh.width, lane, v);
    }
}

// Rows longer than the register path: online max and rescaled sum in one
// pass, then the output in a second pass (element order within a lane).
__global__ __launch_bounds__(kThreads) void softmax_long_kernel(Rows sh, int queries, int causal, float scale,
                                                                const float *x, int64_t ldx,
                                                                float *y, int64_t ldy)
{
    const int lane = lane_id();
    for (int r = wave_id(); r < sh.rows; r += wave_count()) {
        const int keep = causal ? sh.width - queries + r % queries + 1 : sh.width;
        const float *row = x + int64_t(r) * ldx;
        float m = -INFINITY, s = 0.0f;
        for (int c = lane; c < keep; c += kWave) {
            const float z = scale * row[c];
            // A score of -inf adds exp(-inf) = 0 to the sum; it is skipped
            // rather than evaluated, since before the lane's first finite
            // score m is -inf too and exp(-inf - -inf) would be NaN.
            if (z > m) {
                s = s * expf(m - z) + 1.0f;
                m = z;
            } else if (z > -INFINITY) {
                s += expf(z - m);
            }
        }
        const float wm = wave_max(m);
        const float inv = 1.0f / wave_sum(m == -INFINITY ? 0.0f : s * expf(m - wm));
        float *out = y + int64_t(r) * ldy;
        for (int c = lane; c < sh.width; c += kWave)
            out[c] = c < keep ? expf(scale * row[c] - wm) * inv : 0.0f;
    }
}

// ---------------------------------------------------- softmax gradient ---
// dx = scale * y * (dy - sum(dy * y)).
template <int VPL, bool VEC>
__global__ __launch_bounds__(kThreads) void softmax_backward_kernel(Rows sh, float scale,
                                                                    const float *y, int64_t ldy,
                                                                    const float *dy, int64_t lddy,
                                                                    float *dx, int64_t lddx)
{
    const int lane = lane_id();
    for (int r = wave_id(); r < sh.rows; r += wave_count()) {
        float a[4 * VPL], g[4 * VPL];
        load_row<VPL, VEC>(y + int64_t(r) * ldy, sh.width, lane, a, 0.0f);
        load_row<VPL, VEC>(dy + int64_t(r) * lddy, sh.width, lane, g, 0.0f);
        float d = 0.0f;
#pragma unroll
        for (int e = 0; e < 4 * VPL; ++e) d += g[e] * a[e];
        d = wave_sum(d);
#pragma unroll
        for (int e = 0; e < 4 * VPL; ++e) a[e] = scale * a[e] * (g[e] - d);
        store_row<VPL, VEC>(dx + int64_t(r) * lddx, sh.width, lane, a);
    }
}

__global__ __launch_bounds__(kThreads) void softmax_backward_long_kernel(Rows sh, float scale,
                                                                         const float *y, int64_t ldy,
                                                                         const float *dy, int64_t lddy,
                                                                         float *dx, int64_t lddx)
{
    const int lane = lane_id();
    for (int r = wave_id(); r < sh.rows; r += wave_count()) {
        const float *a = y + int64_t(r) * ldy;
        const float *g = dy + int64_t(r) * lddy;
        float d = 0.0f;
        for (int c = lane; c < sh.width; c += kWave) d += g[c] * a[c];
        d = wave_sum(d);
        float *out = dx + int64_t(r) * lddx;
        for (int c = lane; c < sh.width; c += kWave) out[c] = scale * a[c] * (g[c] - d);
    }
}

// ------------------------------------------------------------ normalize ---
// y = (x - mean) / sqrt(var + eps), var the mean squared deviation (taken
// around the mean, a second pass over the registers).
template <int VPL, bool VEC>
__global__ __launch_bounds__(kThreads) void normalize_kernel(Rows sh, float eps, const float *x,
                                                             int64_t ldx, float *y, int64_t ldy)
{
    const int lane = lane_id();
    const float inv_n = 1.0f / float(sh.width);
    for (int r = wave_id(); r < sh.rows; r += wave_count()) {
        float v[4 * VPL];
        load_row<VPL, VEC>(x + int64_t(r) * ldx, sh.width, lane, v, 0.0f);
        float s = 0.0f;
#pragma unroll
        for (int e = 0; e < 4 * VPL; ++e) s += v[e];
        const float mu = wave_sum(s) * inv_n;
        float q = 0.0f;
#pragma unroll
        for (int e = 0; e < 4 * VPL; ++e) {
            v[e] = col_of<VEC>(lane, e) < sh.width ? v[e] - mu : 0.0f;
            q += v[e] * v[e];
        }
        const float rs = 1.0f / sqrtf(wave_sum(q) * inv_n + eps);
#pragma unroll
        for (int e = 0; e < 4 * VPL; ++e) v[e] *= rs;
        store_row<VPL, VEC, true>(y + int64_t(r) * ldy, sh.width, lane, v);
    }
}

__global__ __launch_bounds__(kThreads) void normalize_long_kernel(Rows sh, float eps, const float *x,
                                                                  int64_t ldx, float *y, int64_t ldy)
{
    const int lane = lane_id();
    const float inv_n = 1.0f / float(sh.width);
    for (int r = wave_id(); r < sh.rows; r += wave_count()) {
        const float *row = x + int64_t(r) * ldx;
        float s = 0.0f;
        for (int c = lane; c < sh.width; c += kWave) s += row[c];
        const float mu = wave_sum(s) * inv_n;
        float q = 0.0f;
        for (int c = lane; c < sh.width; c += kWave) {
            const float d = row[c] - mu;
            q += d * d;
        }
        const float rs = 1.0f / sqrtf(wave_sum(q) * inv_n + eps);
        float *out = y + int64_t(r) * ldy;
        for (int c = lane; c < sh.width; c += kWave) out[c] = (row[c] - mu) * rs;
    }
}

// --------------------------------------------------- normalize gradient ---
// dx = (dy - mean(dy) - xhat * mean(dy * xhat)) / sigma, sigma and xhat
// recomputed from x.
template <int VPL, bool VEC>
__global__ __launch_bounds__(kThreads) void normalize_backward_kernel(Rows sh, float eps,
                                                                      const float *x, int64_t ldx,
                                                                      const float *dy, int64_t lddy,
                                                                      float *dx, int64_t lddx)
{
    const int lane = lane_id();
    const float inv_n = 1.0f / float(sh.width);
    for (int r = wave_id(); r < sh.rows; r += wave_count()) {
        float v[4 * VPL], g[4 * VPL];
        load_row<VPL, VEC>(x + int64_t(r) * ldx, sh.width, lane, v, 0.0f);
        load_row<VPL, VEC>(dy + int64_t(r) * lddy, sh.width, lane, g, 0.0f);
        float s = 0.0f;
#pragma unroll
        for (int e = 0; e < 4 * VPL; ++e) s += v[e];
        const float mu = wave_sum(s) * inv_n;
        float q = 0.0f;
#pragma unroll
        for (int e = 0; e < 4 * VPL; ++e) {
            v[e] = col_of<VEC>(lane, e) < sh.width ? v[e] - mu : 0.0f;
            q += v[e] * v[e];
        }
        const float rs = 1.0f / sqrtf(wave_sum(q) * inv_n + eps);
        float sg = 0.0f, sgx = 0.0f;
#pragma unroll
        for (int e = 0; e < 4 * VPL; ++e) {
            v[e] *= rs;  // xhat (0 beyond the row)
            sg += g[e];
            sgx += g[e] * v[e];
        }
        const float mg = wave_sum(sg) * inv_n, mgx = wave_sum(sgx) * inv_n;
#pragma unroll
        for (int e = 0; e < 4 * VPL; ++e) v[e] = (g[e] - mg - v[e] * mgx) * rs;
        store_row<VPL, VEC, true>(dx + int64_t(r) * lddx, sh.width, lane, v);
    }
}

__global__ __launch_bounds__(kThreads) void normalize_backward_long_kernel(Rows sh, float eps,
                                                                           const float *x, int64_t ldx,
                                                                           const float *dy, int64_t lddy,
                                                                           float *dx, int64_t lddx)
{
    const int lane = lane_id();
    const float inv_n = 1.0f / float(sh.width);
    for (int r = wave_id(); r < sh.rows; r += wave_count()) {
        const float *row = x + int64_t(r) * ldx;
        const float *g = dy + int64_t(r) * lddy;
        float s = 0.0f;
        for (int c = lane; c < sh.width; c += kWave) s += row[c];
        const float mu = wave_sum(s) * inv_n;
        float q = 0.0f;
        for (int c = lane; c < sh.width; c += kWave) {
            const float d = row[c] - mu;
            q += d * d;
        }
        const float rs = 1.0f / sqrtf(wave_sum(q) * inv_n + eps);
        float sg = 0.0f, sgx = 0.0f;
        for (int c = lane; c < sh.width; c += kWave) {
            sg += g[c];
            sgx += g[c] * ((row[c] - mu) * rs);
        }
        const float mg = wave_sum(sg) * inv_n, mgx = wave_sum(sgx) * inv_n;
        float *out = dx + int64_t(r) * lddx;
        for (int c = lane; c < sh.width; c += kWave) out[c] = (g[c] - mg - ((row[c] - mu) * rs) * mgx) * rs;
    }
}

// ---------------------------------------------------------------- launch ---

constexpr int kMaxGroups = 4096;  // 16384 waves: 64 per CU; rows beyond are strided

unsigned groups_for(int rows)
{
    const int want = (rows + kWavesPerGroup - 1) / kWavesPerGroup;
    return unsigned(want < kMaxGroups ? want : kMaxGroups);
}

bool vec_ok(const float *p, int64_t ld, int width)
{
    return width % 4 == 0 && ld % 4 == 0 && (reinterpret_cast<uintptr_t>(p) & 15) == 0;
}

// Calls launch(Int VPL, Bool VEC) for the smallest register tile holding the
// row (VPL in 1, 2, 4, 8, 16 vectors per lane), or long_launch() beyond 4096.
template <class F, class G>
void by_width(int width, bool vec, F &&launch, G &&long_launch)
{
    auto pick = [&](auto vpl) {
        if (vec)
            launch(vpl, std::true_type{});
        else
            launch(vpl, std::false_type{});
    };
    if (width <= 256) pick(std::integral_constant<int, 1>{});
    else if (width <= 512) pick(std::integral_constant<int, 2>{});
    else if (width <= 1024) pick(std::integral_constant<int, 4>{});
    else if (width <= 2048) pick(std::integral_constant<int, 8>{});
    else if (width <= 4096) pick(std::integral_constant<int, 16>{});
    else long_launch();
}

constexpr int64_t kDimLimit = int64_t(INT_MAX);

int check_shape(int64_t rows, int64_t width)
{
    if (rows < 0 || rows > kDimLimit) return -1;
    if (width < 0 || width > kDimLimit) return -2;
    return 0;
}

bool ld_ok(int64_t ld, int64_t width) { return ld >= (width > 1 ? width : 1) && ld <= kDimLimit; }

}  // namespace

extern "C" {

int rows_softmax_f32(int64_t rows, int64_t width, int64_t queries, int causal, float scale,
                     const float *x, int64_t ldx, float *y, int64_t ldy, void *stream)
{
    if (int bad = check_shape(rows, width)) return bad;
    if (causal != 0 && causal != 1) return -4;
    if (causal && width > 0 && (queries < 1 || queries > width)) return -3;
    const bool any = rows > 0 && width > 0;
    if (any && x == nullptr) return -6;
    if (!ld_ok(ldx, width)) return -7;
    if (any && y == nullptr) return -8;
    if (!ld_ok(ldy, width)) return -9;
    if (!any) return 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const Rows sh{int(rows), int(width)};
    const int q = causal ? int(queries) : 1;
    const unsigned grid = groups_for(sh.rows);
    by_width(sh.width, vec_ok(x, ldx, sh.width) && vec_ok(y, ldy, sh.width),
             [&](auto vpl, auto vec) {
                 softmax_kernel<decltype(vpl)::value, decltype(vec)::value>
                     <<<grid, kThreads, 0, s>>>(sh, q, causal, scale, x, ldx, y, ldy);
             },
             [&] { softmax_long_kernel<<<grid, kThreads, 0, s>>>(sh, q, causal, scale, x, ldx, y, ldy); });
    const hipError_t err = hipGetLastError();
    return err == hipSuccess ? 0 : int(err);
}

int rows_softmax_backward_f32(int64_t rows, int64_t width, float scale, const float *y, int64_t ldy,
                              const float *dy, int64_t lddy, float *dx, int64_t lddx, void *stream)
{
    if (int bad = check_shape(rows, width)) return bad;
    const bool any = rows > 0 && width > 0;
    if (any && y == nullptr) return -4;
    if (!ld_ok(ldy, width)) return -5;
    if (any && dy == nullptr) return -6;
    if (!ld_ok(lddy, width)) return -7;
    if (any && dx == nullptr) return -8;
    if (!ld_ok(lddx, width)) return -9;
    if (!any) return 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const Rows sh{int(rows), int(width)};
    const unsigned grid = groups_for(sh.rows);
    by_width(sh.width, vec_ok(y, ldy, sh.width) && vec_ok(dy, lddy, sh.width) && vec_ok(dx, lddx, sh.width),
             [&](auto vpl, auto vec) {
                 softmax_backward_kernel<decltype(vpl)::value, decltype(vec)::value>
                     <<<grid, kThreads, 0, s>>>(sh, scale, y, ldy, dy, lddy, dx, lddx);
             },
             [&] { softmax_backward_long_kernel<<<grid, kThreads, 0, s>>>(sh, scale, y, ldy, dy, lddy, dx, lddx); });
    const hipError_t err = hipGetLastError();
    return err == hipSuccess ? 0 : int(err);
}

int rows_normalize_f32(int64_t rows, int64_t n, float eps, const float *x, int64_t ldx, float *y,
                       int64_t ldy, void *stream)
{
    if (int bad = check_shape(rows, n)) return bad;
    if (!(eps >= 0.0f) || std::isinf(eps)) return -3;
    const bool any = rows > 0 && n > 0;
    if (any && x == nullptr) return -4;
    if (!ld_ok(ldx, n)) return -5;
    if (any && y == nullptr) return -6;
    if (!ld_ok(ldy, n)) return -7;
    if (!any) return 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const Rows sh{int(rows), int(n)};
    const unsigned grid = groups_for(sh.rows);
    by_width(sh.width, vec_ok(x, ldx, sh.width) && vec_ok(y, ldy, sh.width),
             [&](auto vpl, auto vec) {
                 normalize_kernel<decltype(vpl)::value, decltype(vec)::value>
                     <<<grid, kThreads, 0, s>>>(sh, eps, x, ldx, y, ldy);
             },
             [&] { normalize_long_kernel<<<grid, kThreads, 0, s>>>(sh, eps, x, ldx, y, ldy); });
    const hipError_t err = hipGetLastError();
    return err == hipSuccess ? 0 : int(err);
}

int rows_normalize_backward_f32(int64_t rows, int64_t n, float eps, const float *x, int64_t ldx,
                                const float *dy, int64_t lddy, float *dx, int64_t lddx, void *stream)
{
    if (int bad = check_shape(rows, n)) return bad;
    if (!(eps >= 0.0f) || std::isinf(eps)) return -3;
    const bool any = rows > 0 && n > 0;
    if (any && x == nullptr) return -4;
    if (!ld_ok(ldx, n)) return -5;
    if (any && dy == nullptr) return -6;
    if (!ld_ok(lddy, n)) return -7;
    if (any && dx == nullptr) return -8;
    if (!ld_ok(lddx, n)) return -9;
    if (!any) return 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const Rows sh{int(rows), int(n)};
    const unsigned grid = groups_for(sh.rows);
    by_width(sh.width, vec_ok(x, ldx, sh.width) && vec_ok(dy, lddy, sh.width) && vec_ok(dx, lddx, sh.width),
             [&](auto vpl, auto vec) {
                 normalize_backward_kernel<decltype(vpl)::value, decltype(vec)::value>
                     <<<grid, kThreads, 0, s>>>(sh, eps, x, ldx, dy, lddy, dx, lddx);
             },
             [&] { normalize_backward_long_kernel<<<grid, kThreads, 0, s>>>(sh, eps, x, ldx, dy, lddy, dx, lddx); });
    const hipError_t err = hipGetLastError();
    return err == hipSuccess ? 0 : int(err);
}

}  // extern "C"
