// gemm_bf16.hip -- mixed-precision GEMM: FP32 operands rounded to bf16 on
// their way into LDS, products on the CDNA4 matrix cores
// (v_mfma_f32_32x32x16_bf16), sums and C in FP32.
//
// This is the mixed precision of the Smallem page ("Rendre le GPU rapide",
// section "Les Tensor Cores"): only the two operands of each product are
// rounded to 16 bits, to nearest with ties to even; every tensor and every
// sum stays FP32.  Layout of the work:
//
//  * A BM x BN tile of C per workgroup of WAVES_M x WAVES_N waves; each
//    wave owns FM x FN blocks of 32 x 32 in registers.  One MFMA covers
//    16 k (32768 flops per wave instruction).
//  * Each stage (BK k) is read from global memory as 16-byte FP32 vectors
//    (predicated at the edges, zero outside the matrix), converted with
//    v_cvt_pk_bf16_f32 (round to nearest even) and written to LDS while the
//    previous stage is multiplied: two LDS buffers, one barrier per stage.
//  * Both LDS tiles are k-contiguous, [rows][BK + 8] bf16, so that every
//    MFMA fragment (8 consecutive k of one row) is one 16-byte LDS read.
//    The 16-byte row padding puts the 16 rows read by 16 consecutive lanes
//    on distinct banks (the course page's padding remedy, section 3.6).
//  * An operand stored with k along its rows (A untransposed, B transposed)
//    is copied row by row.  One stored with k down its columns is
//    transposed on the way in: each thread reads 4 consecutive k rows of 4
//    columns, and writes, per column, the 4 k values as one 8-byte LDS
//    store; 8 lanes fill one 64-byte k-row of the LDS tile.
//  * Lanes 0-31 of a wave supply k slots 0-7 of the MFMA and lanes 32-63
//    slots 8-15, for A and B alike, so every (a_ik, b_kj) pair meets once
//    whatever order the matrix core adds the slots in.
//  * Partial sums over FOLD stages are added into the running tile (sums
//    over short runs of k first, as in the FP32 kernels).
#include "tile_common.hpp"

namespace gemmf32 {
namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

template <int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_, int FOLD_, int GROUP_M_>
struct Config {
    static constexpr int BM = BM_, BN = BN_, BK = BK_;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int THREADS = kWave * WAVES_M * WAVES_N;
    static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;  // per-wave C tile
    static constexpr int FM = WM / 32, FN = WN / 32;            // 32 x 32 blocks per wave
    static constexpr int LD = BK + 8;                           // bf16 per LDS row
    static constexpr int FOLD = FOLD_;
    static constexpr int GROUP_M = GROUP_M_;
    static_assert(WM % 32 == 0 && WN % 32 == 0 && BK % 16 == 0, "whole MFMA blocks");
};

// Load 4 consecutive floats of a stored row (r, c .. c+3).  CHECK: elements
// outside the stored matrix read as zero and are not dereferenced.  VEC:
// one aligned 16-byte load is allowed.
template <bool CHECK, bool VEC>
__device__ __forceinline__ v4f load4(const Operand &op, int r, int c)
{
    const float *src = op.base + int64_t(r) * op.ld + c;
    if (!CHECK || (r < op.rows_total && c + 3 < op.cols_total)) {
        if (VEC) return *reinterpret_cast<const v4f *>(src);
        return v4f{src[0], src[1], src[2], src[3]};
    }
    v4f x;
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = (r < op.rows_total && c + e < op.cols_total) ? src[e] : 0.0f;
    return x;
}

__device__ __forceinline__ v4bf to_bf16(v4f x)
{
    return v4bf{(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3]};
}

// One operand's share of a stage: ROWS rows (m or n) of the tile times BK k.
// KC: the operand is stored with k along its rows.
template <class Cfg, int ROWS, bool KC>
struct Stage;

// k along the stored rows: thread t reads vector (row, 4 k) number
// t + THREADS * q, 8-byte LDS stores in row order.
template <class Cfg, int ROWS>
struct Stage<Cfg, ROWS, true> {
    static constexpr int per_row = Cfg::BK / 4;
    static constexpr int per_thread = ROWS * per_row / Cfg::THREADS;
    static_assert(ROWS * per_row % Cfg::THREADS == 0, "stage splits evenly");

    template <bool CHECK, bool VEC>
    __device__ static __forceinline__ void load(const Operand &op, int row0, int k0, v4f (&reg)[per_thread])
    {
#pragma unroll
        for (int q = 0; q < per_thread; ++q) {
            const int v = int(threadIdx.x) + Cfg::THREADS * q;
            reg[q] = load4<CHECK, VEC>(op, row0 + v / per_row, k0 + 4 * (v % per_row));
        }
    }

    __device__ static __forceinline__ void store(__bf16 *lds, const v4f (&reg)[per_thread])
    {
#pragma unroll
        for (int q = 0; q < per_thread; ++q) {
            const int v = int(threadIdx.x) + Cfg::THREADS * q;
            *reinterpret_cast<v4bf *>(lds + (v / per_row) * Cfg::LD + 4 * (v % per_row)) = to_bf16(reg[q]);
        }
    }
};

// k down the stored columns: thread t owns k group g = t % (BK / 4) (four
// consecutive k rows) and column group c = t / (BK / 4) (four columns) of
// each block of columns; q runs over the k rows, then over column blocks.
template <class Cfg, int ROWS>
struct Stage<Cfg, ROWS, false> {
    static constexpr int kgroups = Cfg::BK / 4;
    static constexpr int cols_per_pass = 4 * (Cfg::THREADS / kgroups);
    static constexpr int passes = ROWS / cols_per_pass;
    static constexpr int per_thread = 4 * passes;
    static_assert(Cfg::THREADS % kgroups == 0 && ROWS % cols_per_pass == 0, "stage splits evenly");

    template <bool CHECK, bool VEC>
    __device__ static __forceinline__ void load(const Operand &op, int row0, int k0, v4f (&reg)[per_thread])
    {
        const int g = int(threadIdx.x) % kgroups, c = int(threadIdx.x) / kgroups;
#pragma unroll
        for (int p = 0; p < passes; ++p)
#pragma unroll
            for (int u = 0; u < 4; ++u)
                reg[4 * p + u] = load4<CHECK, VEC>(op, k0 + 4 * g + u, row0 + cols_per_pass * p + 4 * c);
    }

    __device__ static __forceinline__ void store(__bf16 *lds, const v4f (&reg)[per_thread])
    {
        const int g = int(threadIdx.x) % kgroups, c = int(threadIdx.x) / kgroups;
#pragma unroll
        for (int p = 0; p < passes; ++p) {
            const v4bf h[4] = {to_bf16(reg[4 * p]), to_bf16(reg[4 * p + 1]), to_bf16(reg[4 * p + 2]),
                               to_bf16(reg[4 * p + 3])};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = cols_per_pass * p + 4 * c + e;
                *reinterpret_cast<v4bf *>(lds + row * Cfg::LD + 4 * g) = v4bf{h[0][e], h[1][e], h[2][e], h[3][e]};
            }
        }
    }
};

template <class Cfg, bool A_KC, bool B_KC, bool VEC>
__global__ __attribute__((amdgpu_flat_work_group_size(Cfg::THREADS, Cfg::THREADS))) void
bf16_kernel(int M, int N, int K, const float *__restrict__ A, int64_t lda,
            const float *__restrict__ B, int64_t ldb, float *__restrict__ C, int64_t ldc,
            int tiles_m, int tiles_n, int tile_base)
{
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, LD = Cfg::LD;
    constexpr int FM = Cfg::FM, FN = Cfg::FN, FOLD = Cfg::FOLD;
    using SA = Stage<Cfg, BM, A_KC>;
    using SB = Stage<Cfg, BN, B_KC>;
    constexpr int kTileA = BM * LD, kTileB = BN * LD;
    // Both stage buffers in one array, so that an LDS address in one buffer
    // and the same position in the other differ by a constant the compiler
    // can fold into the instruction's offset.
    __shared__ __attribute__((aligned(16))) __bf16 lds_both[2 * (kTileA + kTileB)];
    __bf16 *const lds0 = lds_both;
    __bf16 *const lds1 = lds_both + kTileA + kTileB;

    int tm, tn;
    tile_of<Cfg::GROUP_M>(tile_base + int(blockIdx.x), tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const bool inside = (m0 + BM <= M) && (n0 + BN <= N);
    const int wave = int(threadIdx.x) / kWave, lane = int(threadIdx.x) % kWave;
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);  // the same, in a scalar register
    const int wm = (wave / Cfg::WAVES_N) * Cfg::WM, wn = (wave % Cfg::WAVES_N) * Cfg::WN;
    const int half = lane / 32, l32 = lane % 32;

    // Stored views: A is M x K (k along rows) or K x M; B is K x N or N x K.
    const Operand opa{A, lda, A_KC ? M : K, A_KC ? K : M};
    const Operand opb{B, ldb, B_KC ? N : K, B_KC ? K : N};

    // Two register sets: stage s + 1 waits in one (loaded an iteration
    // earlier) while stage s + 2 is being fetched into the other.
    v4f ra0[SA::per_thread], rb0[SB::per_thread], ra1[SA::per_thread], rb1[SB::per_thread];
    auto load = [&](int k, auto &ra, auto &rb) {
        if (inside && k + BK <= K) {
            SA::template load<false, VEC>(opa, m0, k, ra);
            SB::template load<false, VEC>(opb, n0, k, rb);
        } else {
            SA::template load<true, VEC>(opa, m0, k, ra);
            SB::template load<true, VEC>(opb, n0, k, rb);
        }
    };
    auto store = [&](__bf16 *lds, const auto &ra, const auto &rb) {
        SA::store(lds, ra);
        SB::store(lds + kTileA, rb);
    };

    v16f acc[FM][FN], part[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = part[i][j] = v16f{0.0f};

    // One stage of products into dst (zeroed first when `fresh`).
    auto compute = [&](const __bf16 *lds, v16f (&dst)[FM][FN], bool fresh) {
        const __bf16 *la = lds + (wm + l32) * LD + 8 * half;
        const __bf16 *lb = lds + kTileA + (wn + l32) * LD + 8 * half;
#pragma unroll
        for (int g = 0; g < BK / 16; ++g) {
            v8bf fa[FM], fb[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) fa[i] = *reinterpret_cast<const v8bf *>(la + 32 * i * LD + 16 * g);
#pragma unroll
            for (int j = 0; j < FN; ++j) fb[j] = *reinterpret_cast<const v8bf *>(lb + 32 * j * LD + 16 * g);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    dst[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        fa[i], fb[j], (g == 0 && fresh) ? v16f{0.0f} : dst[i][j], 0, 0, 0);
        }
    };

    const int stages = ceil_div(K, BK);
    // Stage s: computed from LDS buffer s % 2; its registers were set s % 2.
    auto step = [&](int s, const __bf16 *cur, __bf16 *nxt, auto &la, auto &lb, const auto &sa,
                    const auto &sb) {
        if (s + 2 < stages) load((s + 2) * BK, la, lb);  // set s % 2 is free: stage s is in LDS
        if (FOLD == 0) {
            compute(cur, acc, false);
        } else {
            compute(cur, part, s % FOLD == 0);
            if (s % FOLD == FOLD - 1 || s + 1 == stages) {
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j) acc[i][j] += part[i][j];
            }
        }
        // The other buffer was last read in stage s - 1, which every wave
        // finished before the barrier that ended it.
        if (s + 1 < stages) store(nxt, sa, sb);
        __syncthreads();
    };

    load(0, ra0, rb0);
    if (stages > 1) load(BK, ra1, rb1);
    store(lds0, ra0, rb0);
    __syncthreads();
    for (int s = 0; s < stages; s += 2) {
        step(s, lds0, lds1, ra0, rb0, ra1, rb1);
        if (s + 1 < stages) step(s + 1, lds1, lds0, ra1, rb1, ra0, rb0);
    }

    // Lane l of a 32 x 32 block holds column l % 32 and, in accumulator slot
    // v, row 8 * (v / 4) + 4 * (l / 32) + v % 4.  The lane's position is
    // derived afresh (lane index from the full execution mask, wave index
    // from a scalar register), so nothing lane-dependent has to stay in a
    // vector register across the k loop.
    const int e_lane = int(__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)));
    const int e_wm = (wave_s / Cfg::WAVES_N) * Cfg::WM, e_wn = (wave_s % Cfg::WAVES_N) * Cfg::WN;
    const int e_l32 = e_lane % 32, e_half = e_lane / 32;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int col = n0 + e_wn + 32 * j + e_l32;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = m0 + e_wm + 32 * i + 8 * (v / 4) + 4 * e_half + (v % 4);
                if (inside || (row < M && col < N)) C[int64_t(row) * ldc + col] = acc[i][j][v];
            }
        }
}

// Large: 256 x 256 tiles, 8 waves of 64 x 128, one unchunked accumulator
// (each MFMA already sums 16 products before its one rounding; the relative
// error of a K = 8192 product stays near 5.5e-7).  Small: 128 x 128 tiles,
// 8 waves of 32 x 64, 64-k stages summed into a fresh partial each (4 waves
// of 64 x 64 left one wave per SIMD to hide the converting loads: the
// ragged 2049 x 3071 x 769 product 146 -> 183 TFLOP/s, 1024^3 58 -> 71,
// 1024 x 4096 x 8192 217 -> 240).
#ifndef GEMM_BF16_LARGE_CONFIG
#define GEMM_BF16_LARGE_CONFIG 256, 256, 32, 4, 2, 0, 4
#endif
#ifndef GEMM_BF16_SMALL_CONFIG
#define GEMM_BF16_SMALL_CONFIG 128, 128, 64, 4, 2, 1, 8
#endif
using Large = Config<GEMM_BF16_LARGE_CONFIG>;
using Small = Config<GEMM_BF16_SMALL_CONFIG>;

template <class Cfg, bool A_KC, bool B_KC, bool VEC>
void dispatch(const Problem &p, hipStream_t s)
{
    const int tiles_m = ceil_div(p.M, Cfg::BM), tiles_n = ceil_div(p.N, Cfg::BN);
    const int64_t tiles = int64_t(tiles_m) * tiles_n;
    for (int64_t base = 0; base < tiles; base += kMaxGrid) {
        const int64_t n = tiles - base < kMaxGrid ? tiles - base : kMaxGrid;
        bf16_kernel<Cfg, A_KC, B_KC, VEC><<<dim3(unsigned(n)), dim3(Cfg::THREADS), 0, s>>>(
            p.M, p.N, p.K, p.A, p.lda, p.B, p.ldb, p.C, p.ldc, tiles_m, tiles_n, int(base));
    }
}

template <class Cfg, bool A_KC, bool B_KC>
void dispatch_vec(const Problem &p, hipStream_t s)
{
    if (vec4_ok(p.A, p.lda) && vec4_ok(p.B, p.ldb))
        dispatch<Cfg, A_KC, B_KC, true>(p, s);
    else
        dispatch<Cfg, A_KC, B_KC, false>(p, s);
}

template <class Cfg>
void dispatch_layout(const Problem &p, hipStream_t s)
{
    const bool a_kc = !p.transA, b_kc = p.transB;
    if (a_kc) {
        if (b_kc) dispatch_vec<Cfg, true, true>(p, s); else dispatch_vec<Cfg, true, false>(p, s);
    } else {
        if (b_kc) dispatch_vec<Cfg, false, true>(p, s); else dispatch_vec<Cfg, false, false>(p, s);
    }
}

// The large tile pays off from about half a tile per CU (measured: the
// 8192 x 1024 x 4096 product, 128 large tiles, 459 vs 360 TFLOP/s on the
// small tile); below that, or when a quarter of its area would fall outside
// C, or for K beyond 16384 (where an unchunked sum would drift towards the
// 1e-6 relative error bound), the small tile is used.
#ifndef GEMM_BF16_LARGE_FROM
#define GEMM_BF16_LARGE_FROM 128
#endif
constexpr int kLargeMaxK = 16384;

}  // namespace

hipError_t launch_bf16(const Problem &p, hipStream_t s, int tile)
{
    if (tile == 0) {
        const int64_t tiles = int64_t(ceil_div(p.M, Large::BM)) * ceil_div(p.N, Large::BN);
        const bool fits = 4 * int64_t(p.M) * p.N >= 3 * tiles * Large::BM * Large::BN;
        tile = (tiles >= GEMM_BF16_LARGE_FROM && fits && p.K <= kLargeMaxK) ? Large::BM : Small::BM;
    }
    if (tile == Large::BM)
        dispatch_layout<Large>(p, s);
    else
        dispatch_layout<Small>(p, s);
    return hipGetLastError();
}

}  // namespace gemmf32
