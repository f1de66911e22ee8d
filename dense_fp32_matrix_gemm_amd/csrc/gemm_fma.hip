// gemm_fma.hip -- FP32 GEMM with register-blocked vector FMA (no matrix cores).
//
// This is the register-tile kernel of the course page "3 . La memoire
// partagee", section 3.4, rebuilt for gfx950: a 128 x 128 tile of C per
// workgroup of 256 lanes, each lane owning an 8 x 8 register tile; per k the
// lane reads 8 values of A and 8 of B from LDS and performs the 64 FMAs of
// their outer product (16 LDS reads feed 64 FMAs, the page's 4:1 ratio).
// It is the comparison variant for the MFMA kernel: the same staging,
// double buffering, edge handling and launch order, with the outer product
// done by the vector ALU instead of the matrix core.
//
//  * LDS tiles are k-major, As[k][m] and Bs[k][n] (the page stores A
//    transposed so a column of A is contiguous).  Operands whose stored rows
//    run along k are transposed on their way into LDS, four scalar writes per
//    16-byte global load; rows are padded by 4 floats, and the transposed
//    tiles' 4-float groups are XOR-swizzled by k so those writes spread over
//    the banks.
//  * Lane (ty, tx) of the 16 x 16 lane grid owns rows {4ty..4ty+3,
//    64+4ty..64+4ty+3} and columns {4tx..4tx+3, 64+4tx..64+4tx+3}; its LDS
//    reads are four 16-byte reads per k, and the 16 lanes sharing a ty read
//    the same A address (a broadcast).
//  * Accumulation in chunks: each 32-k stage is summed into a fresh partial
//    tile that is then added to the running one, as in the MFMA kernel.
#include "tile_common.hpp"

namespace gemmf32 {
namespace {

constexpr int kThreads = 256;
constexpr int BM = 128, BN = 128, BK = 32;
constexpr int TM = 8, TN = 8;
// Row padding of the LDS tiles (section 3.6's remedy for bank conflicts);
// GEMM_FMA_PAD 0 builds the unpadded ablation (same results).
#ifndef GEMM_FMA_PAD
#define GEMM_FMA_PAD 4
#endif
constexpr int kPad = GEMM_FMA_PAD;
#ifndef GEMM_FMA_SWIZZLE
#define GEMM_FMA_SWIZZLE 1
#endif
constexpr int kLd = 128 + kPad;  // LDS row length, both operands (BM == BN)
constexpr int kGroupM = 8;

// Loader for one operand's stage slice.  KC: stored rows run along k, so the
// slice is P x BK and is transposed into LDS; otherwise it is BK x P.
template <int P, bool KC>
struct Stage {
    using Load = Slice<KC ? P : BK, KC ? BK : P, kThreads>;
    static constexpr int per_thread = Load::per_thread;

    // Transposed tiles: row k of the LDS tile holds m (or n) position x at
    // column x ^ swz(k).  The transposing writes of one wave cover 8
    // consecutive positions at 8 values of k four apart; with rows of 132
    // floats, k and k + 16 would land on the same bank, and flipping bit 3
    // of the position for k >= 16 separates them.  The flip moves whole
    // 4-float groups, so the 16-byte fragment reads stay contiguous.
    // GEMM_FMA_SWIZZLE 0 builds the unswizzled ablation (same results).
    __device__ static __forceinline__ int swz(int k)
    {
        return (KC && GEMM_FMA_SWIZZLE) ? ((k >> 4) & 1) << 3 : 0;
    }

    __device__ static __forceinline__ void store(float *lds, const v4f (&reg)[per_thread])
    {
#pragma unroll
        for (int q = 0; q < per_thread; ++q) {
            const int r = Load::row(q), c = Load::col(q);
            if (KC) {
#pragma unroll
                for (int e = 0; e < 4; ++e) lds[(c + e) * kLd + (r ^ swz(c + e))] = reg[q][e];
            } else {
                *reinterpret_cast<v4f *>(lds + r * kLd + c) = reg[q];
            }
        }
    }
};

template <bool A_KC, bool B_KC, bool VEC>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(2, 2))) void
fma_kernel(int M, int N, int K, const float *__restrict__ A, int64_t lda,
           const float *__restrict__ B, int64_t ldb, float *__restrict__ C, int64_t ldc,
           int tiles_m, int tiles_n, int vec_c)
{
    using SA = Stage<BM, A_KC>;
    using SB = Stage<BN, B_KC>;
    constexpr int kTile = BK * kLd;
    __shared__ __attribute__((aligned(16))) float smem[4 * kTile];

    const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
    const int tiles = tiles_m * tiles_n;
    for (int t = blockIdx.x; t < tiles; t += gridDim.x) {
        int tm, tn;
        tile_of<kGroupM>(t, tiles_m, tiles_n, tm, tn);
        const int m0 = tm * BM, n0 = tn * BN;
        const bool inside = (m0 + BM <= M) && (n0 + BN <= N);
        const Operand opa{A, lda, A_KC ? M : K, A_KC ? K : M};
        const Operand opb{B, ldb, B_KC ? N : K, B_KC ? K : N};

        v4f ra[SA::per_thread], rb[SB::per_thread];
        auto load = [&](int k) {
            const int ar = A_KC ? m0 : k, ac = A_KC ? k : m0;
            const int br = B_KC ? n0 : k, bc = B_KC ? k : n0;
            if (inside && k + BK <= K) {
                SA::Load::template load<false, VEC>(opa, ar, ac, ra);
                SB::Load::template load<false, VEC>(opb, br, bc, rb);
            } else {
                SA::Load::template load<true, VEC>(opa, ar, ac, ra);
                SB::Load::template load<true, VEC>(opb, br, bc, rb);
            }
        };

        float acc[TM][TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = 0.0f;

        const int stages = ceil_div(K, BK);
        load(0);
        SA::store(smem, ra);
        SB::store(smem + kTile, rb);
        __syncthreads();

        for (int s = 0; s < stages; ++s) {
            const bool next = s + 1 < stages;
            if (next) load((s + 1) * BK);
            const float *la = smem + (s & 1) * 2 * kTile;
            const float *lb = la + kTile;

            float part[TM][TN];
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) part[i][j] = 0.0f;
#pragma unroll 4
            for (int k = 0; k < BK; ++k) {
                const int sa = SA::swz(k), sb = SB::swz(k);
                const v4f a0 = *reinterpret_cast<const v4f *>(la + k * kLd + ((4 * ty) ^ sa));
                const v4f a1 = *reinterpret_cast<const v4f *>(la + k * kLd + ((64 + 4 * ty) ^ sa));
                const v4f b0 = *reinterpret_cast<const v4f *>(lb + k * kLd + ((4 * tx) ^ sb));
                const v4f b1 = *reinterpret_cast<const v4f *>(lb + k * kLd + ((64 + 4 * tx) ^ sb));
                const float a[TM] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
                const float b[TN] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j) part[i][j] = __builtin_fmaf(a[i], b[j], part[i][j]);
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] += part[i][j];

            if (next) {
                float *wa = smem + ((s + 1) & 1) * 2 * kTile;
                SA::store(wa, ra);
                SB::store(wa + kTile, rb);
            }
            __syncthreads();
        }

        // Epilogue: rows 4ty + r and 64 + 4ty + r, columns 4tx.. and 64 + 4tx..
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int row = m0 + (i / 4) * 64 + 4 * ty + (i % 4);
#pragma unroll
            for (int jh = 0; jh < 2; ++jh) {
                const int col = n0 + jh * 64 + 4 * tx;
                float *dst = C + int64_t(row) * ldc + col;
                if (inside && vec_c) {
                    *reinterpret_cast<v4f *>(dst) = v4f{acc[i][4 * jh], acc[i][4 * jh + 1],
                                                        acc[i][4 * jh + 2], acc[i][4 * jh + 3]};
                } else if (row < M) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (col + e < N) dst[e] = acc[i][4 * jh + e];
                }
            }
        }
    }
}

template <bool A_KC, bool B_KC, bool VEC>
void dispatch(const Problem &p, hipStream_t s)
{
    const int tiles_m = ceil_div(p.M, BM), tiles_n = ceil_div(p.N, BN);
    const int64_t tiles = int64_t(tiles_m) * tiles_n;
    const dim3 grid(unsigned(tiles < kMaxGrid ? tiles : kMaxGrid));
    fma_kernel<A_KC, B_KC, VEC><<<grid, dim3(kThreads), 0, s>>>(
        p.M, p.N, p.K, p.A, p.lda, p.B, p.ldb, p.C, p.ldc, tiles_m, tiles_n,
        int(vec4_ok(p.C, p.ldc)));
}

template <bool A_KC, bool B_KC>
void dispatch_vec(const Problem &p, hipStream_t s)
{
    if (vec4_ok(p.A, p.lda) && vec4_ok(p.B, p.ldb))
        dispatch<A_KC, B_KC, true>(p, s);
    else
        dispatch<A_KC, B_KC, false>(p, s);
}

}  // namespace

hipError_t launch_fma(const Problem &p, hipStream_t s)
{
    const bool a_kc = !p.transA, b_kc = p.transB;
    if (a_kc) {
        if (b_kc) dispatch_vec<true, true>(p, s); else dispatch_vec<true, false>(p, s);
    } else {
        if (b_kc) dispatch_vec<false, true>(p, s); else dispatch_vec<false, false>(p, s);
    }
    return hipGetLastError();
}

}  // namespace gemmf32
