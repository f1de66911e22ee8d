// gemm_mfma.hip -- FP32 GEMM on the CDNA4 matrix cores (v_mfma_f32_32x32x2_f32).
//
// The structure is the one the course page "3 . La memoire partagee" builds
// in sections 3.2-3.4: a block of threads owns a tile of C, copies slices of
// A and B into LDS with coalesced loads, synchronises, computes from LDS
// into register tiles, and moves on along k.  What is specific to gfx950:
//
//  * Tile: 128 x 128 of C per workgroup of 256 lanes (4 waves of 64), each
//    wave a 64 x 64 register tile made of 2 x 2 MFMA blocks of 32 x 32.  The
//    register tile is the page's "third level of tiling" with the outer
//    product done by the matrix core: one v_mfma_f32_32x32x2_f32 is a
//    rank-2 update of a 32 x 32 block, 4096 flops per wave instruction.
//  * Staging: each K stage (BK = 32) is loaded with 16-byte vector loads
//    (each row segment of a tile is contiguous in memory), held in
//    registers while the matrix core works on the previous stage, then
//    written to the other of two LDS buffers: one barrier per stage instead
//    of the page's two, because the buffer being written is never the one
//    being read (the double buffering of the cuda-oxide book's summary).
//  * LDS layout: a tile whose rows run along k (A untransposed, B
//    transposed) is stored [rows][32 + 4]; a tile whose rows run along m or
//    n is stored [32][rows + 8].  The padding is the page's section 3.6
//    remedy sized for 16-byte and 4-byte LDS reads of 64-lane waves.
//  * Fragment order in k: inside each group of 8 k values, lanes 0-31 feed
//    the MFMA k = 0 slot with k = s and lanes 32-63 the k = 1 slot with
//    k = 4 + s for the four MFMAs s = 0..3.  Both operands use the same map,
//    so every pair (a_ik, b_kj) meets exactly once, and a k-contiguous
//    operand is read with one 16-byte LDS read per lane per 4 MFMAs.
//  * Accumulation: each stage's 32 k values are summed into a fresh MFMA
//    accumulator (the first MFMA of the stage takes a zero addend) and then
//    added into the running tile, which keeps FP32 rounding error flat in K.
//  * Edges: a workgroup whose tile lies inside M x N and a stage inside K
//    uses unpredicated loads; otherwise loads are predicated per element and
//    out-of-range elements are zero (section 3.3's kernel assumes multiples;
//    the zero fill makes any M, N, K exact).  Stores are predicated.
//    Barriers are outside every data-dependent branch.
//  * Launch order: workgroups are dealt round-robin to the 8 XCDs, each with
//    its own L2.  The tile index is remapped so that each XCD receives a
//    contiguous run of tiles, and that run is walked GROUP_M tile-rows at a
//    time, so co-resident workgroups of one XCD share A and B panels in L2.
#include "tile_common.hpp"

namespace gemmf32 {
namespace {

typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;      // 4 waves
constexpr int kWave = 64;
constexpr int BM = 128, BN = 128;  // C tile per workgroup
constexpr int BK = 32;             // k per stage (and per accumulation chunk)
constexpr int kBlk = 32;           // MFMA output block edge
constexpr int WM = 64, WN = 64;    // C tile per wave (2 x 2 waves)
constexpr int FM = WM / kBlk, FN = WN / kBlk;
constexpr int kPadK = 4;           // padding (floats) of a k-contiguous LDS row
constexpr int kPadMN = 8;          // padding (floats) of an m/n-contiguous LDS row
constexpr int kGroupM = 8;         // tile-rows per group in the launch order

// LDS tile of one operand: P = extent along m (or n); KC = rows run along k.
template <int P, bool KC>
struct Tile {
    static constexpr int rows = KC ? P : BK;  // rows of the stored slice
    static constexpr int cols = KC ? BK : P;  // contiguous extent
    static constexpr int ld = cols + (KC ? kPadK : kPadMN);
    static constexpr int floats = rows * ld;
    using Load = Slice<rows, cols, kThreads>;
    static constexpr int per_thread = Load::per_thread;

    // Registers -> LDS, same slice-to-thread map as the load.
    __device__ static __forceinline__ void store(float *lds, const v4f (&reg)[per_thread])
    {
#pragma unroll
        for (int q = 0; q < per_thread; ++q)
            *reinterpret_cast<v4f *>(lds + Load::row(q) * ld + Load::col(q)) = reg[q];
    }

    // The four k values (one per MFMA u = 0..3) this lane feeds for k group
    // g at m (or n) position p of the tile.  Lane half h covers k = 8g + 4h + u.
    __device__ static __forceinline__ v4f fragment(const float *lds, int p, int g, int h)
    {
        if (KC) {
            return *reinterpret_cast<const v4f *>(lds + p * ld + 8 * g + 4 * h);
        } else {
            const float *col = lds + (8 * g + 4 * h) * ld + p;
            return v4f{col[0], col[ld], col[2 * ld], col[3 * ld]};
        }
    }
};

template <bool A_KC, bool B_KC, bool VEC>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(2, 2))) void
mfma_kernel(int M, int N, int K, const float *__restrict__ A, int64_t lda,
            const float *__restrict__ B, int64_t ldb, float *__restrict__ C, int64_t ldc,
            int tiles_m, int tiles_n)
{
    using TA = Tile<BM, A_KC>;
    using TB = Tile<BN, B_KC>;
    constexpr int kBuf = TA::floats + TB::floats;  // one stage: A tile then B tile
    __shared__ __attribute__((aligned(16))) float smem[2 * kBuf];

    const int tiles = tiles_m * tiles_n;
    for (int t = blockIdx.x; t < tiles; t += gridDim.x) {
        int tm, tn;
        tile_of<kGroupM>(t, tiles_m, tiles_n, tm, tn);
        const int m0 = tm * BM, n0 = tn * BN;
        const bool inside = (m0 + BM <= M) && (n0 + BN <= N);

        const Operand opa{A, lda, A_KC ? M : K, A_KC ? K : M};
        const Operand opb{B, ldb, B_KC ? N : K, B_KC ? K : N};
        // stored origin of the stage starting at k: (row, col)
        auto a_r = [&](int k) { return A_KC ? m0 : k; };
        auto a_c = [&](int k) { return A_KC ? k : m0; };
        auto b_r = [&](int k) { return B_KC ? n0 : k; };
        auto b_c = [&](int k) { return B_KC ? k : n0; };

        v4f ra[TA::per_thread], rb[TB::per_thread];
        auto load = [&](int k) {
            if (inside && k + BK <= K) {
                TA::Load::template load<false, VEC>(opa, a_r(k), a_c(k), ra);
                TB::Load::template load<false, VEC>(opb, b_r(k), b_c(k), rb);
            } else {
                TA::Load::template load<true, VEC>(opa, a_r(k), a_c(k), ra);
                TB::Load::template load<true, VEC>(opb, b_r(k), b_c(k), rb);
            }
        };

        const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
        const int wm = (wave / 2) * WM, wn = (wave % 2) * WN;
        const int half = lane / 32, l32 = lane % 32;

        v16f acc[FM][FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = v16f{0.0f};

        const int stages = ceil_div(K, BK);
        load(0);
        TA::store(smem, ra);
        TB::store(smem + TA::floats, rb);
        __syncthreads();

        for (int s = 0; s < stages; ++s) {
            const bool next = s + 1 < stages;
            if (next) load((s + 1) * BK);  // in flight while the matrix core works

            const float *la = smem + (s & 1) * kBuf;
            const float *lb = la + TA::floats;
            v16f part[FM][FN];
#pragma unroll
            for (int g = 0; g < BK / 8; ++g) {
                v4f fa[FM], fb[FN];
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    fa[i] = TA::fragment(la, wm + i * kBlk + l32, g, half);
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    fb[j] = TB::fragment(lb, wn + j * kBlk + l32, g, half);
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int i = 0; i < FM; ++i)
#pragma unroll
                        for (int j = 0; j < FN; ++j)
                            part[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                                fa[i][u], fb[j][u], (g == 0 && u == 0) ? v16f{0.0f} : part[i][j],
                                0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] += part[i][j];

            if (next) {
                float *wa = smem + ((s + 1) & 1) * kBuf;
                TA::store(wa, ra);
                TB::store(wa + TA::floats, rb);
            }
            __syncthreads();
        }

        // Epilogue.  Lane l of a 32 x 32 block holds column l % 32 and, in
        // accumulator slot v, row 8 * (v / 4) + 4 * (l / 32) + v % 4.
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int col = n0 + wn + j * kBlk + l32;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int row = m0 + wm + i * kBlk + 8 * (v / 4) + 4 * half + (v % 4);
                    if (inside || (row < M && col < N)) C[int64_t(row) * ldc + col] = acc[i][j][v];
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
    mfma_kernel<A_KC, B_KC, VEC><<<grid, dim3(kThreads), 0, s>>>(
        p.M, p.N, p.K, p.A, p.lda, p.B, p.ldb, p.C, p.ldc, tiles_m, tiles_n);
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

hipError_t launch_mfma(const Problem &p, hipStream_t s)
{
    // A is k-contiguous when untransposed; B when transposed.
    const bool a_kc = !p.transA, b_kc = p.transB;
    if (a_kc) {
        if (b_kc) dispatch_vec<true, true>(p, s); else dispatch_vec<true, false>(p, s);
    } else {
        if (b_kc) dispatch_vec<false, true>(p, s); else dispatch_vec<false, false>(p, s);
    }
    return hipGetLastError();
}

}  // namespace gemmf32
