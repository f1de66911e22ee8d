// gemm_mfma_wide.hip -- FP32 GEMM on the CDNA4 matrix cores with a 256 x 256
// tile, for large products whose k is short enough (K <= 1024) that one
// running FP32 sum per output already meets the 1e-6 relative error bound.
//
// The method is the one of gemm_mfma.hip and of the course page "3 . La
// memoire partagee" (sections 3.2-3.4: a workgroup owns a tile of C, stages
// slices of A and B through shared memory, computes register tiles from it
// and moves along k), with a larger tile and a leaner loop:
//
//  * Tile: 256 x 256 of C per workgroup, 8 waves of 64 lanes, each a
//    64 x 128 register tile of 2 x 4 MFMA blocks of 32 x 32
//    (v_mfma_f32_32x32x2_f32).  Per flop it copies half the bytes into LDS
//    of a 128 x 128 tile and a third less than 256 x 128.  About 180
//    registers per lane and two 64 KB stage buffers: one workgroup per CU,
//    two waves per SIMD.
//  * Operands untransposed (A's stored rows run along k, B's along n), M and
//    N multiples of 256, K a multiple of 32, both operands 16-byte aligned
//    with leading dimensions that are multiples of 4 floats: every tile is
//    interior and every stage is one DMA copy.  The host checks all of this
//    (gemm_mfma_wide_fits); other problems go to the kernels of
//    gemm_mfma.hip.
//  * Staging: each 32-k stage is copied global -> LDS with
//    global_load_lds_dwordx4 one stage ahead into the other buffer (one
//    barrier per stage).  The buffer is picked at run time from the stage
//    parity, so the compiler keeps one set of fragment addresses instead of
//    one per buffer.
//  * Fragments: the k order inside a group of 8 k values is the one of
//    gemm_mfma.hip (lanes 0-31 take k = u, lanes 32-63 k = 4 + u for the
//    four MFMAs u of the group).  The fragments of group g + 1 are read while
//    group g's 32 MFMAs run, interleaved one LDS read per three MFMAs.
//  * Accumulation: one running sum per output.  The matrix core rounds once
//    per MFMA (two products), so for zero-mean data the relative error grows
//    like u * sqrt(K / 12) (u = 2^-24): 5.7e-7 at K = 1024, which is why
//    longer products stay on the chunked kernels (a 256 x 256 tile with
//    chunked sums does not fit the register file at speed: measured 136 vs
//    143 TFLOP/s unchunked on 4096^3).
//  * Launch order: the XCD-aware tile order of tile_common.hpp.
#include "tile_common.hpp"

namespace gemmf32 {
namespace {

typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kBM = 256, kBN = 256, kBK = 32;
constexpr int kWaves = 8, kThreads = 64 * kWaves;
constexpr int kFM = 2, kFN = 4;        // 32 x 32 blocks per wave: 64 x 128
constexpr int kAVec = kBK / 4;         // A stage: 256 rows (m) of 8 vectors (k)
constexpr int kBVec = kBN / 4;         // B stage: 32 rows (k) of 64 vectors (n)
constexpr int kAFloats = kBM * kBK, kBFloats = kBK * kBN;
constexpr int kStage = kAFloats + kBFloats;        // 16384 floats = 64 KB
constexpr int kAPieces = kAFloats / 256 / kWaves;  // 1 KB copies per wave per stage
constexpr int kBPieces = kBFloats / 256 / kWaves;
constexpr int kGroupM = 4;  // tile-rows per group of the launch order
constexpr int kWideMaxK = 1024;
constexpr int kWideMinTiles = 256;  // auto selection: at least one tile per CU
static_assert(kAPieces * kWaves * 256 == kAFloats && kBPieces * kWaves * 256 == kBFloats,
              "each stage splits into whole 1 KB copies per wave");

// 16-byte vector v of an A row r (8 vectors) sits in slot v ^ swz_a(r); of a
// B row r (64 vectors) in slot v ^ swz_b(r).  A fragment read takes row
// wm + 32 i + l32 and vector 2 g + half: the XOR spreads the 32 rows of a
// half-wave over all eight slots.  A B fragment read takes 32 consecutive
// floats of row k from lanes 0-31 and of row k + 4 from lanes 32-63; rows
// with bit 2 of k set are shifted by 8 vectors (32 floats), so the two
// halves of the wave hit disjoint banks.
__device__ __forceinline__ int swz_a(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int swz_b(int r) { return ((r >> 2) & 1) << 3; }

// Wait until at most N of this wave's vector-memory operations (the
// global -> LDS copies) are outstanding.  gfx9 encoding: vmcnt in bits 3:0
// and 15:14; expcnt and lgkmcnt left at their maxima.
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit count");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2, 2))) void
wide_kernel(int K, const float *__restrict__ A, int64_t lda, const float *__restrict__ B, int64_t ldb,
            float *__restrict__ C, int64_t ldc, int tiles_m, int tiles_n, int tile_base, int64_t stride_a,
            int64_t stride_b, int64_t stride_c, int64_t batch_base, const float *__restrict__ bias, int act)
{
    __shared__ __attribute__((aligned(1024))) float lds[2 * kStage];

    const int64_t bz = batch_base + blockIdx.y;
    A += bz * stride_a;
    B += bz * stride_b;
    C += bz * stride_c;
    int tm, tn;
    tile_of<kGroupM>(tile_base + int(blockIdx.x), tiles_m, tiles_n, tm, tn);
    const int m0 = tm * kBM, n0 = tn * kBN;

    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    const int wm = (wave / 2) * 64, wn = (wave % 2) * 128;
    const int half = lane / 32, l32 = lane % 32;

    // Byte offsets, from the stage's origin in global memory, of the vector
    // this lane copies in each of its wave's 1 KB pieces.  Piece q of wave w
    // fills LDS vectors s = (w * pieces + q) * 64 + lane; LDS slot s % rowlen
    // of row s / rowlen holds the logical vector slot ^ swz(row).
    uint32_t oa[kAPieces], ob[kBPieces];
#pragma unroll
    for (int q = 0; q < kAPieces; ++q) {
        const int s = (wave * kAPieces + q) * 64 + lane;
        const int r = s / kAVec, v = (s % kAVec) ^ swz_a(r);
        oa[q] = uint32_t((int64_t(r) * lda + 4 * v) * 4);
    }
#pragma unroll
    for (int q = 0; q < kBPieces; ++q) {
        const int s = (wave * kBPieces + q) * 64 + lane;
        const int r = s / kBVec, v = (s % kBVec) ^ swz_b(r);
        ob[q] = uint32_t((int64_t(r) * ldb + 4 * v) * 4);
    }
    const char *ga = reinterpret_cast<const char *>(A + int64_t(m0) * lda);
    const char *gb = reinterpret_cast<const char *>(B + n0);
    auto copy_stage = [&](float *dst, int st) {
        const char *sa = ga + int64_t(st) * kBK * 4;
        const char *sb = gb + int64_t(st) * kBK * ldb * 4;
#pragma unroll
        for (int q = 0; q < kAPieces; ++q)
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const float *>(sa + oa[q]),
                                             dst + (wave * kAPieces + q) * 256, 16, 0, 0);
#pragma unroll
        for (int q = 0; q < kBPieces; ++q)
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const float *>(sb + ob[q]),
                                             dst + kAFloats + (wave * kBPieces + q) * 256, 16, 0, 0);
    };

    // Fragment addresses (floats from a stage's origin) for k group g.
    // A: row wm + l32 (block i adds 32 rows), logical vector 2 g + half.
    // B: rows k = 8 g + 4 half + u, column p = wn + 32 j + l32.  Its vector
    // p / 4 has bits 3-4 equal to j (wn / 4 is 0 or 32, l32 / 4 < 8), and
    // swz_b(k) = 8 * half, so block j of this lane sits at float
    // wn + l32 + 32 * (j ^ half) of the row.
    int a_off[4], b_off[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int r = wm + l32;
        a_off[g] = 4 * (r * kAVec + ((2 * g + half) ^ swz_a(r)));
        b_off[g] = kAFloats + (8 * g + 4 * half) * kBN + wn + l32;
    }
    int jt[kFN];
#pragma unroll
    for (int j = 0; j < kFN; ++j) jt[j] = 32 * (j ^ half);

    v16f acc[kFM][kFN];
#pragma unroll
    for (int i = 0; i < kFM; ++i)
#pragma unroll
        for (int j = 0; j < kFN; ++j) acc[i][j] = v16f{0.0f};

    const int stages = K / kBK;
    copy_stage(lds, 0);
    for (int st = 0; st < stages; ++st) {
        // This wave's copies of stage st have landed; after the barrier
        // everyone's have, and every wave has finished reading the other
        // buffer (stage st - 1), which the next copy overwrites.
        wait_vm<0>();
        __syncthreads();
        const float *c = lds + (st & 1) * kStage;
        if (st + 1 < stages) copy_stage(lds + ((st + 1) & 1) * kStage, st + 1);

        v4f fa[2][kFM], fb[2][kFN];
        auto read = [&](int g, int sl) {
#pragma unroll
            for (int i = 0; i < kFM; ++i) fa[sl][i] = *reinterpret_cast<const v4f *>(c + a_off[g] + i * 32 * kBK);
#pragma unroll
            for (int j = 0; j < kFN; ++j) {
                const float *col = c + b_off[g] + jt[j];
                fb[sl][j] = v4f{col[0], col[kBN], col[2 * kBN], col[3 * kBN]};
            }
        };
        read(0, 0);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int sl = g & 1;
            if (g + 1 < 4) read(g + 1, sl ^ 1);
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int i = 0; i < kFM; ++i)
#pragma unroll
                    for (int j = 0; j < kFN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[sl][i][u], fb[sl][j][u], acc[i][j], 0, 0, 0);
            if (g + 1 < 4) {
                // the next group's 10 LDS reads (2 of A, 4 x 2 of B), one
                // per 3 of this group's 32 MFMAs
#pragma unroll
                for (int q = 0; q < 10; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            }
        }
    }

    // Epilogue: lane l of a 32 x 32 block holds column l % 32 and, in slot
    // v, row 8 * (v / 4) + 4 * (l / 32) + v % 4.  Optional bias[column] and
    // GELU, then a streaming store (C is written once).
#pragma unroll
    for (int i = 0; i < kFM; ++i)
#pragma unroll
        for (int j = 0; j < kFN; ++j) {
            const int col = n0 + wn + 32 * j + l32;
            const float bj = bias != nullptr ? bias[col] : 0.0f;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = m0 + wm + 32 * i + 8 * (v / 4) + 4 * half + (v % 4);
                float x = acc[i][j][v] + bj;
                if (act == 1) x = gelu(x);
                __builtin_nontemporal_store(x, &C[int64_t(row) * ldc + col]);
            }
        }
}

// Every DMA offset of a stage (rows x ld floats plus one row) fits in 32 bits.
bool offsets_fit(int rows, int64_t ld) { return (int64_t(rows) * ld + ld) * 4 < (int64_t(1) << 32); }

}  // namespace

bool mfma_wide_fits(const Problem &p)
{
    const bool batched = p.batch > 1;
    return !p.transA && !p.transB && p.k_total == 0 && p.M % kBM == 0 && p.N % kBN == 0 && p.K % kBK == 0 &&
           p.K >= kBK && p.K <= kWideMaxK && vec4_ok(p.A, p.lda) && vec4_ok(p.B, p.ldb) &&
           (!batched || (p.stride_a % 4 == 0 && p.stride_b % 4 == 0)) && offsets_fit(kBM, p.lda) &&
           offsets_fit(kBK, p.ldb) && int64_t(p.M / kBM) * (p.N / kBN) <= kMaxGrid;
}

bool mfma_wide_preferred(const Problem &p)
{
    return mfma_wide_fits(p) && int64_t(p.M / kBM) * (p.N / kBN) * p.batch >= kWideMinTiles;
}

hipError_t launch_mfma_wide(const Problem &p, hipStream_t s)
{
    const int tiles_m = p.M / kBM, tiles_n = p.N / kBN;
    for (int64_t b0 = 0; b0 < p.batch; b0 += kMaxGridY) {
        const int64_t nb = p.batch - b0 < kMaxGridY ? p.batch - b0 : kMaxGridY;
        wide_kernel<<<dim3(unsigned(tiles_m * tiles_n), unsigned(nb)), dim3(kThreads), 0, s>>>(
            p.K, p.A, p.lda, p.B, p.ldb, p.C, p.ldc, tiles_m, tiles_n, 0, p.stride_a, p.stride_b, p.stride_c, b0,
            p.bias, p.act);
    }
    return hipGetLastError();
}

}  // namespace gemmf32
