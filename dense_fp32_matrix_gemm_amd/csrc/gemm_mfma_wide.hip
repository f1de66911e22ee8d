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
//  * Any transposes (one instantiation per layout), M and N multiples of
//    256, K a multiple of 32, both operands 16-byte aligned with leading
//    dimensions that are multiples of 4 floats: every tile is interior and
//    every stage is one DMA copy.  The host checks all of this
//    (mfma_wide_fits); other problems go to the kernels of gemm_mfma.hip.
//  * Staging: each 32-k stage is copied global -> LDS with buffer loads
//    into LDS (copy16_to_lds) one stage ahead into the other buffer (one
//    barrier per stage).  The buffer is picked at run time from the stage
//    parity, so the compiler keeps one set of fragment addresses instead of
//    one per buffer.
//  * Fragments: the k order inside a group of 8 k values is the one of
//    gemm_mfma.hip (lanes 0-31 take k = u, lanes 32-63 k = 4 + u for the
//    four MFMAs u of the group).  The fragments of group g + 1 are read while
//    group g's 32 MFMAs run, the LDS reads spread evenly between them.
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
constexpr int kP = 256;                // extent of each operand's tile along m or n
static_assert(kBM == kP && kBN == kP, "both operands' tiles are 256 x 32");
constexpr int kAFloats = kBM * kBK, kBFloats = kBK * kBN;
constexpr int kStage = kAFloats + kBFloats;        // 16384 floats = 64 KB
constexpr int kAPieces = kAFloats / 256 / kWaves;  // 1 KB copies per wave per stage
constexpr int kBPieces = kBFloats / 256 / kWaves;
constexpr int kGroupM = 4;  // tile-rows per group of the launch order
constexpr int kWideMaxK = 1024;
constexpr int kWideMinTiles = kCUs;  // auto selection: at least one tile per CU
// Products of at most kShortStages stages keep every stage in LDS at once
// and store the tile in kShortParts column parts (see the kernel).
constexpr int kShortStages = 2;
#ifndef GEMM_WIDE_SHORT_PARTS
#define GEMM_WIDE_SHORT_PARTS 4
#endif
constexpr int kShortParts = GEMM_WIDE_SHORT_PARTS;
#ifndef GEMM_WIDE_SHORT_CHAINS
#define GEMM_WIDE_SHORT_CHAINS 2
#endif
constexpr int kShortChains = GEMM_WIDE_SHORT_CHAINS;
static_assert(4 % kShortChains == 0, "chains divide the 4 MFMAs of a k group");
static_assert(kFN % kShortParts == 0, "parts are whole column blocks");
static_assert(kAPieces * kWaves * 256 == kAFloats && kBPieces * kWaves * 256 == kBFloats,
              "each stage splits into whole 1 KB copies per wave");

// One operand's stage tile in LDS: the 256 rows (or columns) of C it feeds
// times 32 k, in one of two layouts.
//
// KC (the stored rows run along k: A untransposed, B transposed): 256 rows
// of 8 16-byte vectors; vector v of row r sits in slot v ^ swz(r).  A
// fragment read takes row p + l32 and vector 2 g + half, one 16-byte LDS
// read per lane; the XOR spreads the 32 rows of a half-wave over all eight
// slots.  Block b (32 rows further) is 32 * 32 floats further.
//
// Not KC (the stored rows run along m or n): 32 rows (k) of 64 vectors;
// rows with bit 2 of k set have their vectors shifted by 8 (32 floats), so
// lanes 0-31, reading 32 consecutive floats of row k, and lanes 32-63,
// reading row k + 4, hit disjoint banks.  A fragment is four rows k .. k + 3
// of column p + 32 b + l32 with k = 8 g + 4 half.  For p a multiple of 64
// and b < 4, the column's vector index has bits 3-4 equal to b and the
// shift flips bit 3 exactly when half = 1, so block b of this lane sits at
// float p + l32 + 32 * (b ^ half) of the row.
template <bool KC>
struct WideOp;

template <>
struct WideOp<true> {
    static constexpr int reads = 1;  // LDS read instructions per fragment
    __device__ static int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }
    // Byte offset, from the stage's origin in global memory, of LDS vector s.
    __device__ static uint32_t src(int s, int64_t ld)
    {
        const int r = s / (kBK / 4), v = (s % (kBK / 4)) ^ swz(r);
        return uint32_t((int64_t(r) * ld + 4 * v) * 4);
    }
    __device__ static const char *origin(const float *X, int p0, int64_t ld)
    {
        return reinterpret_cast<const char *>(X + int64_t(p0) * ld);
    }
    __device__ static int64_t stage_bytes(int64_t) { return int64_t(kBK) * 4; }
    __device__ static int frag(int p, int l32, int half, int g)
    {
        const int r = p + l32;
        return 4 * (r * (kBK / 4) + ((2 * g + half) ^ swz(r)));
    }
    __device__ static int block(int b, int) { return b * 32 * kBK; }
    __device__ static v4f read(const float *t) { return *reinterpret_cast<const v4f *>(t); }
};

template <>
struct WideOp<false> {
    static constexpr int reads = 2;  // two ds_read2 of rows k, k + 1 and k + 2, k + 3
    __device__ static int swz(int r) { return ((r >> 2) & 1) << 3; }
    __device__ static uint32_t src(int s, int64_t ld)
    {
        const int r = s / (kP / 4), v = (s % (kP / 4)) ^ swz(r);
        return uint32_t((int64_t(r) * ld + 4 * v) * 4);
    }
    __device__ static const char *origin(const float *X, int p0, int64_t)
    {
        return reinterpret_cast<const char *>(X + p0);
    }
    __device__ static int64_t stage_bytes(int64_t ld) { return int64_t(kBK) * ld * 4; }
    __device__ static int frag(int p, int l32, int half, int g) { return (8 * g + 4 * half) * kP + p + l32; }
    __device__ static int block(int b, int half) { return 32 * (b ^ half); }
    __device__ static v4f read(const float *t) { return v4f{t[0], t[kP], t[2 * kP], t[3 * kP]}; }
};

template <bool A_KC, bool B_KC>
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

    using OA = WideOp<A_KC>;
    using OB = WideOp<B_KC>;
    // Byte offsets, from the stage's origin in global memory, of the vector
    // this lane copies in each of its wave's 1 KB pieces.  Piece q of wave w
    // fills LDS vectors s = (w * pieces + q) * 64 + lane.
    uint32_t oa[kAPieces], ob[kBPieces];
#pragma unroll
    for (int q = 0; q < kAPieces; ++q) oa[q] = OA::src((wave * kAPieces + q) * 64 + lane, lda);
#pragma unroll
    for (int q = 0; q < kBPieces; ++q) ob[q] = OB::src((wave * kBPieces + q) * 64 + lane, ldb);
    const char *ga = OA::origin(A, m0, lda);
    const char *gb = OB::origin(B, n0, ldb);
    const int64_t a_step = OA::stage_bytes(lda), b_step = OB::stage_bytes(ldb);
    // The copies' LDS destination goes to M0, a scalar register: take the
    // wave index from one too, so it is not re-read from a vector register
    // for every copy (the mask states its range, which the compiler needs
    // to see that a copy does not write the buffer being read).
    const int wave_c = __builtin_amdgcn_readfirstlane(wave) & (kWaves - 1);
    auto copy_stage = [&](float *dst, int st) {
        const char *sa = ga + st * a_step;
        const char *sb = gb + st * b_step;
        if (GEMM_LDS_POISON) {
#pragma unroll
            for (int q = 0; q < kAPieces; ++q) poison16(dst + (wave * kAPieces + q) * 256 + 4 * lane);
#pragma unroll
            for (int q = 0; q < kBPieces; ++q) poison16(dst + kAFloats + (wave * kBPieces + q) * 256 + 4 * lane);
            poison_wait();
        }
#pragma unroll
        for (int q = 0; q < kAPieces; ++q) copy16_to_lds(dst + (wave_c * kAPieces + q) * 256, sa, oa[q]);
#pragma unroll
        for (int q = 0; q < kBPieces; ++q) copy16_to_lds(dst + kAFloats + (wave_c * kBPieces + q) * 256, sb, ob[q]);
    };

    // Fragment addresses (floats from a stage's origin) for k group g and
    // block 0 of this wave (wm and wn are multiples of 64), and the offsets
    // of its other blocks.
    int a_off[4], b_off[4], it[kFM], jt[kFN];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        a_off[g] = OA::frag(wm, l32, half, g);
        b_off[g] = kAFloats + OB::frag(wn, l32, half, g);
    }
#pragma unroll
    for (int i = 0; i < kFM; ++i) it[i] = OA::block(i, half);
#pragma unroll
    for (int j = 0; j < kFN; ++j) jt[j] = OB::block(j, half);

    const int stages = K / kBK;
    if (stages <= kShortStages) {
        // Short k (32 or 64: the attention scores over a head of 64): both
        // stages are copied at once, and the wave's 64 x 128 tile is then
        // computed in kShortParts parts of whole column blocks.  The stores
        // of part q - 1 are issued a few at a time between the MFMAs of part
        // q, so the output leaves while the products run; with only two
        // stages per tile, storing the whole tile at the end would follow
        // the products with nothing to overlap it (all workgroups start and
        // finish together).
        copy_stage(lds, 0);
        if (stages > 1) copy_stage(lds + kStage, 1);
        wait_vm<0>();
        __syncthreads();
        constexpr int kCols = kFN / kShortParts;   // 32-column blocks per part
        constexpr int kStores = kFM * kCols * 16;  // store instructions per part
        constexpr int kSlots = kShortStages * 4;   // k groups per part
        constexpr int kPer = (kStores + kSlots - 1) / kSlots;
        v16f done[kFM][kCols];  // the previous part, bias and activation applied
        auto put = [&](int q, int s) {
            const int i = s / (16 * kCols), j = (s / 16) % kCols, v = s % 16;
            const int col = n0 + wn + 32 * (q * kCols + j) + l32;
            const int row = m0 + wm + 32 * i + 8 * (v / 4) + 4 * half + (v % 4);
            __builtin_nontemporal_store(done[i][j][v], &C[int64_t(row) * ldc + col]);
        };
#pragma unroll
        for (int q = 0; q < kShortParts; ++q) {
            // kShortChains partial sums per block (MFMA u of each k group
            // feeds sum u % kShortChains), so a wave keeps kShortChains * kFM
            // * kCols independent MFMA chains in flight
            v16f part[kFM][kCols][kShortChains];
#pragma unroll
            for (int i = 0; i < kFM; ++i)
#pragma unroll
                for (int j = 0; j < kCols; ++j)
#pragma unroll
                    for (int c = 0; c < kShortChains; ++c) part[i][j][c] = v16f{0.0f};
#pragma unroll
            for (int st = 0; st < kShortStages; ++st) {
                const float *c = lds + st * kStage;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    if (st < stages) {
                        v4f fa[kFM], fb[kCols];
#pragma unroll
                        for (int i = 0; i < kFM; ++i) fa[i] = OA::read(c + a_off[g] + it[i]);
#pragma unroll
                        for (int j = 0; j < kCols; ++j) fb[j] = OB::read(c + b_off[g] + jt[q * kCols + j]);
#pragma unroll
                        for (int u = 0; u < 4; ++u)
#pragma unroll
                            for (int i = 0; i < kFM; ++i)
#pragma unroll
                                for (int j = 0; j < kCols; ++j)
                                    part[i][j][u % kShortChains] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                                        fa[i][u], fb[j][u], part[i][j][u % kShortChains], 0, 0, 0);
                    }
                    // this slot's share of the previous part's stores (all of
                    // them by the last slot, whether or not it computed)
                    if (q > 0) {
#pragma unroll
                        for (int t = 0; t < kPer; ++t) {
                            const int s = (st * 4 + g) * kPer + t;
                            if (s < kStores) put(q - 1, s);
                        }
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < kCols; ++j) {
                const int col = n0 + wn + 32 * (q * kCols + j) + l32;
                const float bj = bias != nullptr ? bias[col] : 0.0f;
#pragma unroll
                for (int i = 0; i < kFM; ++i)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        float x = part[i][j][0][v];
#pragma unroll
                        for (int c = 1; c < kShortChains; ++c) x += part[i][j][c][v];
                        x += bj;
                        if (act == 1) x = gelu(x);
                        done[i][j][v] = x;
                    }
            }
        }
#pragma unroll
        for (int s = 0; s < kStores; ++s) put(kShortParts - 1, s);
        return;
    }

    v16f acc[kFM][kFN];
#pragma unroll
    for (int i = 0; i < kFM; ++i)
#pragma unroll
        for (int j = 0; j < kFN; ++j) acc[i][j] = v16f{0.0f};

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
            for (int i = 0; i < kFM; ++i) fa[sl][i] = OA::read(c + a_off[g] + it[i]);
#pragma unroll
            for (int j = 0; j < kFN; ++j) fb[sl][j] = OB::read(c + b_off[g] + jt[j]);
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
                // the next group's LDS reads spread evenly over this
                // group's 32 MFMAs
                constexpr int kMfma = 4 * kFM * kFN;
                constexpr int kReads = kFM * OA::reads + kFN * OB::reads;
                constexpr int per = kMfma / kReads;
#pragma unroll
                for (int q = 0; q < kReads; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, per, 0);
                }
                if (kMfma > per * kReads) __builtin_amdgcn_sched_group_barrier(0x008, kMfma - per * kReads, 0);
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
    // rows of one stage as stored: 256 when k runs along the rows, else 32
    const int a_rows = p.transA ? kBK : kBM, b_rows = p.transB ? kBN : kBK;
    return p.k_total == 0 && p.M % kBM == 0 && p.N % kBN == 0 && p.K % kBK == 0 && p.K >= kBK &&
           p.K <= kWideMaxK && vec4_ok(p.A, p.lda) && vec4_ok(p.B, p.ldb) &&
           (!batched || (p.stride_a % 4 == 0 && p.stride_b % 4 == 0)) && offsets_fit(a_rows, p.lda) &&
           offsets_fit(b_rows, p.ldb) && int64_t(p.M / kBM) * (p.N / kBN) <= kMaxGrid;
}

bool mfma_wide_preferred(const Problem &p)
{
    return mfma_wide_fits(p) && int64_t(p.M / kBM) * (p.N / kBN) * p.batch >= kWideMinTiles;
}

namespace {
template <bool A_KC, bool B_KC>
void launch_layout(const Problem &p, hipStream_t s)
{
    const int tiles_m = p.M / kBM, tiles_n = p.N / kBN;
    for (int64_t b0 = 0; b0 < p.batch; b0 += kMaxGridY) {
        const int64_t nb = p.batch - b0 < kMaxGridY ? p.batch - b0 : kMaxGridY;
        wide_kernel<A_KC, B_KC><<<dim3(unsigned(tiles_m * tiles_n), unsigned(nb)), dim3(kThreads), 0, s>>>(
            p.K, p.A, p.lda, p.B, p.ldb, p.C, p.ldc, tiles_m, tiles_n, 0, p.stride_a, p.stride_b, p.stride_c, b0,
            p.bias, p.act);
    }
}
}  // namespace

hipError_t launch_mfma_wide(const Problem &p, hipStream_t s)
{
    // A is k-contiguous when untransposed; B when transposed.
    if (!p.transA)
        p.transB ? launch_layout<true, true>(p, s) : launch_layout<true, false>(p, s);
    else
        p.transB ? launch_layout<false, true>(p, s) : launch_layout<false, false>(p, s);
    return hipGetLastError();
}

}  // namespace gemmf32
