// gemm_mfma.hip -- FP32 GEMM on the CDNA4 matrix cores (v_mfma_f32_32x32x2_f32).
//
// The structure is the one the course page "3 . La memoire partagee" builds
// in sections 3.2-3.4: a block of threads owns a tile of C, copies slices of
// A and B into LDS with coalesced loads, synchronises, computes from LDS
// into register tiles, and moves on along k.  What is specific to gfx950:
//
//  * Tile: 128 x 128 of C per workgroup.  The default configuration has 8
//    waves of 64 lanes, each wave a 32 x 64 register tile of 1 x 2 MFMA
//    blocks of 32 x 32 (the page's "third level of tiling", with the outer
//    product done by the matrix core: one v_mfma_f32_32x32x2_f32 is a rank-2
//    update of a 32 x 32 block, 4096 flops per wave instruction).  At about
//    128 registers per lane, two workgroups (16 waves) share a CU, four
//    waves per SIMD to hide LDS and barrier latency.  Large grids with long
//    k take a 256 x 128 tile (one workgroup per CU), small grids a 64 x 64
//    tile whose k groups are split over two slices of waves; the
//    configurations and where each is used are listed below the kernel.
//  * Staging, interior tiles: each K stage (BK = 32; 16, 64 or 128 in some
//    configurations) is copied from global memory straight into LDS with
//    buffer loads into LDS (buffer_load_dwordx4 ... lds on a raw descriptor
//    of the stage's origin; each wave instruction moves 64 x 16 bytes; no
//    registers, no LDS write instructions), issued a stage ahead into
//    another LDS buffer, so one barrier per stage suffices (the double
//    buffering of the cuda-oxide book's summary; the page's second barrier
//    is not needed because the buffer being filled is never the one being
//    read).
//  * Staging, edge tiles and the last partial stage: on the small tiles the
//    copies go on by DMA with the buffer descriptor's range check stopping
//    them at the end of each operand's storage, and values past K are
//    replaced by zero in the fragments; elsewhere 16-byte (or scalar) loads
//    into registers with every element predicated, zero outside the matrix
//    (section 3.3's kernel assumes tile multiples), written to LDS in the
//    same layout.  Stores to C are predicated.  Barriers are outside every
//    data-dependent branch.
//  * LDS layout: unpadded, with an XOR swizzle of the 16-byte vectors in
//    each row (the alternative to padding named in section 3.6): a DMA
//    instruction writes 1 KB contiguously, so padding is not possible, and
//    the swizzle keeps the fragment reads free of bank conflicts.
//  * Fragment order in k: inside each group of 8 k values, lanes 0-31 feed
//    the MFMA k = 0 slot with k = u and lanes 32-63 the k = 1 slot with
//    k = 4 + u for the four MFMAs u = 0..3.  Both operands use the same map,
//    so every pair (a_ik, b_kj) meets exactly once, and a k-contiguous
//    operand is read with one 16-byte LDS read per lane per 4 MFMAs.
//  * Accumulation: each run of 128-256 k values (per configuration) is
//    summed into a fresh MFMA accumulator (the first MFMA of the run takes a
//    zero addend) and then added into the running tile.  The matrix core
//    adds one product at a time in FP32, so without this the relative error
//    of a K = 8192 product grows past 1e-6; with it the error stays near
//    2.5e-7.  Longer runs mean fewer folds (each one drains the wave's MFMA
//    chain) at a small cost in accuracy.
//  * Launch order: workgroups are dealt round-robin to the 8 XCDs, each with
//    its own L2.  The tile index is remapped so that each XCD receives a
//    contiguous run of tiles, and that run is walked GROUP_M tile-rows at a
//    time, so co-resident workgroups of one XCD share A and B panels in L2.
#include "tile_common.hpp"


namespace gemmf32 {
namespace {

template <bool V>
struct Bool {
    static constexpr bool value = V;
};
template <int V>
struct Int {
    static constexpr int value = V;
};
using Yes = Bool<true>;
using No = Bool<false>;

// f(Int<0>{}), f(Int<1>{}), ..., f(Int<N-1>{}): a loop unrolled with the
// index as a compile-time constant.
template <int N, int I = 0, class F>
__device__ __forceinline__ void unroll_for(F &&f)
{
    if constexpr (I < N) {
        f(Int<I>{});
        unroll_for<N, I + 1>(f);
    }
}

typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;
constexpr int kBlk = 32;  // MFMA output block edge

// A tile configuration: BM x BN of C per workgroup, BK k per stage (and per
// accumulation chunk), WAVES_M x WAVES_N waves each owning a
// (BM/WAVES_M) x (BN/WAVES_N) register tile of 32 x 32 MFMA blocks, WPE
// waves per SIMD requested from the register allocator, GROUP_M tile-rows
// per group in the launch order, and WRITE_G, the k group of a stage after
// whose fragment reads register-staged data for the next stage is written
// to LDS (BK / 8 means after the last group), and CHAINS, the number of
// independent partial sums each block keeps within a stage (MFMA u of a k
// group feeds chain u % CHAINS).  One chain suffices when a wave owns
// several blocks; a wave with a single block needs more than one to keep
// consecutive MFMAs independent.  KSPLIT > 1 splits every stage's k groups
// over KSPLIT slices of WAVES_M x WAVES_N waves (slice s takes groups s,
// s + KSPLIT, ...); each slice accumulates its own partial tile and the
// slices are summed through LDS at the end.  It gives small grids more
// waves per SIMD without any memory outside the output.  NBUF stage
// buffers let the copy of stage s + NBUF - 1 run while stage s is computed;
// FOLD stages form one accumulation chunk on that path (0: no chunks, one
// running accumulator; only the unchunked ablation builds use it, since it
// does not meet the 1e-6 relative error bound at K = 4096).  PREFETCH reads the
// LDS fragments of the next k group before the current group's MFMAs
// (faster with one k-slice; slower when two slices already interleave).
// PRIO raises a wave's issue priority while it issues its MFMAs, so that
// waves feeding the matrix core are preferred over waves copying or waiting.
// STAGGER (copy path): the second half of the waves issues its share of the
// next stage's copies after the fragment reads of k group WRITE_G instead of
// right after the barrier, so the two waves of a SIMD do not both stall on
// copy issue at the same time.  CROSS (rings of three or more buffers with
// prefetch): each barrier also certifies the stage after the one it starts,
// and a stage reads the next stage's first fragments before its last MFMAs.
template <int BM_, int BN_, int BK_, int WAVES_M, int WAVES_N, int WPE_, int GROUP_M_,
          int WRITE_G_, int CHAINS_, int KSPLIT_, int NBUF_, int FOLD_, int PREFETCH_, int PRIO_ = 0,
          int STAGGER_ = 0, int CROSS_ = 0>
struct Config {
    static constexpr int BM = BM_, BN = BN_, BK = BK_;
    static constexpr int nbuf = NBUF_;  // LDS stage buffers (copies issued NBUF - 1 stages ahead)
    static constexpr int fold = FOLD_;  // stages per accumulation chunk on the copy path
    static constexpr bool prefetch = PREFETCH_;  // read k group t + 1 before group t's MFMAs
    static constexpr bool prio = PRIO_;          // raised issue priority while issuing MFMAs
    static constexpr bool stagger = STAGGER_;    // half the waves copy after k group WRITE_G
    static constexpr bool cross = CROSS_;        // read the next stage's first group ahead
    static constexpr int ksplit = KSPLIT_;                 // k-slices of waves
    static constexpr int waves_mn = WAVES_M * WAVES_N;     // waves per k-slice
    static constexpr int waves = waves_mn * KSPLIT_;
    static constexpr int threads = kWave * waves;
    static constexpr int waves_n = WAVES_N;
    static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    static constexpr int FM = WM / kBlk, FN = WN / kBlk;
    static constexpr int wpe = WPE_;
    static constexpr int group_m = GROUP_M_;
    static constexpr int write_g = WRITE_G_;
    static constexpr int chains = CHAINS_;  // independent partial sums per block
    static_assert(4 % CHAINS_ == 0, "chains divide the 4 MFMAs of a k group");
    static_assert(WM % kBlk == 0 && WN % kBlk == 0, "wave tiles are whole MFMA blocks");
    static_assert(BK % 8 == 0, "stages are whole 8-k fragment groups");
    static_assert((BK / 8) % KSPLIT_ == 0, "k-slices share a stage's groups evenly");
    static_assert(KSPLIT_ == 1 || KSPLIT_ == 2 || KSPLIT_ == 4, "k-slices reduce as a binary tree");
    static_assert(NBUF_ >= 2 && NBUF_ <= 4 && (FOLD_ == 0 || NBUF_ % FOLD_ == 0 || FOLD_ % NBUF_ == 0),
                  "2-4 stage buffers; a chunk divides, or is a multiple of, the buffer cycle");
    static_assert(KSPLIT_ == 1 || BM * BN <= (BM + BN) * BK,
                  "a k-slice's partial tile fits in one stage buffer for the reduction");
};

#ifndef GEMM_MFMA_DEEP
#define GEMM_MFMA_DEEP 1
#endif

// GEMM_MFMA_SINGLE_BUFFER 1 builds the ablation without double buffering:
// one stage buffer, each copy issued after the previous stage's compute and
// awaited before the next (the same results).
#ifndef GEMM_MFMA_SINGLE_BUFFER
#define GEMM_MFMA_SINGLE_BUFFER 0
#endif

// GEMM_MFMA_SWIZZLE 0 builds the ablation with unswizzled LDS rows (the same
// results; its bank conflicts show what the swizzle removes).  The library
// is built with 1.
#ifndef GEMM_MFMA_SWIZZLE
#define GEMM_MFMA_SWIZZLE 1
#endif

// LDS tile of one operand for one stage.  P = extent along m (or n); KC =
// the stored rows of the operand run along k (A untransposed, B transposed):
// then the tile is P rows of BK floats, else BK rows of P floats.  Rows are
// unpadded; 16-byte vector v of row r sits at vector slot
// r * vpr + (v ^ swz(r)).
template <class Cfg, int P, bool KC>
struct Tile {
    static constexpr int rows = KC ? P : Cfg::BK;
    static constexpr int cols = KC ? Cfg::BK : P;
    static constexpr int vpr = cols / 4;  // 16-byte vectors per row
    static constexpr int floats = rows * cols;
    static constexpr int chunks = rows * vpr / kWave;  // 1 KB pieces, one per DMA instruction
    static constexpr int dma_per_wave = (chunks + Cfg::waves - 1) / Cfg::waves;
    static_assert(chunks % Cfg::waves == 0 || Cfg::waves % chunks == 0,
                  "DMA instructions split evenly over the waves, or over the first waves");
    // False only for the waves past the last piece when pieces < waves.
    __device__ static __forceinline__ bool dma_active(int wave, int q)
    {
        return chunks % Cfg::waves == 0 || wave * dma_per_wave + q < chunks;
    }
    static_assert((vpr & (vpr - 1)) == 0, "rows hold a power-of-two number of vectors");
    using Load = Slice<rows, cols, Cfg::threads>;
    static constexpr int per_thread = Load::per_thread;
    // LDS read instructions per fragment: one 16-byte read along k, or four
    // floats down the rows, which the compiler pairs into two reads.
    static constexpr int reads = KC ? 1 : 2;

    // KC: a fragment read takes 16 bytes from each of 32 consecutive rows,
    //   and the LDS serves 16 lanes of a 16-byte read per cycle, which must
    //   fall in 16 different 16-byte groups of the 256-byte bank line.  Rows
    //   of 8 vectors (128 bytes) alternate between the line's halves, and
    //   (r & 7) ^ ((r >> 3) & 1) gives the 8 rows of each parity among any 16
    //   consecutive rows 8 different groups.  Rows of 16 or more vectors all
    //   start a bank line, so r & 15 gives 16 consecutive rows 16 different
    //   groups (measured: 8 groups left two-way conflicts, 2.5e6 stalled
    //   cycles per launch of the ragged 2049 x 3071 x 769 product).
    // MC: a fragment read takes 4 bytes from 32 consecutive floats of row k
    //   (lanes 0-31) and of row k + 4 (lanes 32-63); flipping bit 3 of the
    //   vector index every 4 rows puts the two halves in opposite 128-byte
    //   halves of a 256-byte bank line.
    //   With 4 vectors per row (BK = 16) the same two properties come from
    //   ((r >> 1) ^ (r >> 2)) & 3.
    __device__ static __forceinline__ int swz(int r)
    {
        if (!GEMM_MFMA_SWIZZLE) return 0;  // the unswizzled ablation build
        if (KC) {
            if (vpr == 4) return ((r >> 1) ^ (r >> 2)) & 3;
            if (vpr >= 16) return r & 15;
            return ((r & 7) ^ ((r >> 3) & 1)) & (vpr - 1);
        }
        return (((r >> 2) & 1) << 3) & (vpr - 1);
    }
    __device__ static __forceinline__ int slot(int r, int v) { return r * vpr + (v ^ swz(r)); }

    // Registers -> LDS for the register-staged path (same slice-to-thread
    // map as the load).
    __device__ static __forceinline__ void store(float *lds, const v4f (&reg)[per_thread],
                                                 int tid = int(threadIdx.x))
    {
#pragma unroll
        for (int q = 0; q < per_thread; ++q)
            if (Load::active(q, tid))
                *reinterpret_cast<v4f *>(lds + 4 * slot(Load::row(q, tid), Load::col(q, tid) / 4)) = reg[q];
    }
    // The race-detection build's NaN over the bytes store() will write.
    __device__ static __forceinline__ void poison(float *lds)
    {
#pragma unroll
        for (int q = 0; q < per_thread; ++q)
            if (Load::active(q)) poison16(lds + 4 * slot(Load::row(q), Load::col(q) / 4));
    }

    // Byte offset, from the stage's stored origin, of the vector this lane
    // copies in its wave's DMA piece q.  Lane l of chunk c fills vector slot
    // 64c + l, i.e. row (64c + l) / vpr, and fetches the vector the swizzle
    // places there; the lanes of a row read one contiguous segment.  The
    // caller guarantees rows * ld * 4 < 2^32.
    __device__ static __forceinline__ uint32_t dma_offset(int64_t ld, int wave, int lane, int q)
    {
        const int s = (wave * dma_per_wave + q) * kWave + lane;
        const int r = s / vpr;
        const int v = (s % vpr) ^ swz(r);
        return uint32_t((int64_t(r) * ld + 4 * v) * 4);
    }
    // Copy one stage: `origin` is the stage's stored origin (wave-uniform).
    __device__ static __forceinline__ void dma(float *lds, const char *origin,
                                               const uint32_t (&off)[dma_per_wave], int wave, uint32_t avail)
    {
        if (GEMM_LDS_POISON) {
#pragma unroll
            for (int q = 0; q < dma_per_wave; ++q)
                if (dma_active(wave, q)) poison16(lds + (wave * dma_per_wave + q) * 256 + 4 * (threadIdx.x % kWave));
            poison_wait();
        }
#pragma unroll
        for (int q = 0; q < dma_per_wave; ++q)
            if (dma_active(wave, q)) copy16_to_lds(lds + (wave * dma_per_wave + q) * 256, origin, off[q], avail);
    }

    // The four k values (one per MFMA u = 0..3) this lane feeds for k group
    // g at m (or n) position p of the tile.  Lane half h covers k = 8g + 4h + u.
    __device__ static __forceinline__ v4f fragment(const float *lds, int p, int g, int h)
    {
        if (KC) {
            return *reinterpret_cast<const v4f *>(lds + 4 * slot(p, 2 * g + h));
        } else {
            const int k = 8 * g + 4 * h;  // rows k..k+3 share one swizzle
            const float *col = lds + 4 * slot(k, p >> 2) + (p & 3);
            return v4f{col[0], col[4 * vpr], col[8 * vpr], col[12 * vpr]};
        }
    }
};

// A few rows left over below the last whole row of 64 x 64 tiles (M = 64 q
// + r, r <= kThinMaxRows) would cost a whole row of tiles that run the full
// k loop for r valid rows each, and with them a partial extra round of
// workgroups (2049 x 3071 x 769: 110 us against 94 us without its last
// row).  Instead, extra workgroups placed first in the grid compute those
// rows as a matrix-vector style product: each takes kWave / kThinSplit
// columns; k is cut into waves x kThinSplit contiguous slices, one per
// wave and lane group, and each lane sums its column's products in FP32
// over its slice; the slices' sums are then added in slice order through
// LDS (a fixed order: results do not depend on timing), the fused bias and
// activation applied, and the rows stored.  The extra workgroups hold tile
// slots while the tiles start, so they are made short: many of them, each
// with a few batches of loads per lane.
constexpr int kThinMaxRows = 4;
#ifndef GEMM_THIN_SPLIT
#define GEMM_THIN_SPLIT 4
#endif
constexpr int kThinSplit = GEMM_THIN_SPLIT;  // lane groups per wave (k slices per wave)
constexpr int kThinCols = kWave / kThinSplit;  // columns per workgroup
static_assert(kWave % kThinSplit == 0, "whole lane groups");

// R rows from m_lo; this lane's column; its slice [k_lo, k_hi) of k.  Every
// load is unconditional (a load past the slice reads its last element and
// the product is dropped), so the compiler issues a whole batch of them
// before the first use: the loop is bound by memory latency, not by
// arithmetic.
template <int R, bool A_KC, bool B_KC>
__device__ __forceinline__ void thin_slice(float (&acc)[kThinMaxRows], int m_lo, int col, int k_lo, int k_hi,
                                           const float *__restrict__ A, int64_t lda, const float *__restrict__ B,
                                           int64_t ldb)
{
    auto ld_b = [&](int k) { return B_KC ? B[int64_t(col) * ldb + k] : B[int64_t(k) * ldb + col]; };
    auto ld_a = [&](int i, int k) { return A_KC ? A[int64_t(m_lo + i) * lda + k] : A[int64_t(k) * lda + (m_lo + i)]; };
    constexpr int U = 16;  // loads in flight per row
    auto batch = [&](int k, auto clamp_t) {
        constexpr bool kClamp = decltype(clamp_t)::value;
        float b[U], a[R][U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int kk = kClamp ? min(k + u, k_hi - 1) : k + u;
            b[u] = ld_b(kk);
#pragma unroll
            for (int i = 0; i < R; ++i) a[i][u] = ld_a(i, kk);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int i = 0; i < R; ++i) acc[i] = !kClamp || k + u < k_hi ? fmaf(a[i][u], b[u], acc[i]) : acc[i];
    };
    int k = k_lo;
    for (; k + U <= k_hi; k += U) batch(k, Bool<false>{});
    if (k < k_hi) batch(k, Bool<true>{});
}

template <class Cfg, bool A_KC, bool B_KC>
__device__ __forceinline__ void thin_rows(int m_lo, int rows, int N, int K, const float *__restrict__ A,
                                          int64_t lda, const float *__restrict__ B, int64_t ldb,
                                          float *__restrict__ C, int64_t ldc, const float *__restrict__ bias,
                                          int act, float *red)
{
    constexpr int kSlices = Cfg::waves * kThinSplit;
    static_assert(kSlices * kThinMaxRows * kThinCols <= (Cfg::BM + Cfg::BN) * Cfg::BK,
                  "the slice sums fit in one stage buffer");
    const int wave = int(threadIdx.x) / kWave, lane = int(threadIdx.x) % kWave;
    const int first = int(blockIdx.x) * kThinCols;
    if (first >= N) return;  // a workgroup of the rounding to whole XCD rounds
    const int cl = lane % kThinCols, slice = wave * kThinSplit + lane / kThinCols;
    const int col = first + cl;
    const bool col_ok = col < N;
    const int per = ceil_div(K, kSlices);
    const int k_lo = min(K, slice * per), k_hi = min(K, k_lo + per);
    float acc[kThinMaxRows];
#pragma unroll
    for (int i = 0; i < kThinMaxRows; ++i) acc[i] = 0.0f;
    const int c = col_ok ? col : N - 1;
    switch (rows) {
    case 1: thin_slice<1, A_KC, B_KC>(acc, m_lo, c, k_lo, k_hi, A, lda, B, ldb); break;
    case 2: thin_slice<2, A_KC, B_KC>(acc, m_lo, c, k_lo, k_hi, A, lda, B, ldb); break;
    case 3: thin_slice<3, A_KC, B_KC>(acc, m_lo, c, k_lo, k_hi, A, lda, B, ldb); break;
    default: thin_slice<kThinMaxRows, A_KC, B_KC>(acc, m_lo, c, k_lo, k_hi, A, lda, B, ldb); break;
    }
#pragma unroll
    for (int i = 0; i < kThinMaxRows; ++i) red[(slice * kThinMaxRows + i) * kThinCols + cl] = acc[i];
    __syncthreads();
    if (wave == 0 && lane < kThinCols && col_ok) {
        for (int i = 0; i < rows; ++i) {
            float x = 0.0f;
            for (int q = 0; q < kSlices; ++q) x += red[(q * kThinMaxRows + i) * kThinCols + cl];
            if (bias != nullptr) x += bias[col];
            if (act == 1) x = gelu(x);
            C[int64_t(m_lo + i) * ldc + col] = x;
        }
    }
}

template <class Cfg, bool A_KC, bool B_KC, bool VEC>
__global__ __attribute__((amdgpu_flat_work_group_size(Cfg::threads, Cfg::threads),
                          amdgpu_waves_per_eu(Cfg::wpe, Cfg::wpe))) void
mfma_kernel(int M, int N, int K, const float *__restrict__ A, int64_t lda,
            const float *__restrict__ B, int64_t ldb, float *__restrict__ C, int64_t ldc,
            int tiles_m, int tiles_n, int tile_base, int dma_ok, int64_t stride_a,
            int64_t stride_b, int64_t stride_c, int64_t batch_base,
            const float *__restrict__ bias, int act, int k_total, int thin_blocks, int thin_rows_n)
{
    // Strided batch: grid y is the product index.
    const int64_t bz = batch_base + blockIdx.y;
    A += bz * stride_a;
    B += bz * stride_b;
    C += bz * stride_c;
    // Split k: product bz covers k in [bz * K, min(k_total, (bz + 1) * K)),
    // its operands already offset by the strides; only the last is shorter.
    if (k_total > 0) K = int(min(int64_t(K), int64_t(k_total) - bz * K));
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK;
    constexpr int FM = Cfg::FM, FN = Cfg::FN;
    using TA = Tile<Cfg, BM, A_KC>;
    using TB = Tile<Cfg, BN, B_KC>;
    // Stage buffers as separate objects, so the compiler can tell a copy into
    // one from reads of another.
    constexpr int kStage = TA::floats + TB::floats;
    __shared__ __attribute__((aligned(1024))) float buf0[kStage];
    __shared__ __attribute__((aligned(1024))) float buf1[kStage];
    __shared__ __attribute__((aligned(1024))) float buf2[Cfg::nbuf > 2 ? kStage : 1];
    __shared__ __attribute__((aligned(1024))) float buf3[Cfg::nbuf > 3 ? kStage : 1];

    // Rows M .. M + thin_rows_n - 1 (below the tiles; single products only).
    if (int(blockIdx.x) < thin_blocks) {
        thin_rows<Cfg, A_KC, B_KC>(M, thin_rows_n, N, K, A, lda, B, ldb, C, ldc, bias, act, buf0);
        return;
    }
    int tm, tn;
    tile_of<Cfg::group_m>(tile_base + int(blockIdx.x) - thin_blocks, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const bool inside = (m0 + BM <= M) && (n0 + BN <= N);
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    // The same, in a scalar register.  The mask states its range, which the
    // compiler cannot see through the scalar read: without it, a copy's LDS
    // destination could be anywhere, and the compiler would wait for every
    // copy in flight before each LDS read.
    static_assert((Cfg::waves & (Cfg::waves - 1)) == 0, "a power-of-two wave count");
    const int wave_s = __builtin_amdgcn_readfirstlane(wave) & (Cfg::waves - 1);
    const int kslice = wave / Cfg::waves_mn, wmn = wave % Cfg::waves_mn;
    const int kslice_s = wave_s / Cfg::waves_mn;  // the same, scalar
    const int wm = (wmn / Cfg::waves_n) * Cfg::WM, wn = (wmn % Cfg::waves_n) * Cfg::WN;
    const int half = lane / 32, l32 = lane % 32;
    const int stages = ceil_div(K, BK);
    const int full = K / BK;  // stages that lie entirely inside K

    v16f acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = v16f{0.0f};

    // MFMAs over the BK k values in `lds` into a fresh partial tile, folded
    // into acc at the end.  `mid` runs after the fragment reads of k group
    // write_g (the register-staged path writes the next stage there; the
    // buffer it writes was last read in the previous stage, which every wave
    // finished before that stage's barrier).
    constexpr int CH = Cfg::chains;
    constexpr bool kChunked = Cfg::fold > 0;
    v16f part[kChunked ? CH : 1][kChunked ? FM : 1][kChunked ? FN : 1];
    auto fold_part = [&] {
        if constexpr (kChunked) {
#pragma unroll
            for (int c = 0; c < CH; ++c)
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j) acc[i][j] += part[c][i][j];
        }
    };
    // MFMAs over the BK k values in `lds` into the partial tile; FRESH starts
    // a chunk (the first MFMA of each chain takes a zero addend), FOLD ends
    // it (the partial tile is added into acc).  `mid` runs after the
    // fragment reads of k group write_g (the register-staged path writes the
    // next stage there; the buffer it writes was last read in the previous
    // stage, which every wave finished before that stage's barrier).
    // PREFETCH_T: read the next group's fragments ahead (the copy path; the
    // register-staged path, whose loaded stage is live across the MFMAs,
    // reads them just in time to stay within the register budget).
    // TAIL_T: the stage holds the last kv < BK k values of the product and
    // whatever follows them (zeros on the register-staged path; on the copy
    // path the next row's values, or zeros past the end of the storage): the
    // k groups past kv are skipped (a slice's first group still runs, to
    // start its chunk) and each fragment value past kv is replaced by zero.
    constexpr int kGroups = BK / 8 / Cfg::ksplit;  // k groups per slice per stage
    constexpr bool kPrefetchCfg = Cfg::prefetch && !(Cfg::BM == 256 && !A_KC && B_KC);
    // The first k group's fragments of the next stage, read ahead by the
    // previous stage (cross-stage prefetch only).
    v4f xa[FM], xb[FN];
    auto read_at = [&](const float *lds, int t, v4f (&ra)[FM], v4f (&rb)[FN]) {
        const int g = Cfg::ksplit == 1 ? t : t * Cfg::ksplit + kslice;
#pragma unroll
        for (int i = 0; i < FM; ++i) ra[i] = TA::fragment(lds, wm + i * kBlk + l32, g, half);
#pragma unroll
        for (int j = 0; j < FN; ++j) rb[j] = TB::fragment(lds + TA::floats, wn + j * kBlk + l32, g, half);
    };
    // CROSS_T (the copy ring, with prefetch): the first group's fragments
    // were read ahead (xa, xb), and the last group's MFMAs are preceded by
    // the read of `next`'s first group, so that after the next barrier a
    // wave starts its MFMAs without waiting on LDS.
    auto compute_x = [&](const float *lds, const float *next, auto mid, auto fresh_t, auto fold_t, auto prefetch_t,
                         auto tail_t, auto cross_t, int kv) {
        constexpr bool kFresh = decltype(fresh_t)::value;
        constexpr bool kFold = decltype(fold_t)::value;
        constexpr bool kTail = decltype(tail_t)::value;
        constexpr bool kPrefetch = kPrefetchCfg && decltype(prefetch_t)::value;
        constexpr bool kCross = kPrefetch && decltype(cross_t)::value;
        static_assert(!kCross || !kTail, "a full stage");
        // With prefetch, the fragments of k group t + 1 are read before the
        // MFMAs of group t, so LDS latency overlaps matrix-core work.
        v4f fa[2][FM], fb[2][FN];
        auto read = [&](int t, int slot) { read_at(lds, t, fa[slot], fb[slot]); };
        if (kCross) {
#pragma unroll
            for (int i = 0; i < FM; ++i) fa[0][i] = xa[i];
#pragma unroll
            for (int j = 0; j < FN; ++j) fb[0][j] = xb[j];
        } else if (kPrefetch) {
            read(0, 0);
        }
        if constexpr (Cfg::prio) __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int t = 0; t < kGroups; ++t) {
            const int g = Cfg::ksplit == 1 ? t : t * Cfg::ksplit + kslice_s;
            if (kTail && t > 0 && 8 * g >= kv) break;
            const int cur = kPrefetch ? (t & 1) : 0;
            if (!kPrefetch)
                read(t, 0);
            else if (t + 1 < kGroups)
                read(t + 1, (t + 1) & 1);
            else if (kCross)
                read_at(next, 0, xa, xb);
            if (Cfg::ksplit == 1 && t == Cfg::write_g) mid();
            if (kTail) {
                // lane half h feeds k = 8g + 4h + u
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const bool ok = 8 * g + 4 * half + u < kv;
#pragma unroll
                    for (int i = 0; i < FM; ++i) fa[cur][i][u] = ok ? fa[cur][i][u] : 0.0f;
#pragma unroll
                    for (int j = 0; j < FN; ++j) fb[cur][j][u] = ok ? fb[cur][j][u] : 0.0f;
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j) {
                        v16f &p = kChunked ? part[kChunked ? u % CH : 0][kChunked ? i : 0][kChunked ? j : 0]
                                           : acc[i][j];
                        p = __builtin_amdgcn_mfma_f32_32x32x2f32(
                            fa[cur][i][u], fb[cur][j][u],
                            (kChunked && kFresh && t == 0 && u < CH) ? v16f{0.0f} : p, 0, 0, 0);
                    }
            // With prefetch, ask the scheduler to spread the next group's LDS
            // reads between this group's MFMAs (one read, then an even share
            // of the MFMAs) instead of clustering them: +0.5-1.5 %.
            if (kPrefetch && (t + 1 < kGroups || kCross)) {
                constexpr int kReads = TA::reads * FM + TB::reads * FN;
                constexpr int kMfma = 4 * FM * FN;
                constexpr int per = kMfma / kReads > 0 ? kMfma / kReads : 1;
#pragma unroll
                for (int q = 0; q < kReads; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
                    __builtin_amdgcn_sched_group_barrier(0x008, per, 0);  // MFMAs
                }
                if (kMfma > per * kReads) __builtin_amdgcn_sched_group_barrier(0x008, kMfma - per * kReads, 0);
            }
        }
        if constexpr (Cfg::prio) __builtin_amdgcn_s_setprio(0);
        if (Cfg::ksplit > 1 || Cfg::write_g >= kGroups) mid();
        if (kFold) fold_part();
    };
    auto compute = [&](const float *lds, auto mid, auto fresh_t, auto fold_t, auto prefetch_t, auto tail_t, int kv) {
        compute_x(lds, lds, mid, fresh_t, fold_t, prefetch_t, tail_t, No{}, kv);
    };
    auto nothing = [] {};

    const Operand opa{A, lda, A_KC ? M : K, A_KC ? K : M};
    const Operand opb{B, ldb, B_KC ? N : K, B_KC ? K : N};
    // stored origin of the stage starting at k: (row, col)
    auto a_r = [&](int k) { return A_KC ? m0 : k; };
    auto a_c = [&](int k) { return A_KC ? k : m0; };
    auto b_r = [&](int k) { return B_KC ? n0 : k; };
    auto b_c = [&](int k) { return B_KC ? k : n0; };
    // Register-staged stages s .. stages-1 with every load predicated; stage
    // s is already in LDS buffer s & 1.
    auto staged = [&](int s) {
        for (; s < stages; ++s) {
            float *cur = (s & 1) ? buf1 : buf0;
            float *nxt = (s & 1) ? buf0 : buf1;
            if (s + 1 < stages) {
                // nxt was released by the barrier that ended stage s - 1
                if (GEMM_LDS_POISON) {
                    TA::poison(nxt);
                    TB::poison(nxt + TA::floats);
                    poison_wait();
                }
                v4f ra[TA::per_thread], rb[TB::per_thread];
                const int k = (s + 1) * BK;
                TA::Load::template load<true, VEC>(opa, a_r(k), a_c(k), ra);
                TB::Load::template load<true, VEC>(opb, b_r(k), b_c(k), rb);
                compute(cur, [&] {
                    TA::store(nxt, ra);
                    TB::store(nxt + TA::floats, rb);
                }, Yes{}, Yes{}, No{}, No{}, BK);
            } else {
                compute(cur, nothing, Yes{}, Yes{}, No{}, No{}, BK);
            }
            __syncthreads();
        }
    };

    // Bytes from a tile's first stage origin to the end of each operand's
    // storage (its last stored element, rounded up to the 16-byte vector
    // that holds it: the vectors are aligned, so that never crosses a page).
    const int64_t a_left = ((4 * (A_KC ? int64_t(M - 1) * lda + K : int64_t(K - 1) * lda + M) + 15) & ~int64_t(15)) -
                           4 * (int64_t(a_r(0)) * lda + a_c(0));
    const int64_t b_left = ((4 * (B_KC ? int64_t(N - 1) * ldb + K : int64_t(K - 1) * ldb + N) + 15) & ~int64_t(15)) -
                           4 * (int64_t(b_r(0)) * ldb + b_c(0));
    // (Edge tiles by DMA on the small tiles, which serve the ragged
    // mid-size products; the large tiles keep the register-staged edge path,
    // their scalar registers being fully used.)
    constexpr bool kEdgeDma = GEMM_BUFFER_DMA && Cfg::BM * Cfg::BN <= 128 * 64;
    const bool edge_dma = kEdgeDma && a_left < (int64_t(1) << 32) && b_left < (int64_t(1) << 32);
    if (VEC && dma_ok && (inside || edge_dma) && full >= 1) {
        // Full stages copied straight into LDS, NBUF - 1 ahead.  Edge tiles
        // too: their copies stop at the end of the operand's storage (the
        // buffer loads' range check, with the bytes left from each stage's
        // origin), and what they read from a row's padding or past the
        // matrix's last row or column only reaches outputs outside C, which
        // are never stored.  Interior tiles copy without a limit.
        uint32_t oa[TA::dma_per_wave], ob[TB::dma_per_wave];
#pragma unroll
        for (int q = 0; q < TA::dma_per_wave; ++q) oa[q] = TA::dma_offset(lda, wave, lane, q);
#pragma unroll
        for (int q = 0; q < TB::dma_per_wave; ++q) ob[q] = TB::dma_offset(ldb, wave, lane, q);
        // Moving one stage along k moves an operand's stored origin by BK
        // columns (KC) or BK rows (otherwise).
        const char *ga = reinterpret_cast<const char *>(A + int64_t(a_r(0)) * lda + a_c(0));
        const char *gb = reinterpret_cast<const char *>(B + int64_t(b_r(0)) * ldb + b_c(0));
        const int64_t a_step = 4 * (A_KC ? int64_t(BK) : int64_t(BK) * lda);
        const int64_t b_step = 4 * (B_KC ? int64_t(BK) : int64_t(BK) * ldb);
        constexpr int NB = Cfg::nbuf, FOLD = Cfg::fold > 0 ? Cfg::fold : 1;
        // Copies per wave per stage; every wave issues the same number, so a
        // count of outstanding copies names a stage.
        constexpr int D = TA::dma_per_wave + TB::dma_per_wave;
        static_assert(NB == 2 || (TA::chunks % Cfg::waves == 0 && TB::chunks % Cfg::waves == 0),
                      "deeper pipelines need the same copy count on every wave");
        auto bufp = [&](auto idx) -> float * {
            constexpr int I = decltype(idx)::value;
            return I == 0 ? buf0 : I == 1 ? buf1 : I == 2 ? buf2 : buf3;
        };
        // 32-bit byte counts: an edge tile copies by DMA only if both fit
        // (checked above), and a stage's step is below 2^32 (dma_ok).
        const uint32_t a_left32 = uint32_t(a_left), b_left32 = uint32_t(b_left);
        const uint32_t a_step32 = uint32_t(a_step), b_step32 = uint32_t(b_step);
        // Where copies can be range-limited, the partial last stage (K % BK
        // k values) is copied like the full ones, a stage ahead, with the
        // limit on every tile: its copy reads on past k = K into the storage
        // that follows (the next row, or zeros past the end), values that
        // the tail compute replaces by zeros.  (Not when both operands are
        // stored k-major: that layout has no scalar registers to spare, and
        // keeps the register-staged tail.)
        constexpr bool kTailDma = kEdgeDma && !GEMM_MFMA_SINGLE_BUFFER && (A_KC || B_KC);
        const bool tail_dma = kTailDma && edge_dma && full < stages;
        const int ndma = full + int(tail_dma);  // stages copied into LDS
        auto dma = [&](float *lds, int stage) {
            const bool open = !kEdgeDma || (inside && (!kTailDma || stage < full));
            const uint32_t aa = open ? 0xFFFFFFFFu : a_left32 - uint32_t(stage) * a_step32;
            const uint32_t ab = open ? 0xFFFFFFFFu : b_left32 - uint32_t(stage) * b_step32;
            TA::dma(lds, ga + stage * a_step, oa, wave_s, aa);
            TB::dma(lds + TA::floats, gb + stage * b_step, ob, wave_s, ab);
        };
        // The deep ring (below) issues exactly NB - 1 stages up front,
        // repeating the last one where there are fewer.
        constexpr bool kDeep = GEMM_MFMA_DEEP && NB > 2 && !GEMM_MFMA_SINGLE_BUFFER && !Cfg::stagger;
        constexpr bool kCross = kDeep && Cfg::cross && kPrefetchCfg;
        dma(buf0, 0);
        if (!GEMM_MFMA_SINGLE_BUFFER && NB > 2 && (kDeep || 1 < ndma)) dma(bufp(Int<1 % NB>{}), min(1, ndma - 1));
        if (!GEMM_MFMA_SINGLE_BUFFER && NB > 3 && (kDeep || 2 < ndma)) dma(bufp(Int<2 % NB>{}), min(2, ndma - 1));
        // TRIP stages per trip (a multiple of NB and of FOLD) so that each
        // buffer and each chunk boundary is a compile-time choice.
        constexpr int TRIP = NB > FOLD ? NB : FOLD;
        constexpr int DTRIP = TRIP * (GEMM_MFMA_DEEP > 0 ? GEMM_MFMA_DEEP : 1);
        if (kDeep) {
            // Copies NB - 1 stages ahead that stay in flight across the
            // barriers: each wave waits for its own copies of the stage it
            // is about to read, and the barrier is not fenced (a fence would
            // wait for every copy in flight).  Every stage issues one copy
            // (past the last stage, the last one again, into a buffer that
            // is not read), so that a count of outstanding copies names a
            // stage; the trips of DTRIP whole stages have no branches, so
            // the compiler can tell which buffer each copy writes and does
            // not wait for copies before the reads.  (The partial last
            // stage, if copied, lands in buffer full % NB like any other,
            // and the repeats after it go to the other buffers.)
            //
            // With kCross, each barrier also certifies the stage after the
            // one it starts (each wave first waits for its own copies of
            // both), so a stage reads the next stage's first fragments before
            // its last MFMAs: the copies then have NB - 2 stages to land
            // instead of NB - 1.
            if constexpr (kCross) {
                wait_vm<(NB - 3) * D>();  // stages 0 and 1 have landed
                __builtin_amdgcn_s_waitcnt(0xC07F);
                __builtin_amdgcn_s_barrier();
                __builtin_amdgcn_sched_barrier(0);
                read_at(buf0, 0, xa, xb);
            }
            auto stage = [&](auto bi, int st) {
                constexpr int b = decltype(bi)::value;
                wait_vm<(kCross ? NB - 3 : NB > 2 ? NB - 2 : 0) * D>();  // stage st (and st + 1) have landed
                __builtin_amdgcn_s_waitcnt(0xC07F);    // this wave's LDS reads are done
                __builtin_amdgcn_s_barrier();
                __builtin_amdgcn_sched_barrier(0);
                dma(bufp(Int<(b + NB - 1) % NB>{}), min(st + NB - 1, ndma - 1));
                compute_x(bufp(Int<b % NB>{}), bufp(Int<(b + 1) % NB>{}), nothing, Bool<b % FOLD == 0>{},
                          Bool<b % FOLD == FOLD - 1>{}, Yes{}, No{}, Bool<kCross>{}, BK);
            };
            int s = 0;
            for (; s + DTRIP <= full; s += DTRIP) unroll_for<DTRIP>([&](auto bi) { stage(bi, s + decltype(bi)::value); });
            if (s < full)
                unroll_for<DTRIP>([&](auto bi) {
                    if (s + decltype(bi)::value < full) stage(bi, s + decltype(bi)::value);
                });
            wait_vm<0>();
        } else
        for (int s = 0; s < full; s += TRIP) {
            unroll_for<TRIP>([&](auto bi) {
                constexpr int b = decltype(bi)::value;
                const int st = s + b;
                if (GEMM_MFMA_SINGLE_BUFFER && st < full) {
                    // The ablation: the course page's pattern with one
                    // buffer -- copy, barrier, compute, barrier, next copy.
                    wait_vm<0>();
                    __syncthreads();
                    compute(buf0, nothing, Bool<b % FOLD == 0>{}, Bool<b % FOLD == FOLD - 1>{}, Yes{}, No{}, BK);
                    __syncthreads();
                    if (st + 1 < full) dma(buf0, st + 1);
                } else if (st < full) {
                    // Stage st has landed (at most the copies of the NB - 2
                    // later stages are outstanding); after the barrier every
                    // wave's share is visible, and every wave is done with
                    // stage st - 1, whose buffer the next copy refills.
                    // __syncthreads' release fence also makes the compiler
                    // wait for every outstanding copy before the barrier, so
                    // in effect each stage's copies have one stage to land
                    // whatever NB is.  A barrier without the fence (keeping
                    // the later stages in flight) was measured and gained
                    // nothing (4096^3 138.4 vs 138.3 TFLOP/s; the ragged
                    // ring 83.2 vs 85.3): the copies are not latency bound.
                    if (NB == 2 || st + NB - 2 >= ndma)
                        wait_vm<0>();
                    else
                        wait_vm<(NB - 2) * D>();
                    __syncthreads();
                    // Copies are counted per wave in issue order, so a wave
                    // that copies later in the stage still has the same
                    // count outstanding at the next wait.
                    const bool late = Cfg::stagger && wave >= Cfg::waves / 2;
                    if (!late && st + NB - 1 < ndma) dma(bufp(Int<(b + NB - 1) % NB>{}), st + NB - 1);
                    compute(bufp(Int<b % NB>{}), [&] {
                        if (late && st + NB - 1 < ndma) dma(bufp(Int<(b + NB - 1) % NB>{}), st + NB - 1);
                    }, Bool<b % FOLD == 0>{}, Bool<b % FOLD == FOLD - 1>{}, Yes{}, No{}, BK);
                }
            });
        }
        if (full % FOLD != 0) fold_part();  // the last chunk was cut short
        if (tail_dma) {
            // The partial stage has landed in buffer full % NB.
            wait_vm<0>();
            __syncthreads();
            const int tb = full % NB;
            compute(tb == 0 ? buf0 : tb == 1 ? buf1 : tb == 2 ? buf2 : buf3, nothing, Yes{}, Yes{}, Yes{}, Yes{},
                    K - full * BK);
            __syncthreads();
        } else {
            __syncthreads();  // every wave is done with the last full stage's buffer
            if (full < stages) {
                // The partial last stage, predicated, through registers.
                // Its thread index is derived afresh (the lane counted from
                // the full execution mask, the wave from a scalar register)
                // and its fragments are read as in the loop, so that nothing
                // besides the accumulators has to stay live across the loop
                // for it.
                const int tid =
                    kWave * wave_s + int(__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)));
                v4f ra[TA::per_thread], rb[TB::per_thread];
                TA::Load::template load<true, VEC>(opa, a_r(full * BK), a_c(full * BK), ra, tid);
                TB::Load::template load<true, VEC>(opb, b_r(full * BK), b_c(full * BK), rb, tid);
                TA::store(buf0, ra, tid);
                TB::store(buf0 + TA::floats, rb, tid);
                __syncthreads();
                compute(buf0, nothing, Yes{}, Yes{}, Yes{}, Yes{}, K - full * BK);
                __syncthreads();
            }
        }
    } else {
        v4f ra[TA::per_thread], rb[TB::per_thread];
        TA::Load::template load<true, VEC>(opa, a_r(0), a_c(0), ra);
        TB::Load::template load<true, VEC>(opb, b_r(0), b_c(0), rb);
        TA::store(buf0, ra);
        TB::store(buf0 + TA::floats, rb);
        __syncthreads();
        staged(0);
    }

    // Epilogue for accumulator slots V0 .. V1 - 1.  Lane l of a 32 x 32
    // block holds column l % 32 and, in accumulator slot v, row 8 * (v / 4)
    // + 4 * (l / 32) + v % 4.  The fused variant adds bias[column] and
    // applies the activation before the store (both flags are uniform over
    // the launch).  The lane's position is derived afresh -- the lane index
    // counted from the (full) execution mask, the wave index from a scalar
    // register -- so that nothing lane-dependent has to stay in a vector
    // register across the k loop.
    auto epilogue = [&](auto v0_t, auto v1_t) {
        constexpr int V0 = decltype(v0_t)::value, V1 = decltype(v1_t)::value;
        const int e_lane = int(__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)));
        const int e_wmn = wave_s % Cfg::waves_mn;
        const int e_wm = (e_wmn / Cfg::waves_n) * Cfg::WM, e_wn = (e_wmn % Cfg::waves_n) * Cfg::WN;
        const int e_l32 = e_lane % 32, e_half = e_lane / 32;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int col = n0 + e_wn + j * kBlk + e_l32;
                const float bj = (bias != nullptr && col < N) ? bias[col] : 0.0f;
#pragma unroll
                for (int v = V0; v < V1; ++v) {
                    const int row = m0 + e_wm + i * kBlk + 8 * (v / 4) + 4 * e_half + (v % 4);
                    float x = acc[i][j][v] + bj;
                    if (act == 1) x = gelu(x);
                    if (inside || (row < M && col < N)) {
                        // C is written once and not read again here: a
                        // streaming (non-temporal) store, except for split-k
                        // partials, which the reduction reads straight back
                        // (64 products of 512 x 512 x 64: 66.3 vs 64.6
                        // TFLOP/s; 1024^3 97.4 vs 96.4).
                        if (k_total > 0)
                            C[int64_t(row) * ldc + col] = x;
                        else
                            __builtin_nontemporal_store(x, &C[int64_t(row) * ldc + col]);
                    }
                }
            }
    };

    if constexpr (Cfg::ksplit == 2) {
        // Two k-slices: each finishes half of every block's rows.  Slice 0
        // keeps accumulator slots 0-7 and hands 8-15 to slice 1 through the
        // (now idle) first stage buffer, slice 1 the reverse; each adds the
        // half it receives to its own and stores that half, so all the
        // waves share the final stores.  a + b equals b + a exactly, so the
        // sums do not depend on which slice forms them.
        auto slot = [&](int slice, int i, int j, int vv) {
            return ((((slice * Cfg::waves_mn + wmn) * FM + i) * FN + j) * 8 + vv) * kWave + lane;
        };
        auto give = [&](auto v0_t) {
            constexpr int V0 = decltype(v0_t)::value;
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int vv = 0; vv < 8; ++vv) buf0[slot(kslice, i, j, vv)] = acc[i][j][V0 + vv];
        };
        auto take = [&](auto v0_t) {
            constexpr int V0 = decltype(v0_t)::value;
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int vv = 0; vv < 8; ++vv) acc[i][j][V0 + vv] += buf0[slot(1 - kslice, i, j, vv)];
        };
        if (kslice_s == 0)
            give(Int<8>{});
        else
            give(Int<0>{});
        __syncthreads();
        if (kslice_s == 0) {
            take(Int<0>{});
            epilogue(Int<0>{}, Int<8>{});
        } else {
            take(Int<8>{});
            epilogue(Int<8>{}, Int<16>{});
        }
        return;
    } else if constexpr (Cfg::ksplit > 1) {
        // Sum the k-slices' partial tiles, pairwise through the (now idle)
        // stage buffers: at each level the upper half of the slices writes,
        // the lower half adds.  Every stage buffer holds at least one BM x BN
        // tile.
#pragma unroll
        for (int width = Cfg::ksplit / 2; width >= 1; width /= 2) {
            const bool writer = kslice >= width && kslice < 2 * width;
            const bool reader = kslice < width;
            float *xbuf = ((kslice % width) == 0) ? buf0 : buf1;  // width <= 2
            if (writer) {
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
#pragma unroll
                        for (int v = 0; v < 16; ++v)
                            xbuf[(((wmn * FM + i) * FN + j) * 16 + v) * kWave + lane] = acc[i][j][v];
            }
            __syncthreads();
            if (reader) {
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
#pragma unroll
                        for (int v = 0; v < 16; ++v)
                            acc[i][j][v] += xbuf[(((wmn * FM + i) * FN + j) * 16 + v) * kWave + lane];
            }
            __syncthreads();
        }
        if (kslice != 0) return;  // slice 0 holds the sum; no barrier follows
    }
    epilogue(Int<0>{}, Int<16>{});
}

#ifndef GEMM_MFMA_CONFIG
#define GEMM_MFMA_CONFIG 128, 128, 16, 4, 2, 4, 8, 3, 1, 1, 4, 8, 1
#endif
#ifndef GEMM_MFMA_SMALL_CONFIG
#define GEMM_MFMA_SMALL_CONFIG 64, 64, 64, 2, 2, 4, 8, 3, 1, 2, 4, 4, 1, 1
#endif
#ifndef GEMM_MFMA_SMALL_PAIR_CONFIG
#define GEMM_MFMA_SMALL_PAIR_CONFIG 64, 64, 64, 2, 2, 4, 8, 3, 1, 2, 2, 2, 1, 1
#endif
#ifndef GEMM_MFMA_HUGE_CONFIG
#define GEMM_MFMA_HUGE_CONFIG 256, 128, 16, 4, 2, 2, 4, 1, 1, 1, 4, 16, 1, 0, 0, 1
#endif
#ifndef GEMM_MFMA_KK_CONFIG
#define GEMM_MFMA_KK_CONFIG 128, 128, 16, 4, 2, 4, 8, 3, 1, 1, 4, 8, 1, 1, 0, 1
#endif
#ifndef GEMM_MFMA_ONE_ROUND_CONFIG
#define GEMM_MFMA_ONE_ROUND_CONFIG 128, 128, 32, 4, 2, 4, 8, 1, 1, 1, 4, 8, 1, 0, 0, 1
#endif
#ifndef GEMM_MFMA_NARROW_CONFIG
#define GEMM_MFMA_NARROW_CONFIG 128, 64, 64, 4, 2, 4, 8, 7, 1, 1, 2, 4, 1, 1
#endif
// 128 x 128 tile, two workgroups per CU: 16-k stages in four buffers (64 KB)
// whose copies stay in flight across the barriers, 128-k chunks (against 32-k
// stages in two buffers: 4096 x 2048 x 1024 138.2-139.0 vs 137.3-137.7
// TFLOP/s, 3072^2 x 1024 107.5 vs 105.0-105.2, 2560^2 x 2048 114.3-114.4 vs
// 113.1; raised issue priority lost 1 %).
using Default = Config<GEMM_MFMA_CONFIG>;
// 64 x 64 tile, two k-slices of 4 waves, for grids of up to one tile per CU:
// 64-k stages in four buffers (128 KB) whose copies stay in flight across
// the barriers, 256-k accumulation chunks (1024^3: 108.0-108.9 TFLOP/s
// against 105.7-106.3 for 128-k stages in two fenced buffers; 32-k stages
// 102.4, three buffers 105.6, 512-k chunks 107.0, without the read-ahead
// 104.7, without raised priority 97.7, four k-slices 99.2).  Earlier, with
// fenced barriers, 128-k stages in two buffers: a stage long enough to hide
// one stage of copy latency with a quarter of the barriers of 32-k stages
// (1024^3, one tile per CU: 96.3 vs 94.2 TFLOP/s; 64 products
// of 512 x 64 x 512: 84.9 vs 82.6, and 85.6 vs 83.9 with raised MFMA issue
// priority; three or four 64-k buffers or 128-k stages were slower; reading
// the next k group's fragments before the current group's MFMAs: 1024^3
// 97.6 vs 95.4).  With the copies as buffer loads, 128-k stages (one per
// accumulation chunk; 128 KB of LDS) are ahead instead: 1024^3 104.7-104.9
// vs 103.3-103.5 for 64-k stages; 256-k chunks rather than one per stage
// 105.7-105.9 vs 105.3-105.4 (two partial chains 104.2, four k-slices of
// 16 waves 100.4, 64-k stages with 256-k chunks 102.9).  With more tiles per CU (the ragged
// 2049 x 3071 x 769 product: six) two workgroups share a CU and hide each
// other's barriers and start-up: SmallPair, 64-k stages in two buffers (64 KB
// of LDS each), 128-k accumulation chunks, the next k group's fragments
// read ahead and raised MFMA issue priority (111.5-112.3 TFLOP/s there,
// against 106.8-107.2 for 32-k stages in a four-buffer ring; without the
// read-ahead 110.5-110.9, without the priority 102.3-102.6, with 64-k or
// 256-k chunks 109.5-109.9 / 111.2-111.5).
using Small = Config<GEMM_MFMA_SMALL_CONFIG>;
using SmallPair = Config<GEMM_MFMA_SMALL_PAIR_CONFIG>;
// 256 x 128 tile, 8 waves of 64 x 64, one workgroup per CU: 16-k stages in
// four 24 KB buffers whose copies stay in flight across the barriers, each
// barrier also certifying the next stage, whose first fragments are read
// before the current stage's last MFMAs; 256-k accumulation chunks,
// tile-groups of 4 rows.  A quarter fewer
// bytes copied into LDS per flop than the 128 x 128 tile: on 4096^3 136 vs
// 134 TFLOP/s in the first build.  Needs enough tiles to fill every CU
// twice.  History at 4096^3 (and the 8192 x 1024 x 4096 input gradient):
// with fenced barriers, which drain every copy, two buffers and 256-k
// chunks with half the waves copying after k group 1 were best (145.0 vs
// 143.8-144.2 for three buffers; 145.8 vs 144.7); with the copies kept in
// flight, three buffers reach 148.3-148.4 (147.8-147.9) against 144.3-145.5
// (145.2-146.0), raised MFMA issue priority costing 1-1.5 %, 96-k chunks
// 1.5 %; 384-k chunks are level.  16-k stages in four buffers with the
// read-ahead across the barriers then gave 148.5-149.4 against 148.2-148.4
// (148.2-148.7 against 147.7-147.8), and without the read-ahead were level;
// 256-k chunks rather than 192-k then gave 150.2-150.3 against 149.4-149.8
// (149.4-149.7 against 148.9-149.2) on a faster machine.  Relative Frobenius
// error at 4096^3 about 3e-7.
using Huge = Config<GEMM_MFMA_HUGE_CONFIG>;
// Large tile when both operands are k-contiguous (A untransposed, B
// transposed): every DMA row segment is a short run along k, and 16-k
// stages in four buffers were measured faster (the
// 8192 x 1024 x 4096 input-gradient product: 125 -> 129 TFLOP/s; with
// raised MFMA issue priority 131.1 -> 135.1).  With the copies kept in
// flight across the barriers (2048^3 128.7 -> 136.0), and with each barrier
// also certifying the next stage, whose first fragments are read before the
// current stage's last MFMAs: 2048^3 136.3-136.8 -> 139.9-140.6, 4096 x 2048
// x 1024 138.9-139.2 -> 140.4-141.4, 2560^2 x 2048 113.4-113.7 -> 114.9-115.4
// (one session).  (The other layouts of the 128 x 128 tile would spill
// registers with this read-ahead at two workgroups per CU.)
using DefaultKK = Config<GEMM_MFMA_KK_CONFIG>;
// 128 x 128 tile for grids of at most one tile per CU, where no second
// workgroup shares a CU: four stage buffers whose copies stay in flight
// across the barriers (three stages ahead), 256-k accumulation chunks (the
// 1024 x 4096 x 8192 weight gradient, 256 tiles: 147.5-147.7 TFLOP/s
// against 143.0-143.3 for two buffers with fenced barriers, raised MFMA
// issue priority and staggered copies, which had given 137.4-137.6 against
// 132.7-133.1 in the first build; with the copies in flight the priority
// costs 1.7 %, and 128-k chunks 1 %).  Each barrier also certifies the
// stage after the one it starts, and a stage reads the next stage's first
// fragments before its last MFMAs (copies two stages ahead instead of
// three): 148.2-148.8 against 146.7 in one session.  (The same on the
// 256 x 128 tile, whose copies would then have one stage to land, and on
// the one-tile-per-CU 64 x 64 tile was level or slower.)
using OneRound = Config<GEMM_MFMA_ONE_ROUND_CONFIG>;
// 128 x 64 tile for outputs at most 64 columns wide (8 waves of 32 x 32,
// 64-k stages in two buffers, 256-k accumulation chunks): a quarter fewer
// bytes copied per flop than the 64 x 64 tile, and one tile per CU from
// 256 tiles up (64 attention-value products of 512 x 64 x 512: 94-98
// against 86-87 TFLOP/s on 64 x 64 tiles).
using Narrow = Config<GEMM_MFMA_NARROW_CONFIG>;

// True if every DMA offset of an operand's stage fits in 32 bits.
inline bool dma_offsets_fit(int rows, int64_t ld) { return (int64_t(rows) * ld + ld) * 4 < (int64_t(1) << 32); }

template <class Cfg, bool A_KC, bool B_KC, bool VEC>
void dispatch(const Problem &p, hipStream_t s)
{
    using TA = Tile<Cfg, Cfg::BM, A_KC>;
    using TB = Tile<Cfg, Cfg::BN, B_KC>;
    // 64-row tiles with at most kThinMaxRows rows left over: those rows go
    // to the matrix-vector workgroups at the front of the grid, the tiles
    // cover the rows above them.
    const int rest = p.M % Cfg::BM;
    const bool thin = Cfg::BM == 64 && p.batch == 1 && p.k_total == 0 && p.M > Cfg::BM && rest > 0 &&
                      rest <= kThinMaxRows;
    const int m_tiles = thin ? p.M - rest : p.M;
    // (a multiple of the XCD count, so that tile t still runs on XCD t % 8)
    const int thin_blocks = thin ? kXcds * ceil_div(ceil_div(p.N, kThinCols), kXcds) : 0;
    const int tiles_m = ceil_div(m_tiles, Cfg::BM), tiles_n = ceil_div(p.N, Cfg::BN);
    const int64_t tiles = int64_t(tiles_m) * tiles_n;
    const int dma_ok = dma_offsets_fit(TA::rows, p.lda) && dma_offsets_fit(TB::rows, p.ldb);
    // One workgroup per tile (grid x) and product (grid y); grids larger
    // than the caps are split into launches whose first tile index is a
    // multiple of 8, so the XCD of a workgroup still follows its tile index.
    for (int64_t b0 = 0; b0 < p.batch; b0 += kMaxGridY) {
        const int64_t nb = p.batch - b0 < kMaxGridY ? p.batch - b0 : kMaxGridY;
        for (int64_t base = 0; base < tiles; base += kMaxGrid) {
            const int64_t n = tiles - base < kMaxGrid ? tiles - base : kMaxGrid;
            const int extra = base == 0 ? thin_blocks : 0;  // the first launch carries them
            mfma_kernel<Cfg, A_KC, B_KC, VEC>
                <<<dim3(unsigned(n + extra), unsigned(nb)), dim3(Cfg::threads), 0, s>>>(
                    m_tiles, p.N, p.K, p.A, p.lda, p.B, p.ldb, p.C, p.ldc, tiles_m, tiles_n,
                    int(base), dma_ok, p.stride_a, p.stride_b, p.stride_c, b0, p.bias, p.act,
                    p.k_total, extra, rest);
        }
    }
}

template <class Cfg, bool A_KC, bool B_KC>
void dispatch_vec(const Problem &p, hipStream_t s)
{
    // Product b reads A + b * stride_a and B + b * stride_b, so in a batch
    // the strides must keep every product's operands 16-byte aligned too.
    const bool strides_ok = p.batch <= 1 || (p.stride_a % kVec == 0 && p.stride_b % kVec == 0);
    if (strides_ok && vec4_ok(p.A, p.lda) && vec4_ok(p.B, p.ldb))
        dispatch<Cfg, A_KC, B_KC, true>(p, s);
    else
        dispatch<Cfg, A_KC, B_KC, false>(p, s);
}

template <class Cfg, class CfgKK = Cfg>
void dispatch_layout(const Problem &p, hipStream_t s)
{
    // A is k-contiguous when untransposed; B when transposed.
    const bool a_kc = !p.transA, b_kc = p.transB;
    if (a_kc) {
        if (b_kc) dispatch_vec<CfgKK, true, true>(p, s); else dispatch_vec<Cfg, true, false>(p, s);
    } else {
        if (b_kc) dispatch_vec<Cfg, false, true>(p, s); else dispatch_vec<Cfg, false, false>(p, s);
    }
}

// The large tile needs about two workgroups per CU to keep the matrix cores
// busy.  Below 256 large tiles (one per CU), or below 512 when K is short
// enough that each tile's k loop cannot amortise its start-up, the 64 x 64
// tile, with each stage's k groups split over two slices of waves, gives
// more parallelism (measured: S1k 30 -> 88 TFLOP/s, the 2049 x 3071 x 769
// ragged product 81 -> 86; the 1024 x 4096 x 8192 weight gradient, 256
// large tiles, stays faster on the large tile).  It is also used when more
// than a quarter of the large tiles' area would fall outside C (e.g. N = 64).
// The paired variant once there are more small tiles than CUs (then a
// second workgroup per CU has work; measured with K = 1024: 1536 x 1024,
// 384 tiles, 88.2 vs 83.3 TFLOP/s; 2048 x 1024 116.8 vs 109.4; 1600 x 1200
// x 700 97.5 vs 89.0; at 256 tiles, one per CU, the single workgroup with
// 128-k stages stays ahead).
#ifndef GEMM_MFMA_SMALL_PAIR_ABOVE
#define GEMM_MFMA_SMALL_PAIR_ABOVE 256
#endif
#ifndef GEMM_MFMA_SMALL_BELOW
#define GEMM_MFMA_SMALL_BELOW 256
#endif
#ifndef GEMM_MFMA_HUGE_FROM
#define GEMM_MFMA_HUGE_FROM 384
#endif
#ifndef GEMM_MFMA_SHORT_K_SMALL_BELOW
#define GEMM_MFMA_SHORT_K_SMALL_BELOW 512
#endif
constexpr int kShortK = 1024;
// The 256 x 128 tile runs one workgroup per CU; with only a few stages per
// tile its start-up copy and output store are not overlapped by a second
// workgroup, so short products stay on the 128 x 128 tile (the 64-product
// attention-score batch, K = 64: 59.7 vs 55.9 TFLOP/s).
constexpr int kHugeMinK = 512;
// Long products whose large tiles fill whole rounds of one per CU leave no
// tail, and the 256 x 128 tile's lower copy traffic wins below
// GEMM_MFMA_HUGE_FROM too (the 8192 x 1024 x 4096 input-gradient product,
// 256 tiles: 138.7 vs 135.7 TFLOP/s).
constexpr int kHugeLongK = 2048;

}  // namespace

int plan_mfma(const Problem &p, int tile)
{
    if (tile == 0 && mfma_wide_preferred(p)) return GEMM_F32_PLAN_MFMA_256X256;
    bool narrow = false;
    if (tile == 0) {
        const int64_t big_tiles =
            int64_t(ceil_div(p.M, Default::BM)) * ceil_div(p.N, Default::BN) * p.batch;
        const int64_t area = int64_t(p.M) * p.N * p.batch;
        const bool wasteful = 4 * area < 3 * big_tiles * Default::BM * Default::BN;
        const bool small = big_tiles < GEMM_MFMA_SMALL_BELOW || wasteful ||
                           (p.K <= kShortK && big_tiles < GEMM_MFMA_SHORT_K_SMALL_BELOW);
        const int64_t huge_tiles =
            int64_t(ceil_div(p.M, Huge::BM)) * ceil_div(p.N, Huge::BN) * p.batch;
        const bool huge_fits = 4 * area >= 3 * huge_tiles * Huge::BM * Huge::BN;
        const bool whole_rounds = p.K >= kHugeLongK && huge_tiles % kCUs == 0;
        const bool huge = (huge_tiles >= GEMM_MFMA_HUGE_FROM || whole_rounds) && huge_fits && p.K >= kHugeMinK;
        tile = small ? Small::BM : huge ? Huge::BM : Default::BM;
        const int64_t narrow_tiles = int64_t(ceil_div(p.M, Narrow::BM)) * p.batch;
        narrow = small && p.N <= Narrow::BN && narrow_tiles >= kCUs;
    }
    if (narrow) return GEMM_F32_PLAN_MFMA_128X64;
    if (tile == Small::BM) {
        const int64_t small_tiles = int64_t(ceil_div(p.M, Small::BM)) * ceil_div(p.N, Small::BN) * p.batch;
        return small_tiles > GEMM_MFMA_SMALL_PAIR_ABOVE ? GEMM_F32_PLAN_MFMA_64X64_PAIR : GEMM_F32_PLAN_MFMA_64X64;
    }
    if (tile == Huge::BM) return GEMM_F32_PLAN_MFMA_256X128;
    // A is k-contiguous when untransposed; B when transposed.
    if (!p.transA && p.transB) return GEMM_F32_PLAN_MFMA_128X128_KK;
    const int64_t tiles = int64_t(ceil_div(p.M, Default::BM)) * ceil_div(p.N, Default::BN) * p.batch;
    return tiles <= kCUs ? GEMM_F32_PLAN_MFMA_128X128_ONE_ROUND : GEMM_F32_PLAN_MFMA_128X128;
}

hipError_t launch_mfma(const Problem &p, hipStream_t s, int tile)
{
    switch (plan_mfma(p, tile)) {
    case GEMM_F32_PLAN_MFMA_256X256: return launch_mfma_wide(p, s);
    case GEMM_F32_PLAN_MFMA_128X64: dispatch_layout<Narrow>(p, s); break;
    case GEMM_F32_PLAN_MFMA_64X64_PAIR: dispatch_layout<SmallPair>(p, s); break;
    case GEMM_F32_PLAN_MFMA_64X64: dispatch_layout<Small>(p, s); break;
    case GEMM_F32_PLAN_MFMA_256X128: dispatch_layout<Huge>(p, s); break;
    case GEMM_F32_PLAN_MFMA_128X128_ONE_ROUND: dispatch_layout<OneRound, DefaultKK>(p, s); break;
    default: dispatch_layout<Default, DefaultKK>(p, s); break;
    }
    return hipGetLastError();
}

}  // namespace gemmf32
