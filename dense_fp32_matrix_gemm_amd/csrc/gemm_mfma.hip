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
//    waves per SIMD to hide LDS and barrier latency.
//  * Staging, interior tiles: each K stage (BK = 32) is copied from global
//    memory straight into LDS with global_load_lds_dwordx4 (each wave
//    instruction moves 64 x 16 bytes; no registers, no LDS write
//    instructions), issued one stage ahead into the other of two LDS
//    buffers, so one barrier per stage suffices (the double buffering of the
//    cuda-oxide book's summary; the page's second barrier is not needed
//    because the buffer being filled is never the one being read).
//  * Staging, edge tiles and the last partial stage: 16-byte (or scalar)
//    loads into registers with every element predicated, zero outside the
//    matrix (section 3.3's kernel assumes tile multiples), written to LDS
//    in the same layout.  Stores to C are predicated.  Barriers are outside
//    every data-dependent branch.
//  * LDS layout: unpadded, with an XOR swizzle of the 16-byte vectors in
//    each row (the alternative to padding named in section 3.6): a DMA
//    instruction writes 1 KB contiguously, so padding is not possible, and
//    the swizzle keeps the fragment reads free of bank conflicts.
//  * Fragment order in k: inside each group of 8 k values, lanes 0-31 feed
//    the MFMA k = 0 slot with k = u and lanes 32-63 the k = 1 slot with
//    k = 4 + u for the four MFMAs u = 0..3.  Both operands use the same map,
//    so every pair (a_ik, b_kj) meets exactly once, and a k-contiguous
//    operand is read with one 16-byte LDS read per lane per 4 MFMAs.
//  * Accumulation: each stage's 32 k values are summed into a fresh MFMA
//    accumulator (the first MFMA of the stage takes a zero addend) and then
//    added into the running tile.  The matrix core adds one product at a
//    time in FP32, so without this the relative error of a K = 8192 product
//    grows past 1e-6; with it the error stays near 3e-7.
//  * Launch order: workgroups are dealt round-robin to the 8 XCDs, each with
//    its own L2.  The tile index is remapped so that each XCD receives a
//    contiguous run of tiles, and that run is walked GROUP_M tile-rows at a
//    time, so co-resident workgroups of one XCD share A and B panels in L2.
#include "tile_common.hpp"

namespace gemmf32 {
namespace {

template <bool V>
struct integral_constant {
    static constexpr bool value = V;
};
using Yes = integral_constant<true>;
using No = integral_constant<false>;

typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;
constexpr int kBlk = 32;  // MFMA output block edge

// A tile configuration: BM x BN of C per workgroup, BK k per stage (and per
// accumulation chunk), WAVES_M x WAVES_N waves each owning a
// (BM/WAVES_M) x (BN/WAVES_N) register tile of 32 x 32 MFMA blocks, WPE
// waves per SIMD requested from the register allocator, GROUP_M tile-rows
// per group in the launch order, and WRITE_G, the k group of a stage after
// whose fragment reads register-staged data for the next stage is written
// to LDS (BK / 8 means after the last group).
template <int BM_, int BN_, int BK_, int WAVES_M, int WAVES_N, int WPE_, int GROUP_M_,
          int WRITE_G_>
struct Config {
    static constexpr int BM = BM_, BN = BN_, BK = BK_;
    static constexpr int waves = WAVES_M * WAVES_N;
    static constexpr int threads = kWave * waves;
    static constexpr int waves_n = WAVES_N;
    static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    static constexpr int FM = WM / kBlk, FN = WN / kBlk;
    static constexpr int wpe = WPE_;
    static constexpr int group_m = GROUP_M_;
    static constexpr int write_g = WRITE_G_;
    static_assert(WM % kBlk == 0 && WN % kBlk == 0, "wave tiles are whole MFMA blocks");
    static_assert(BK % 8 == 0, "stages are whole 8-k fragment groups");
};

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
    static constexpr int dma_per_wave = chunks / Cfg::waves;
    static_assert(chunks % Cfg::waves == 0, "DMA instructions split evenly over the waves");
    static_assert((vpr & (vpr - 1)) == 0, "rows hold a power-of-two number of vectors");
    using Load = Slice<rows, cols, Cfg::threads>;
    static constexpr int per_thread = Load::per_thread;

    // KC: a fragment read takes 16 bytes from each of 32 consecutive rows.
    //   (r & 7) ^ ((r >> 3) & 1) makes any 8 consecutive rows hit 8 different
    //   16-byte bank groups, and any 16 consecutive rows with equal parity of
    //   r hit 8 different ones, so it is conflict-free whether the LDS serves
    //   8 or 16 lanes of a 16-byte read per cycle.
    // MC: a fragment read takes 4 bytes from 32 consecutive floats of row k
    //   (lanes 0-31) and of row k + 4 (lanes 32-63); flipping bit 3 of the
    //   vector index every 4 rows puts the two halves in opposite 128-byte
    //   halves of a 256-byte bank line.
    __device__ static __forceinline__ int swz(int r)
    {
        return KC ? (((r & 7) ^ ((r >> 3) & 1)) & (vpr - 1)) : ((((r >> 2) & 1) << 3) & (vpr - 1));
    }
    __device__ static __forceinline__ int slot(int r, int v) { return r * vpr + (v ^ swz(r)); }

    // Registers -> LDS for the register-staged path (same slice-to-thread
    // map as the load).
    __device__ static __forceinline__ void store(float *lds, const v4f (&reg)[per_thread])
    {
#pragma unroll
        for (int q = 0; q < per_thread; ++q)
            *reinterpret_cast<v4f *>(lds + 4 * slot(Load::row(q), Load::col(q) / 4)) = reg[q];
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
                                               const uint32_t (&off)[dma_per_wave], int wave)
    {
#pragma unroll
        for (int q = 0; q < dma_per_wave; ++q)
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const float *>(origin + off[q]),
                                             lds + (wave * dma_per_wave + q) * 256, 16, 0, 0);
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

// Wait until this wave's global->LDS copies have landed.
__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0F70); /* vmcnt(0) */ }

template <class Cfg, bool A_KC, bool B_KC, bool VEC>
__global__ __attribute__((amdgpu_flat_work_group_size(Cfg::threads, Cfg::threads),
                          amdgpu_waves_per_eu(Cfg::wpe, Cfg::wpe))) void
mfma_kernel(int M, int N, int K, const float *__restrict__ A, int64_t lda,
            const float *__restrict__ B, int64_t ldb, float *__restrict__ C, int64_t ldc,
            int tiles_m, int tiles_n, int tile_base, int dma_ok)
{
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK;
    constexpr int FM = Cfg::FM, FN = Cfg::FN;
    using TA = Tile<Cfg, BM, A_KC>;
    using TB = Tile<Cfg, BN, B_KC>;
    // Two stage buffers as separate objects, so the compiler can tell a
    // copy into one from reads of the other.
    __shared__ __attribute__((aligned(1024))) float buf0[TA::floats + TB::floats];
    __shared__ __attribute__((aligned(1024))) float buf1[TA::floats + TB::floats];

    int tm, tn;
    tile_of<Cfg::group_m>(tile_base + int(blockIdx.x), tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const bool inside = (m0 + BM <= M) && (n0 + BN <= N);
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int wm = (wave / Cfg::waves_n) * Cfg::WM, wn = (wave % Cfg::waves_n) * Cfg::WN;
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
    auto compute = [&](const float *lds, auto mid) {
        const float *la = lds;
        const float *lb = lds + TA::floats;
        v16f part[FM][FN];
#pragma unroll
        for (int g = 0; g < BK / 8; ++g) {
            v4f fa[FM], fb[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) fa[i] = TA::fragment(la, wm + i * kBlk + l32, g, half);
#pragma unroll
            for (int j = 0; j < FN; ++j) fb[j] = TB::fragment(lb, wn + j * kBlk + l32, g, half);
            if (g == Cfg::write_g) mid();
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        part[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                            fa[i][u], fb[j][u], (g == 0 && u == 0) ? v16f{0.0f} : part[i][j], 0, 0,
                            0);
        }
        if (Cfg::write_g >= BK / 8) mid();
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] += part[i][j];
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
                v4f ra[TA::per_thread], rb[TB::per_thread];
                const int k = (s + 1) * BK;
                TA::Load::template load<true, VEC>(opa, a_r(k), a_c(k), ra);
                TB::Load::template load<true, VEC>(opb, b_r(k), b_c(k), rb);
                compute(cur, [&] {
                    TA::store(nxt, ra);
                    TB::store(nxt + TA::floats, rb);
                });
            } else {
                compute(cur, nothing);
            }
            __syncthreads();
        }
    };

    if (VEC && dma_ok && inside && full >= 1) {
        // Interior tile: full stages copied straight into LDS, one ahead.
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
        auto dma = [&](float *lds, int stage) {
            TA::dma(lds, ga + stage * a_step, oa, wave);
            TB::dma(lds + TA::floats, gb + stage * b_step, ob, wave);
        };
        dma(buf0, 0);
        wait_dma();
        __syncthreads();
        int s = 0;
        // Two stages per trip so each buffer is a compile-time choice.
        for (; s + 2 < full; s += 2) {
            dma(buf1, s + 1);
            compute(buf0, nothing);
            wait_dma();
            __syncthreads();
            dma(buf0, s + 2);
            compute(buf1, nothing);
            wait_dma();
            __syncthreads();
        }
        if (s + 1 < full) {
            dma(buf1, s + 1);
            compute(buf0, nothing);
            wait_dma();
            __syncthreads();
            ++s;
        }
        // Stage s, the last full one, is in buffer s & 1; a partial stage
        // after it, if any, goes through the predicated path.
        staged(s);
    } else {
        v4f ra[TA::per_thread], rb[TB::per_thread];
        TA::Load::template load<true, VEC>(opa, a_r(0), a_c(0), ra);
        TB::Load::template load<true, VEC>(opb, b_r(0), b_c(0), rb);
        TA::store(buf0, ra);
        TB::store(buf0 + TA::floats, rb);
        __syncthreads();
        staged(0);
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

#ifndef GEMM_MFMA_CONFIG
#define GEMM_MFMA_CONFIG 128, 128, 32, 4, 2, 4, 8, 3
#endif
using Default = Config<GEMM_MFMA_CONFIG>;

// True if every DMA offset of an operand's stage fits in 32 bits.
inline bool dma_offsets_fit(int rows, int64_t ld) { return (int64_t(rows) * ld + ld) * 4 < (int64_t(1) << 32); }

template <class Cfg, bool A_KC, bool B_KC, bool VEC>
void dispatch(const Problem &p, hipStream_t s)
{
    using TA = Tile<Cfg, Cfg::BM, A_KC>;
    using TB = Tile<Cfg, Cfg::BN, B_KC>;
    const int tiles_m = ceil_div(p.M, Cfg::BM), tiles_n = ceil_div(p.N, Cfg::BN);
    const int64_t tiles = int64_t(tiles_m) * tiles_n;
    const int dma_ok = dma_offsets_fit(TA::rows, p.lda) && dma_offsets_fit(TB::rows, p.ldb);
    // One workgroup per tile; a grid larger than the cap is split into
    // launches whose first tile index is a multiple of 8, so the XCD of a
    // workgroup still follows its tile index.
    for (int64_t base = 0; base < tiles; base += kMaxGrid) {
        const int64_t n = tiles - base < kMaxGrid ? tiles - base : kMaxGrid;
        mfma_kernel<Cfg, A_KC, B_KC, VEC><<<dim3(unsigned(n)), dim3(Cfg::threads), 0, s>>>(
            p.M, p.N, p.K, p.A, p.lda, p.B, p.ldb, p.C, p.ldc, tiles_m, tiles_n, int(base),
            dma_ok);
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
    // A is k-contiguous when untransposed; B when transposed.
    const bool a_kc = !p.transA, b_kc = p.transB;
    if (a_kc) {
        if (b_kc) dispatch_vec<Cfg, true, true>(p, s); else dispatch_vec<Cfg, true, false>(p, s);
    } else {
        if (b_kc) dispatch_vec<Cfg, false, true>(p, s); else dispatch_vec<Cfg, false, false>(p, s);
    }
}

}  // namespace

hipError_t launch_mfma(const Problem &p, hipStream_t s)
{
    dispatch_layout<Default>(p, s);
    return hipGetLastError();
}

}  // namespace gemmf32
